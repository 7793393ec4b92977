"""Independent host-side reader of the packed weight layout, written from its
specification (not from the library's code), used to check the packer
bit-exactly:

  The K x N codes are cut into tiles of 128 k x 16 n; tile (nt, kt) is the
  256 uint32 starting at (nt * K/128 + kt) * 256.  Within a tile, lane
  l = 0..63 owns uint32 4l .. 4l+3; its column is l mod 16 and its k-quarter
  kq = l div 16.  In uint32 j, the nibble at bits 4p..4p+3 holds the code of
      k = 32*step + 8*kq + slot,  slot = 4*(j mod 2) + 2*b1(p) + b2(p),
      step = (j div 2) + 2*b0(p)
  where b0, b1, b2 are bits 0, 1, 2 of p.
"""
import numpy as np


def _k_map():
    # kmap[kq, j, p] -> k within the tile
    kmap = np.zeros((4, 4, 8), dtype=np.int64)
    for kq in range(4):
        for j in range(4):
            for p in range(8):
                b0, b1, b2 = p & 1, (p >> 1) & 1, (p >> 2) & 1
                slot = 4 * (j % 2) + 2 * b1 + b2
                step = (j // 2) + 2 * b0
                kmap[kq, j, p] = 32 * step + 8 * kq + slot
    return kmap


def unpack_codes(w: np.ndarray, K: int, N: int) -> np.ndarray:
    """uint32 (or int32) array of K*N/8 words -> uint8 codes [K, N]."""
    w = np.ascontiguousarray(w).view(np.uint32).reshape(N // 16, K // 128, 64, 4)
    kmap = _k_map()
    q = np.zeros((K, N), dtype=np.uint8)
    lanes = np.arange(64)
    cols = lanes % 16
    kqs = lanes // 16
    for j in range(4):
        for p in range(8):
            nib = ((w[:, :, :, j] >> np.uint32(4 * p)) & np.uint32(15)).astype(np.uint8)  # [nt, kt, lane]
            kl = kmap[kqs, j, p]                                                           # [lane]
            kk = (np.arange(K // 128)[None, :, None] * 128 + kl[None, None, :])
            nn = (np.arange(N // 16)[:, None, None] * 16 + cols[None, None, :])
            q[np.broadcast_to(kk, nib.shape), np.broadcast_to(nn, nib.shape)] = nib
    return q


def layout_is_permutation() -> bool:
    kmap = _k_map()
    seen = set()
    for kq in range(4):
        for j in range(4):
            for p in range(8):
                seen.add((kq, int(kmap[kq, j, p])))
    # each lane-quarter kq covers 32 distinct k; together all 128
    ks = sorted(int(kmap[kq, j, p]) for kq in range(4) for j in range(4) for p in range(8))
    return ks == list(range(128)) and len(seen) == 128
