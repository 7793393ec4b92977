"""GPU parity over a seeded sweep of shapes that crosses every dispatch
boundary: M around the decode / skinny / mid / tiled limits (16, 32, 48, 64,
80, 128, 256), K and N with and without tails, group sizes 32, 64, 128, 256
and one group over K, symmetric and AWQ-style asymmetric weights, plain and
gated (SwiGLU).  Each case is checked against the oracle ("Marlin INT4 on Ada
- how it works", "The core mismatch: symmetric vs asymmetric") on a sample of
rows spread over the m-tiles, to the W4A16 bar (relative Frobenius <= 2e-3
and the elementwise guard)."""
import numpy as np
import pytest
import torch

import int4_weight_only_uint32_amd as qg
import oracle
import synth
from tests.gpu_util import dev, elementwise_guard, host, note, rel_fro

pytestmark = pytest.mark.gpu

TOL = 2e-3
MS = [1, 3, 15, 16, 17, 31, 32, 33, 47, 48, 63, 64, 65, 79, 80, 81, 96, 127, 128, 129, 200, 256, 257]
KS = [128, 384, 1000, 1024, 1152, 2048, 3072, 4096]
NS = [64, 192, 1000, 1024, 2048, 4100, 8192, 8704]
GS = [32, 64, 128, 256, -1]


def _cases(n=120, seed=20261202):
    """Seeded shapes: (M, K, N, g, asym, gated); the group size must fit K
    (g <= K), the gated pair has no K or N tail, and weights stay under ~2^26
    elements so the oracle's sampled rows take well under a second each."""
    r = np.random.RandomState(seed)
    out = []
    while len(out) < n:
        M, K, N = int(r.choice(MS)), int(r.choice(KS)), int(r.choice(NS))
        g = int(r.choice(GS))
        gated = bool(r.rand() < 0.2)
        if gated and N % 128:
            N = (N // 128 + 1) * 128      # the pair's output width: multiple of 128
        g = K if g == -1 else g
        if g > K or (g >= 128 and g % 128 and g != K) or K * N * (2 if gated else 1) > (1 << 26):
            continue
        if gated and K % 128:
            continue                      # the gated pair takes no K tail
        out.append((M, K, N, g, bool(r.rand() < 0.6), gated))
    return out


def _rows(M, k=12):
    if M <= k:
        return np.arange(M)
    return np.unique(np.concatenate([[0, M - 1], np.linspace(0, M - 1, k).astype(int)]))


@pytest.mark.parametrize("M,K,N,g,asym,gated", _cases())
def test_shape_sweep(M, K, N, g, asym, gated):
    Nw = 2 * N if gated else N
    c = synth.w4a16_case(M, K, Nw, g, asym=asym, signed_scales=not asym, stream=88,
                         case_id=M * 131 + K * 7 + N + g, zero_points="awq" if asym else "noise")
    note(f"sweep M={M} K={K} N={N} g={g} asym={asym} gated={gated}")
    pw = qg.pack(dev(c.q), dev(c.s), dev(c.z) if asym else None, g, fold=True)
    A = dev(c.A)
    out = qg.w4a16_swiglu(A, pw) if gated else qg.w4a16(A, pw)
    torch.cuda.synchronize()
    got = host(out).astype(np.float64)
    assert got.shape == (M, N)
    assert np.all(np.isfinite(got))
    rows = _rows(M)
    z = c.z if asym else None
    ref = (oracle.w4a16_swiglu(c.A[rows], c.q, c.s, z, g, fold=True) if gated
           else oracle.w4a16(c.A[rows], c.q, c.s, z, g, fold=True))
    assert rel_fro(got[rows], ref) <= TOL
    assert elementwise_guard(got[rows], ref) <= 0
