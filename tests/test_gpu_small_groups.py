"""GPU parity with weight groups of 64 and 32 along K.

Every 32-k MFMA step of a packed 128-k tile lies inside one such group (the
packed layout gives k-steps 0, 1 to the low nibbles and 2, 3 to the high
ones), so the decode and skinny kernels scale each step's products with its
own group's scale and delta, the 8-wave mid kernel takes its low- and
high-nibble sums as the two groups of 64, and the generic tiled kernels
dequantize each step with its group's scale; the grouped W4A8 kernel takes groups of 64 (one 64-k int8
MFMA step each) and of 32 (one 16x16x32 int8 MFMA on each 8-byte half of a
step's operands).  Checked against the oracle, which applies W = q s + z per
group of g consecutive k ("Marlin INT4 on Ada - how it works", "The core
mismatch: symmetric vs asymmetric"), to the W4A16 bar (relative Frobenius
<= 2e-3 and the elementwise guard) with AWQ-style zero-points (delta as large
as the scale term) and with random-sign symmetric scales; W4A8's integer
group products bit-exact."""
import numpy as np
import pytest
import torch

import int4_weight_only_uint32_amd as qg
import oracle
import synth
from tests.gpu_util import dev, elementwise_guard, host, note, rel_fro

pytestmark = pytest.mark.gpu

TOL = 2e-3


@pytest.fixture(scope="module", autouse=True)
def _device():
    assert torch.cuda.is_available()
    assert qg.qg_device_supported(0), "GPU visible but not gfx950"
    oracle.build(force=False)


def _rows(M, every=16):
    if M <= 64:
        return np.arange(M)
    i = np.arange((M + every - 1) // every)
    return np.minimum(every * i + i % every, M - 1)


def _w4a16(M, K, N, g, asym, flags=0, case_id=0):
    c = synth.w4a16_case(M, K, N, g, asym=asym, signed_scales=not asym, stream=98,
                         case_id=case_id, zero_points="awq" if asym else "noise")
    note(f"small groups w4a16 M={M} K={K} N={N} g={g} asym={asym} flags={flags}")
    pw = qg.pack(dev(c.q), dev(c.s), dev(c.z) if asym else None, g, fold=True)
    C = qg.w4a16(dev(c.A), pw, flags=flags)
    torch.cuda.synchronize()
    got = host(C).astype(np.float64)
    assert np.all(np.isfinite(got))
    rows = _rows(M)
    ref = oracle.w4a16(c.A[rows], c.q, c.s, c.z if asym else None, g, fold=True)
    err = rel_fro(got[rows], ref)
    assert err <= TOL, err
    assert elementwise_guard(got[rows], ref) <= 0
    return err


# decode kernel (M <= 16, with and without K splits), the skinny kernel
# (narrow decode shapes, 17 <= M <= 80, every configuration), the generic
# 64x128 tiles (mid-size batches), the 8-wave mid kernel (g = 64 on mid-size
# batches over wide N; g = 32 takes the 64x128 tiles there), the generic
# 128x256 tiles and the prefill-size row split
@pytest.mark.parametrize("g", [64, 32])
@pytest.mark.parametrize("M,K,N", [(1, 4096, 4096), (16, 5120, 8192), (16, 17408, 5120),
                                   (8, 1024, 1024), (33, 2048, 1024), (64, 4096, 2048),
                                   (80, 1024, 4096), (256, 2048, 4096), (256, 2048, 8192),
                                   (200, 1536, 8192), (2048, 1024, 8192), (4096, 1024, 17408)])
def test_w4a16_small_groups_asym(M, K, N, g):
    _w4a16(M, K, N, g, True, case_id=M + g)


@pytest.mark.parametrize("g", [64, 32])
@pytest.mark.parametrize("M,K,N", [(4, 4096, 4096), (100, 1024, 2048), (256, 1024, 8192),
                                   (2048, 1024, 8192)])
def test_w4a16_small_groups_symmetric_signed(M, K, N, g):
    _w4a16(M, K, N, g, False, case_id=1000 + M + g)


@pytest.mark.parametrize("g", [64, 32])
def test_w4a16_small_groups_separate_correction(g):
    _w4a16(16, 4096, 4096, g, True, flags=qg.QG_CORR_SEPARATE, case_id=2000 + g)


@pytest.mark.parametrize("g,M,K", [(64, 16, 1000), (32, 300, 1000), (64, 16, 1025), (32, 100, 1025)])
def test_w4a16_small_groups_k_and_n_tails(g, M, K):
    """K = 1000 (padded to 1024) or 1025 (padded to 1152, which adds whole
    groups past the input's ceil(K/g): the pack gives them zero scale and
    delta) and N = 1000 (padded to 1024, cropped)."""
    _w4a16(M, K, 1000, g, True, case_id=3000 + g + K)


def test_w4a16_groups_of_64_mid_kernel_tails():
    """K = 1000 and N = 8100 (padded to 1024 and 8192) at M = 256: the 8-wave
    mid kernel over the padded shape, whose last group of 64 is partly and
    the padded columns wholly outside the logical weight."""
    _w4a16(256, 1000, 8100, 64, True, case_id=3500)


@pytest.mark.parametrize("g", [64, 32])
@pytest.mark.parametrize("M,K,N", [(16, 4096, 4096), (40, 2048, 1024), (512, 1024, 2048)])
def test_swiglu_small_groups(M, K, N, g):
    c = synth.w4a16_case(M, K, 2 * N, g, asym=True, stream=98, case_id=4000 + M + g,
                         zero_points="awq")
    note(f"small groups swiglu M={M} K={K} N={N} g={g}")
    pw = qg.pack(dev(c.q), dev(c.s), dev(c.z), g, fold=True)
    H = qg.w4a16_swiglu(dev(c.A), pw)
    torch.cuda.synchronize()
    got = host(H).astype(np.float64)
    rows = _rows(M)
    ref = oracle.w4a16_swiglu(c.A[rows], c.q, c.s, c.z, g, fold=True)
    assert rel_fro(got[rows], ref) <= TOL
    assert elementwise_guard(got[rows], ref) <= 0


@pytest.mark.parametrize("g", [64, 32])
@pytest.mark.parametrize("asym", [False, True])
def test_w4a8_small_groups(asym, g):
    """4 experts with ragged rows (one empty), K 2048, N 1024: the integer
    group products (acc_debug) bit-exact against the oracle's, C to 1e-2."""
    c = synth.w4a8_case(4, 0, 2048, 1024, g, signed_scales=not asym, stream=98,
                        case_id=5000 + asym + g, rows=[70, 0, 33, 64], asym=asym)
    note(f"small groups w4a8 g={g} asym={asym}")
    packs = [qg.pack(dev(c.q[e]), dev(c.s[e]), dev(c.z[e]) if asym else None, g)
             for e in range(c.E)]
    W = torch.stack([p.w for p in packs]).contiguous()
    S = torch.stack([p.scale for p in packs]).contiguous()
    D = torch.stack([p.delta for p in packs]).contiguous() if asym else None
    mr = int(np.max(np.diff(c.offsets)))
    acc = torch.zeros((c.M_total, c.K // g, c.N), dtype=torch.int32, device="cuda")
    C = qg.w4a8(dev(c.Aq), dev(c.a_scale), W, S, dev(c.offsets), c.E, mr, c.N, g,
                acc_debug=acc, w_delta=D)
    C2 = qg.w4a8(dev(c.Aq), dev(c.a_scale), W, S, dev(c.offsets), c.E, mr, c.N, g, w_delta=D)
    torch.cuda.synchronize()
    ref, ref_acc = oracle.w4a8(c.Aq, c.a_scale, c.q, c.s, c.offsets, g, fold=True, z=c.z)
    assert np.array_equal(host(acc).astype(np.int64), ref_acc)
    for out in (C, C2):
        got = host(out).astype(np.float64)
        assert np.all(np.isfinite(got))
        assert rel_fro(got, ref) <= 1e-2
    assert torch.equal(C, C2)
