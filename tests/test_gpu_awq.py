"""GPU parity of every fused-delta W4A16 path with AWQ-style zero-points.

The configs' asymmetric recipe, z = -8 s + N(0, 1e-3), makes delta = z + 8 s
tiny next to the scale term, so a wrong delta term would hardly show.  Here
z = -zp * s with an integer zp ~ U{0..15} per group and column, so delta =
(8 - zp) s is as large as the scale term itself ("Marlin INT4 on Ada - how it
works", "The core mismatch: symmetric vs asymmetric": C = A.W_sym +
A_group_sum @ delta).  Each kernel that applies delta is reached by a shape
the dispatcher sends to it, and checked against the oracle (which uses z
itself, W = q s + z) to the W4A16 bar: relative Frobenius error <= 2e-3 and
the elementwise guard."""
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


def _case(M, K, N, g, case_id):
    gg = K if g == -1 else g
    c = synth.w4a16_case(M, K, N, gg, asym=True, stream=94, case_id=case_id,
                         zero_points="awq", name="awq")
    _, dh = oracle.delta(c.s, c.z)
    d = np.abs(dh.view(np.float16).astype(np.float64))
    assert d.max() >= 4 * np.abs(c.s.astype(np.float64)).mean()   # delta is not small here
    return c


def _rows(M, every=16):
    """One row of every `every`-row band (at a varying offset), or all rows."""
    if M <= 64:
        return np.arange(M)
    i = np.arange((M + every - 1) // every)
    return np.minimum(every * i + i % every, M - 1)


def _check(c, flags=0, rows=None):
    note(f"awq M={c.M} K={c.K} N={c.N} g={c.g} flags={flags}")
    pw = qg.pack(dev(c.q), dev(c.s), dev(c.z), c.g, fold=True)
    C = qg.w4a16(dev(c.A), pw, flags=flags)
    torch.cuda.synchronize()
    got = host(C).astype(np.float64)
    assert np.all(np.isfinite(got))
    rows = np.arange(c.M) if rows is None else rows
    ref = oracle.w4a16(c.A[rows], c.q, c.s, c.z, c.g)
    err = rel_fro(got[rows], ref)
    assert err <= TOL, err
    assert elementwise_guard(got[rows], ref) <= 0
    return err


# decode kernel: 2 splits (K5120 x N17408), 6 splits (K17408 x N5120), 8
# splits (K16384 x N4096, every group form), unsplit (wide N)
@pytest.mark.parametrize("M,K,N,g", [
    (16, 5120, 17408, 128), (1, 5120, 17408, 128),
    (16, 17408, 5120, 128), (4, 17408, 5120, 128),
    (16, 16384, 4096, 128), (9, 16384, 4096, 256), (16, 16384, 4096, -1),
    (5, 1024, 32768, 128),
])
def test_awq_decode(M, K, N, g):
    _check(_case(M, K, N, g, case_id=M * 3 + K + N + (g if g > 0 else 7)))


# skinny kernel: M <= 16 where the decode kernel loses, and 17 <= M <= 80
@pytest.mark.parametrize("M,K,N,g", [(16, 4096, 4096, 128), (37, 2048, 1024, 128),
                                     (80, 1024, 2048, 256)])
def test_awq_skinny(M, K, N, g):
    _check(_case(M, K, N, g, case_id=100 + M))


# mid kernel (64 x 64 tiles): scaled every k-tile (g = 128, 512), every
# second one (g = 256), once (per-column)
@pytest.mark.parametrize("g", [128, 256, 512, -1])
def test_awq_mid(g):
    _check(_case(256, 4096, 8192, g, case_id=200 + (g if g > 0 else 1)), rows=_rows(256, 8))


# tiled 64 x 128 (fused delta as an extra MFMA k-step per window of 16
# groups): 18 groups (a full window and a partial one), two-k-tile groups,
# per-column
@pytest.mark.parametrize("K,g", [(2304, 128), (2048, 256), (1024, -1)])
def test_awq_tiled_64x128(K, g):
    c = _case(512, K, 8192, g, case_id=300 + K)
    assert qg.qg_workspace_bytes(qg.QG_OP_W4A16, 512, 8192, K, g) == 0
    _check(c, rows=_rows(512))


# tiled 128 x 256 with the fused delta (one launch), and the same shape with
# the two-kernel correction
@pytest.mark.parametrize("flags", [0, 1])
def test_awq_tiled_128x256(flags):
    c = _case(2048, 2304, 16384, 128, case_id=400)
    _check(c, flags=qg.QG_CORR_SEPARATE if flags else 0, rows=_rows(2048))


def test_awq_separate_correction_decode():
    _check(_case(16, 5120, 17408, 128, case_id=500), flags=qg.QG_CORR_SEPARATE)


@pytest.mark.parametrize("M,K,N,g", [(16, 1000, 300, 128), (7, 1000, 300, -1),
                                     (300, 1000, 520, 256)])
def test_awq_tails(M, K, N, g):
    _check(_case(M, K, N, g, case_id=600 + M))


# the gate/up pair: the gated decode kernel (one launch, split-K) and the
# GEMM-then-elementwise path of larger batches
@pytest.mark.parametrize("M,K,N", [(16, 5120, 17408), (4, 17408, 5120), (64, 2048, 1024)])
def test_awq_swiglu(M, K, N):
    c = _case(M, K, 2 * N, 128, case_id=700 + M)
    note(f"awq swiglu M={M} K={K} N={N}")
    pair = qg.pack(dev(c.q), dev(c.s), dev(c.z), 128, fold=True)
    H = qg.w4a16_swiglu(dev(c.A), pair)
    torch.cuda.synchronize()
    got = host(H).astype(np.float64)
    ref = oracle.w4a16_swiglu(c.A, c.q, c.s, c.z, 128)
    assert rel_fro(got, ref) <= TOL
    assert elementwise_guard(got, ref) <= 0
