"""GPU parity of the decode kernel with several 16-row m-tiles (17 <= M <= 80).

Batches of 17 to 80 rows run the decode kernel with MT = ceil(M/16) m-tiles
when it beats the skinny kernel (two m-tiles always, three to five on weights
of more than 2^24 elements): every wave dequantizes each code tile to fp16
weights (v - 8) s + delta (one rounding) and multiplies it into all MT m-tiles
of the shared activation tile, and the split-K partial sums hold 16 MT rows.  Checked against the oracle ("Marlin INT4 on Ada - how it works", "The
core mismatch: symmetric vs asymmetric") to the W4A16 bar (relative Frobenius
<= 2e-3 and the elementwise guard), with AWQ-style zero-points, random-sign
symmetric scales, groups of 32, 64, 128 and 256 and one group over K, rows past M in
the last m-tile, K and N tails, and the gated SwiGLU pair."""
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


def _w4a16(M, K, N, g, asym, case_id):
    c = synth.w4a16_case(M, K, N, g, asym=asym, signed_scales=not asym, stream=99,
                         case_id=case_id, zero_points="awq" if asym else "noise")
    note(f"multi-tile decode M={M} K={K} N={N} g={g} asym={asym}")
    # the decode kernel's split-K is what takes a workspace at these shapes
    assert qg.qg_workspace_bytes(qg.QG_OP_W4A16, M, N, K, g, 1, 0) > 0
    pw = qg.pack(dev(c.q), dev(c.s), dev(c.z) if asym else None, g, fold=True)
    C = qg.w4a16(dev(c.A), pw)
    torch.cuda.synchronize()
    got = host(C).astype(np.float64)
    assert np.all(np.isfinite(got))
    ref = oracle.w4a16(c.A, c.q, c.s, c.z if asym else None, g, fold=True)
    assert rel_fro(got, ref) <= TOL
    assert elementwise_guard(got, ref) <= 0


@pytest.mark.parametrize("M", [17, 32, 33, 48, 64, 80])
def test_decode_multi_tile_asym(M):
    _w4a16(M, 2048, 8704, 128, True, case_id=M)


@pytest.mark.parametrize("M,g", [(48, 256), (40, 2048), (24, 256), (40, 64), (80, 64), (33, 32),
                                 (64, 32)])
def test_decode_multi_tile_group_sizes(M, g):
    _w4a16(M, 2048, 8704, g, True, case_id=100 + M + g)


@pytest.mark.parametrize("M", [20, 80])
def test_decode_multi_tile_symmetric_signed(M):
    _w4a16(M, 2048, 8704, 128, False, case_id=200 + M)


def test_decode_multi_tile_long_k():
    """K = 17408, N = 5120: six K splits of 22-23 k-tiles, four m-tiles."""
    _w4a16(64, 17408, 5120, 128, True, case_id=300)


def test_decode_multi_tile_tails():
    """K = 1000 and N = 17000 (padded to 1024 and 17024) at M = 50."""
    _w4a16(50, 1000, 17000, 128, True, case_id=400)


@pytest.mark.parametrize("M,g", [(24, 128), (40, 128), (80, 128), (48, 64)])
def test_swiglu_decode_multi_tile(M, g):
    """The gated decode kernel over MT m-tiles: gate and up waves of the same
    columns, silu(gate) * up formed after the LDS hand-over of every m-tile."""
    K, N = 2048, 4352
    c = synth.w4a16_case(M, K, 2 * N, g, asym=True, stream=99, case_id=500 + M + g,
                         zero_points="awq")
    note(f"multi-tile gated decode M={M} K={K} N={N} g={g}")
    assert qg.qg_workspace_bytes(qg.QG_OP_W4A16_SWIGLU, M, N, K, g, 1, 0) > 0
    pw = qg.pack(dev(c.q), dev(c.s), dev(c.z), g, fold=True)
    H = qg.w4a16_swiglu(dev(c.A), pw)
    torch.cuda.synchronize()
    got = host(H).astype(np.float64)
    assert np.all(np.isfinite(got))
    ref = oracle.w4a16_swiglu(c.A, c.q, c.s, c.z, g, fold=True)
    assert rel_fro(got, ref) <= TOL
    assert elementwise_guard(got, ref) <= 0
