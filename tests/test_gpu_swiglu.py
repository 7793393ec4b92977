"""GPU parity of the SwiGLU of a gate/up pair (one packed [K, 2N] weight,
gate columns first) against the oracle's silu(A . W_gate) * (A . W_up): one
launch at every batch size, the gate and up products of the same columns
held in fp32 and H rounded once -- the gated decode kernel (M <= 16, split-K
included) and the gated epilogues of the skinny, mid and tiled kernels
(64x128, 128x256 with fused delta, the symmetric 128x256 kernel, and the
prefill-size pair with its row split), symmetric and asymmetric weights."""
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


def _check(M, K, N, g, asym=True, signed=False, case_id=0, rows=None):
    """rows: the output rows compared with the oracle (all by default)."""
    c = synth.w4a16_case(M, K, 2 * N, g, asym=asym, signed_scales=signed, stream=91,
                         case_id=case_id)
    note(f"swiglu M={M} K={K} N={N} g={g} asym={asym} signed={signed}")
    pair = qg.pack(dev(c.q), dev(c.s), dev(c.z) if asym else None, g, fold=True)
    # only the decode kernel (M <= 80) takes a workspace, for its split-K
    assert qg.qg_workspace_bytes(qg.QG_OP_W4A16_SWIGLU, M, N, K, g, 1, 0) == 0 or M <= 80
    H = torch.full((M, N), float("nan"), dtype=torch.float16, device="cuda")
    qg.w4a16_swiglu(dev(c.A), pair, H=H)
    torch.cuda.synchronize()
    got = host(H).astype(np.float64)
    assert np.all(np.isfinite(got))
    rows = np.arange(M) if rows is None else rows
    ref = oracle.w4a16_swiglu(c.A[rows], c.q, c.s, c.z if asym else None, c.g, fold=True)
    err = rel_fro(got[rows], ref)
    assert err <= TOL, err
    assert elementwise_guard(got[rows], ref) <= 0
    return err


@pytest.mark.parametrize("M", [1, 4, 16])
def test_swiglu_decode_mlp_shape(M):
    """The gate and up projections of the MLP, K 5120 -> N 17408 each."""
    err = _check(M, 5120, 17408, 128, case_id=M)
    note(f"rel_fro {err:.3e}")


@pytest.mark.parametrize("M,K,N,g", [(16, 17408, 5120, 128), (9, 16384, 2048, -1)])
def test_swiglu_decode_split_k(M, K, N, g):
    assert qg.qg_workspace_bytes(qg.QG_OP_W4A16_SWIGLU, M, N, K, g, 1, 0) > 0
    _check(M, K, N, g, case_id=20 + M)


def test_swiglu_decode_symmetric_signed():
    _check(8, 4096, 2048, 128, asym=False, signed=True, case_id=30)


# skinny (M = 1 where the decode kernel is not chosen, M = 33), mid (per-column
# and g128 with a ragged last row tile)
@pytest.mark.parametrize("M,K,N,g", [(1, 1024, 512, 128), (33, 1024, 1024, 256),
                                     (256, 2048, 1024, -1), (300, 1024, 2048, 128)])
def test_swiglu_fused_small_batches(M, K, N, g):
    _check(M, K, N, g, case_id=40 + M)


def _band_rows(M, every):
    """One row of every `every`-row band, at a varying offset in the band."""
    i = np.arange((M + every - 1) // every)
    return np.minimum(every * i + i % every, M - 1)


# the 8-wave mid-batch kernel (K split inside the workgroup), gated
@pytest.mark.parametrize("M,K,N,g", [(256, 2048, 4096, 256), (192, 1152, 8192, 128)])
def test_swiglu_fused_mid_ksplit(M, K, N, g):
    _check(M, K, N, g, case_id=50 + M + K)


# tiled kernels: 64x128 tiles (fused delta, and symmetric), 128x256 tiles with
# the fused delta, the symmetric 128x256 kernel (random-sign scales, folded)
@pytest.mark.parametrize("M,K,N,asym", [(512, 2048, 4096, True), (512, 1024, 4096, False),
                                        (2048, 1024, 8192, True), (2048, 1024, 8192, False)])
def test_swiglu_fused_tiled(M, K, N, asym):
    _check(M, K, N, 128, asym=asym, signed=not asym, case_id=60 + M + asym,
           rows=_band_rows(M, 16))


def test_swiglu_fused_prefill_pair():
    """The MLP pair at prefill size (M 4096, K 5120 -> N 17408 per half,
    symmetric, random-sign scales): 128x256 tiles over the first 3840 rows
    and a second launch over the rest, checked on one row of every 64-row
    band plus one row of every 16-row band of the second launch."""
    M = 4096
    rows = np.unique(np.concatenate([_band_rows(M, 64), 3840 + _band_rows(256, 16)]))
    _check(M, 5120, 17408, 128, asym=False, signed=True, case_id=80, rows=rows)


def test_swiglu_shares_a_workspace_with_w4a16():
    """One zero-filled workspace serves SwiGLU and W4A16 calls in turn (the
    counter region is common and left at zero)."""
    M, K, N, g = 16, 17408, 5120, 128
    c = synth.w4a16_case(M, K, 2 * N, g, stream=91, case_id=50)
    pair = qg.pack(dev(c.q), dev(c.s), dev(c.z), g)
    n = max(qg.qg_workspace_bytes(qg.QG_OP_W4A16_SWIGLU, M, N, K, g, 1, 0),
            qg.qg_workspace_bytes(qg.QG_OP_W4A16, M, 2 * N, K, g, 1, 0))
    ws = torch.zeros(n, dtype=torch.uint8, device="cuda")
    A = dev(c.A)
    H1 = qg.w4a16_swiglu(A, pair, workspace=ws)
    Y = qg.w4a16(A, pair, workspace=ws)
    H2 = qg.w4a16_swiglu(A, pair, workspace=ws)
    torch.cuda.synchronize()
    assert torch.equal(H1, H2)
    Yf = Y.float()
    Hy = (Yf[:, :N] * torch.sigmoid(Yf[:, :N]) * Yf[:, N:]).cpu().numpy()
    assert rel_fro(host(H1).astype(np.float64), Hy.astype(np.float64)) <= TOL
    assert int(ws[:qg.QG_W4A16_WS_COUNTER_BYTES].count_nonzero()) == 0
