"""GPU parity of the decode kernel's balanced grid.

When the plain decode grid leaves a small remainder over whole rounds of 256
CUs, the column groups that fill those rounds keep their split count and the
last ones take several times as many shorter K splits (or, in a grid that
splits nothing else, are the only ones split).  Each column group keeps one
counter and adds its partial sums in split order.  Here every column of the
finer-split column groups, and a block of the others, is compared with the
oracle ("Marlin INT4 on Ada - how it works", "The core mismatch: symmetric
vs asymmetric": W = q s + z, with AWQ-style zero-points so that the delta
term is as large as the scale term), over the factor boundaries:
K5120 x N17408 at M = 1 and 4 (last 16 column groups in 4 splits) and M = 48
(three m-tiles, in 8 splits), and the unsplit 34816-column grid at M = 1 (its
last 32 column groups in 4 splits) and M = 16 (in 8).  Repeated calls must be
bitwise identical and leave the workspace's counters at zero."""
import ctypes

import numpy as np
import pytest
import torch

import int4_weight_only_uint32_amd as qg
import oracle
import synth
from tests.gpu_util import dev, elementwise_guard, host, note, rel_fro

pytestmark = pytest.mark.gpu

TOL = 2e-3
COLS = 64          # columns per decode workgroup


def _p(t):
    return ctypes.c_void_p(t.data_ptr()) if t is not None else None


@pytest.mark.parametrize("M,N,main_cgs", [(1, 17408, 256), (4, 17408, 256), (48, 17408, 256),
                                          (1, 34816, 512), (16, 34816, 512)])
def test_balanced_decode_grid(M, N, main_cgs):
    K, g = 5120, 128
    note(f"balanced grid M={M} K={K} N={N}")
    c = synth.w4a16_case(M, K, N, g, asym=True, stream=97, case_id=M * 7 + N,
                         name="balanced-grid", zero_points="awq")
    pw = qg.pack(dev(c.q), dev(c.s), dev(c.z), g, fold=True)
    A = dev(c.A)
    L = qg.lib()
    nb = L.qg_workspace_bytes(qg.QG_OP_W4A16, M, N, K, g, 1, 0)
    assert nb > qg.QG_W4A16_WS_COUNTER_BYTES       # the finer splits need partial sums
    ws = torch.zeros(nb, dtype=torch.uint8, device="cuda")
    st = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    outs = []
    for rep in range(3):
        C = torch.full((M, N), float("nan"), dtype=torch.float16, device="cuda")
        rc = L.qgemm_w4a16(_p(A), _p(pw.w), _p(pw.scale), _p(pw.delta), _p(C), M, N, K, g, 0,
                           _p(ws), ws.numel(), st)
        assert rc == qg.QG_OK, L.qg_last_error()
        torch.cuda.synchronize()
        assert int(ws[:qg.QG_W4A16_WS_COUNTER_BYTES].count_nonzero()) == 0
        outs.append(host(C))
    for o in outs[1:]:
        assert np.array_equal(o.view(np.uint16), outs[0].view(np.uint16))
    got = outs[0].astype(np.float64)
    # every column of the finer-split column groups, and the first 256 others
    cols = np.concatenate([np.arange(0, 256), np.arange(main_cgs * COLS, N)])
    ref = oracle.w4a16(c.A, c.q[:, cols], c.s[:, cols], c.z[:, cols], g)
    assert np.all(np.isfinite(got[:, cols]))
    assert rel_fro(got[:, cols], ref) <= TOL
    assert elementwise_guard(got[:, cols], ref) <= 0
