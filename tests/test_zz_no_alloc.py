"""qgemm_w4a16_noalloc (the W4A16 GEMM on the library's static device
scratch, for callers that cannot allocate) against qgemm_w4a16 with a
caller workspace, through the C ABI.  Both run the same kernels, so their
outputs must be bit-identical; both are also held to the oracle at the W4A16
bar.  Each sequence makes two calls in a row, the second on a smaller input,
so the second runs on scratch the first has written."""
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


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr()) if t is not None else None


def _noalloc(A, pw, C, M, flags):
    st = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    return qg.lib().qgemm_w4a16_noalloc(_ptr(A), _ptr(pw.w), _ptr(pw.scale), _ptr(pw.delta),
                                        _ptr(C), M, pw.N, pw.K, pw.group_size, flags, st)


def _with_workspace(A, pw, C, M, flags):
    n = qg.qg_workspace_bytes(qg.QG_OP_W4A16, M, pw.N, pw.K, pw.group_size, 1,
                              flags if pw.delta is not None else 0)
    ws = torch.zeros(max(n, 256), dtype=torch.uint8, device="cuda")
    st = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    rc = qg.lib().qgemm_w4a16(_ptr(A), _ptr(pw.w), _ptr(pw.scale), _ptr(pw.delta), _ptr(C), M,
                              pw.N, pw.K, pw.group_size, flags, _ptr(ws), ws.numel(), st)
    return rc, n


# (M, K, N, g, asym, flags): the split-K decode kernel (partial sums and
# counters in the scratch), then a smaller split-K decode call; a tail shape
# (padded A and C in the scratch), then a smaller one; the separate
# correction (group sums in the scratch), then a smaller one
SEQUENCES = [
    [(16, 5120, 17408, 128, True, 0), (4, 17408, 5120, 128, True, 0)],
    [(16, 1000, 3000, 128, True, 0), (3, 1000, 300, -1, True, 0)],
    [(16, 4096, 8192, 128, True, qg.QG_CORR_SEPARATE), (9, 2048, 1024, 256, True, qg.QG_CORR_SEPARATE)],
    [(16, 16384, 4096, 128, False, 0), (1, 5120, 17408, -1, False, 0)],
    # the decode kernel with five m-tiles (80-row partial sums), then two
    [(80, 5120, 17408, 128, True, 0), (20, 2048, 8704, 128, True, 0)],
]


@pytest.mark.parametrize("seq", range(len(SEQUENCES)))
def test_noalloc_matches_workspace_entry_point(seq):
    assert torch.cuda.is_available() and qg.qg_device_supported(0)
    torch.cuda.set_device(0)
    for i, (M, K, N, g, asym, flags) in enumerate(SEQUENCES[seq]):
        gg = K if g == -1 else g
        c = synth.w4a16_case(M, K, N, gg, asym=asym, signed_scales=not asym, stream=95,
                             case_id=100 * seq + i)
        note(f"noalloc seq {seq} call {i}: M={M} K={K} N={N} g={gg} asym={asym} flags={flags}")
        pw = qg.pack(dev(c.q), dev(c.s), dev(c.z) if asym else None, g, fold=True)
        A = dev(c.A)
        assert qg.qg_workspace_bytes(qg.QG_OP_W4A16, M, N, K, g, 1, flags) <= qg.QG_NOALLOC_SCRATCH_BYTES
        C1 = torch.full((M, N), float("nan"), dtype=torch.float16, device="cuda")
        C2 = torch.full((M, N), float("nan"), dtype=torch.float16, device="cuda")
        assert _noalloc(A, pw, C1, M, flags) == qg.QG_OK, qg.lib().qg_last_error()
        rc, _ = _with_workspace(A, pw, C2, M, flags)
        assert rc == qg.QG_OK
        torch.cuda.synchronize()
        got1 = host(C1).astype(np.float64)
        got2 = host(C2).astype(np.float64)
        assert np.array_equal(got1, got2)
        ref = oracle.w4a16(c.A, c.q, c.s, c.z if asym else None, gg, fold=True)
        assert rel_fro(got1, ref) <= TOL
        assert elementwise_guard(got1, ref) <= 0
