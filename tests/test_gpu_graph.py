"""HIP-graph capture of the library's calls, the multi-launch ones included
(the split-K decode with its self-resetting counters, the separate
correction's three launches, the quantizer followed by the W4A8 GEMM): one
graph holds all of them, and every replay -- with new inputs written in
place and eager work and synchronizations between replays -- must equal the
eager calls on the same inputs, bit for bit.  No call records a memset: the
split-K counters are left at zero by each call instead."""
import numpy as np
import pytest
import torch

import int4_weight_only_uint32_amd as qg
import synth
from tests.gpu_util import dev, note

pytestmark = pytest.mark.gpu


def test_graph_replays_match_eager():
    assert torch.cuda.is_available() and qg.qg_device_supported(0)
    torch.cuda.set_device(0)
    c = synth.w4a16_case(16, 16384, 4096, 128, asym=True, stream=90, case_id=0)   # 8 k-splits
    pw = qg.pack(dev(c.q), dev(c.s), dev(c.z), 128)
    w8 = synth.w4a8_case(2, 24, 512, 256, 128, stream=90, case_id=1, asym=True)
    p8 = [qg.pack(dev(w8.q[e]), dev(w8.s[e]), dev(w8.z[e]), 128) for e in range(2)]
    W8 = torch.stack([p.w for p in p8]).contiguous()
    S8 = torch.stack([p.scale for p in p8]).contiguous()
    D8 = torch.stack([p.delta for p in p8]).contiguous()
    off = dev(w8.offsets)
    M, K, N = 16, 16384, 4096
    A = dev(c.A)
    A8 = dev(w8.A16)
    n_ws = max(qg.qg_workspace_bytes(qg.QG_OP_W4A16, M, N, K, 128, 1, f) for f in (0, 1))
    ws1 = torch.zeros(n_ws, dtype=torch.uint8, device="cuda")
    ws2 = torch.zeros(n_ws, dtype=torch.uint8, device="cuda")
    C1 = torch.empty((M, N), dtype=torch.float16, device="cuda")
    C2 = torch.empty((M, N), dtype=torch.float16, device="cuda")
    Aq = torch.empty((w8.M_total, 512), dtype=torch.int8, device="cuda")
    asc = torch.empty((w8.M_total,), dtype=torch.float32, device="cuda")
    C8 = torch.empty((w8.M_total, 256), dtype=torch.float16, device="cuda")

    def calls():
        qg.qgemm_w4a16(A, pw.w, pw.scale, pw.delta, C1, M, N, K, 128, 0, ws1)
        qg.qgemm_w4a16(A, pw.w, pw.scale, pw.delta, C2, M, N, K, 128, qg.QG_CORR_SEPARATE, ws2)
        qg.quantize_rows_int8(A8, w8.M_total, 512, Aq, asc)
        qg.qgemm_w4a8(Aq, asc, W8, S8, off, 2, w8.M_total, 24, 256, 512, 128, C8, w_delta=D8)

    def outputs():
        return [t.clone() for t in (C1, C2, Aq, asc, C8)]

    note("graph: capture")
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        calls()                      # warm-up on the capture stream
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        calls()
    torch.cuda.synchronize()

    rng = np.random.default_rng(3)
    for rep in range(4):
        note(f"graph: replay {rep}")
        # new inputs in place, then eager reference results
        A.copy_(dev(rng.standard_normal((M, K)).astype(np.float16)))
        A8.copy_(dev(rng.standard_normal((w8.M_total, 512)).astype(np.float16)))
        torch.cuda.synchronize()
        calls()
        torch.cuda.synchronize()
        ref = outputs()
        for t in (C1, C2, Aq, asc, C8):
            t.zero_()
        torch.cuda.synchronize()
        junk = (torch.randn(256, 256, device="cuda") @ torch.randn(256, 256, device="cuda")).sum()
        g.replay()
        torch.cuda.synchronize()
        got = outputs()
        assert float(junk) == float(junk)
        for r, o in zip(ref, got):
            assert torch.equal(r, o), rep
    # the split-K counters are back at zero after every call
    assert int(ws1[:qg.QG_W4A16_WS_COUNTER_BYTES].count_nonzero()) == 0
    assert int(ws2[:qg.QG_W4A16_WS_COUNTER_BYTES].count_nonzero()) == 0
