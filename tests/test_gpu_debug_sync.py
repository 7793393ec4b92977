"""Race check: every GEMM kernel family against its QG_DEBUG_SYNC build.

libqgemm_debugsync.so is built from the same sources with every pipeline
stage waiting for all of the wave's outstanding memory operations (nothing
loaded ahead stays in flight across a stage) and every call waiting for its
kernels.  The arithmetic and its order are unchanged, so both libraries must
produce the same bits on the same inputs; a missing wait in the normal build
would show as a difference in some tiles -- the failure mode of the SGLang
w4a8 article (preface: a race that corrupts a subset of the output)."""
import ctypes

import pytest
import torch

import int4_weight_only_uint32_amd as qg
import synth
from tests.gpu_util import dev, note

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def libs():
    assert torch.cuda.is_available()
    assert qg.qg_device_supported(0), "GPU visible but not gfx950"
    return qg.lib(), qg.debug_sync_lib()


def _p(t):
    return ctypes.c_void_p(t.data_ptr()) if t is not None else None


def _stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _w4a16_both(libs, fn_name, M, K, N, g, asym, signed=False, op=qg.QG_OP_W4A16, flags=0):
    """Run one W4A16 (or SwiGLU) call through both libraries; returns the two
    outputs.  N is the output width (the pair is 2N wide for SwiGLU)."""
    Nw = 2 * N if op == qg.QG_OP_W4A16_SWIGLU else N
    c = synth.w4a16_case(M, K, Nw, g, asym=asym, signed_scales=signed, stream=96,
                         case_id=M + K + N, zero_points="awq" if asym else "noise")
    pw = qg.pack(dev(c.q), dev(c.s), dev(c.z) if asym else None, g, fold=True)
    A = dev(c.A)
    outs = []
    for L in libs:
        nb = L.qg_workspace_bytes(op, M, N, K, g, 1, flags)
        ws = torch.zeros(max(nb, 256), dtype=torch.uint8, device="cuda")
        C = torch.full((M, N), float("nan"), dtype=torch.float16, device="cuda")
        rc = getattr(L, fn_name)(_p(A), _p(pw.w), _p(pw.scale), _p(pw.delta), _p(C), M, N, K, g,
                                 flags, _p(ws), ws.numel(), _stream())
        assert rc == qg.QG_OK, L.qg_last_error()
        torch.cuda.synchronize()
        assert int(ws[:min(ws.numel(), qg.QG_W4A16_WS_COUNTER_BYTES)].count_nonzero()) == 0
        outs.append(C)
    return outs


# one shape per kernel path: decode (2 and 6 K-splits), skinny, the two mid
# kernels, 64x128 tiled (fused delta), 128x256 tiled (fused delta and the
# symmetric hand-ordered kernel), the row split, the separate correction,
# groups of 64 and 32 (decode, skinny, 8-wave mid and generic tiled kernels)
@pytest.mark.parametrize("M,K,N,g,asym,flags", [
    (16, 5120, 17408, 128, True, 0),
    (4, 17408, 5120, 128, True, 0),
    (33, 1024, 1024, 128, True, 0),
    (200, 2048, 1024, 128, True, 0),
    (256, 2048, 4096, 256, True, 0),
    (512, 2048, 4096, 128, True, 0),
    (2048, 1024, 8192, 128, True, 0),
    (2048, 1024, 8192, 128, False, 0),
    (4096, 1024, 17408, 128, False, 0),
    (16, 4096, 4096, 128, True, qg.QG_CORR_SEPARATE),
    (48, 2048, 8704, 128, True, 0),         # decode with three m-tiles
    (80, 17408, 5120, 128, False, 0),
    (16, 4096, 4096, 64, True, 0),          # groups of 64 and 32
    (33, 2048, 1024, 64, True, 0),
    (64, 4096, 2048, 32, False, 0),
    (256, 2048, 8192, 64, True, 0),
    (512, 2048, 4096, 32, True, 0),
    (2048, 1024, 8192, 64, False, 0),
])
def test_w4a16_matches_debug_sync_build(libs, M, K, N, g, asym, flags):
    note(f"debug-sync w4a16 M={M} K={K} N={N} g={g} asym={asym} flags={flags}")
    a, b = _w4a16_both(libs, "qgemm_w4a16", M, K, N, g, asym, signed=not asym, flags=flags)
    assert torch.isfinite(a.float()).all()
    assert torch.equal(a, b)


@pytest.mark.parametrize("M,K,N", [(16, 5120, 17408), (64, 2048, 2048), (512, 1024, 4096)])
def test_swiglu_matches_debug_sync_build(libs, M, K, N):
    note(f"debug-sync swiglu M={M} K={K} N={N}")
    a, b = _w4a16_both(libs, "qgemm_w4a16_swiglu", M, K, N, 128, True, op=qg.QG_OP_W4A16_SWIGLU)
    assert torch.isfinite(a.float()).all()
    assert torch.equal(a, b)


@pytest.mark.parametrize("g,asym", [(128, False), (128, True), (256, False), (64, True), (32, False), (32, True)])
def test_w4a8_matches_debug_sync_build(libs, g, asym):
    note(f"debug-sync w4a8 8x64 K=2048 N=7168 g={g} asym={asym}")
    c = synth.w4a8_case(8, 64, 2048, 7168, g, stream=96, case_id=g + asym, asym=asym)
    packs = [qg.pack(dev(c.q[e]), dev(c.s[e]), dev(c.z[e]) if asym else None, g) for e in range(c.E)]
    W = torch.stack([p.w for p in packs]).contiguous()
    S = torch.stack([p.scale for p in packs]).contiguous()
    D = torch.stack([p.delta for p in packs]).contiguous() if asym else None
    Aq, asc, off = dev(c.Aq), dev(c.a_scale), dev(c.offsets)
    outs = []
    for L in libs:
        # the production kernel, then the one that also stores the integer
        # group products
        C = torch.full((c.M_total, c.N), float("nan"), dtype=torch.float16, device="cuda")
        rc = L.qgemm_w4a8(_p(Aq), _p(asc), _p(W), _p(S), _p(D), _p(off), c.E, c.M_total, 64, c.N,
                          c.K, g, _p(C), None, None, 0, 0, _stream())
        assert rc == qg.QG_OK, L.qg_last_error()
        C2 = torch.full_like(C, float("nan"))
        acc = torch.zeros((c.M_total, c.K // g, c.N), dtype=torch.int32, device="cuda")
        rc = L.qgemm_w4a8(_p(Aq), _p(asc), _p(W), _p(S), _p(D), _p(off), c.E, c.M_total, 64, c.N,
                          c.K, g, _p(C2), _p(acc), None, 0, 0, _stream())
        assert rc == qg.QG_OK, L.qg_last_error()
        torch.cuda.synchronize()
        outs.append((C, C2, acc))
    assert torch.isfinite(outs[0][0].float()).all()
    for x, y in zip(outs[0], outs[1]):
        assert torch.equal(x, y)


def test_quantizer_matches_debug_sync_build(libs):
    note("debug-sync quantize_rows_int8 4096x5120")
    A = dev(synth.activations(4096, 5120, stream=96, case_id=7))
    outs = []
    for L in libs:
        q = torch.empty((4096, 5120), dtype=torch.int8, device="cuda")
        s = torch.empty(4096, dtype=torch.float32, device="cuda")
        rc = L.quantize_rows_int8(_p(A), 4096, 5120, _p(q), _p(s), _stream())
        assert rc == qg.QG_OK, L.qg_last_error()
        torch.cuda.synchronize()
        outs.append((q, s))
    assert torch.equal(outs[0][0], outs[1][0]) and torch.equal(outs[0][1], outs[1][1])


def test_first_dispatch_log_line():
    """QGEMM_LOG=1: one stderr line per distinct call, on its first launch
    ("Marlin INT4 on Ada - how it works", "End-to-end result on RTX 4090")."""
    import os
    import subprocess
    import sys
    code = (
        "import numpy as np, torch, synth, int4_weight_only_uint32_amd as qg\n"
        "c = synth.w4a16_case(16, 1024, 1024, 128, stream=96, case_id=1)\n"
        "d = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()\n"
        "pw = qg.pack(d(c.q), d(c.s), d(c.z), 128)\n"
        "A = d(c.A)\n"
        "qg.w4a16(A, pw); qg.w4a16(A, pw); qg.w4a16(A[:4], pw)\n"
        "torch.cuda.synchronize()\n")
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    env = dict(os.environ, QGEMM_LOG="1", PYTHONPATH=root)
    r = subprocess.run([sys.executable, "-c", code], env=env, cwd=root, capture_output=True,
                       text=True, timeout=300)
    assert r.returncode == 0, r.stderr[-2000:]
    lines = [l for l in r.stderr.splitlines() if l.startswith("[qgemm] first dispatch ok:")]
    assert sum("pack_int4_weights K=1024 N=1024 gs=128 asymmetric" in l for l in lines) == 1, lines
    assert sum("qgemm_w4a16 M=16 N=1024 K=1024 gs=128 asymmetric" in l for l in lines) == 1, lines
    assert sum("qgemm_w4a16 M=4 N=1024 K=1024 gs=128 asymmetric" in l for l in lines) == 1, lines
