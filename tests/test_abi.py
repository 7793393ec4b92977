"""CPU checks of the C ABI: the library loads, exports every entry point the
header declares, and rejects bad arguments on the host before touching a
device.  No compute call is made here."""
import ctypes
import os
import re

import pytest

import int4_weight_only_uint32_amd as qg

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "qgemm.h")

P = ctypes.c_void_p
FAKE = P(0x10000)     # never dereferenced: validation fails (or the device check does) first


def _declared(header=HEADER):
    txt = open(header).read()
    txt = re.sub(r"/\*.*?\*/", "", txt, flags=re.S)
    return sorted(set(re.findall(r"\b([a-z_][a-z0-9_]*)\s*\(", txt)) - {"defined"})


def test_header_declares_the_four_calls():
    names = _declared()
    for n in ("pack_int4_weights", "qgemm_w4a16", "group_sum_correction", "qgemm_w4a8"):
        assert n in names


def test_library_exports_every_declared_symbol():
    L = qg.lib()
    for n in _declared():
        assert hasattr(L, n), n
    assert sorted(qg.EXPORTED) == _declared()


def test_debug_sync_library_exports_every_declared_symbol():
    """The QG_DEBUG_SYNC build (race checks) carries the same entry points
    and validates arguments the same way."""
    L = qg.debug_sync_lib()
    for n in _declared():
        assert hasattr(L, n), n
    assert L.qgemm_w4a16(None, FAKE, FAKE, None, FAKE, 16, 128, 128, 128, 0, None, 0, None) \
        == qg.QG_ERR_INVALID_ARG
    assert b"qgemm_w4a16" in L.qg_last_error()


def test_probe_library_exports_every_declared_symbol():
    from int4_weight_only_uint32_amd import probe
    L = probe.lib()
    names = _declared(os.path.join(ROOT, "include", "qgprobe.h"))
    for n in names:
        assert hasattr(L, n), n
    assert sorted(probe.EXPORTED) == names
    # host-side argument checks: rejected before any launch
    assert L.qgprobe_mfma_f16(8, FAKE, 1, 1, None) == 1
    assert L.qgprobe_mfma_f16(16, FAKE, 0, 1, None) == 1
    assert L.qgprobe_hbm_read(FAKE, 4096, FAKE, 1, 3, None) == 1
    assert L.qgprobe_hbm_read(FAKE, 4096, FAKE, 1, 32, None) == 1
    assert L.qgprobe_hbm_read(FAKE, 100, FAKE, 1, 2, None) == 1
    assert L.qgprobe_mfma_flops(16, 2, 3) == 16 * 16 * 32 * 2 * 16 * 3 * 2 * 4
    assert L.qgprobe_mfma_flops(32, 2, 3) == 32 * 32 * 16 * 2 * 4 * 3 * 2 * 4
    assert L.qgprobe_mfma_flops(64, 2, 3) == 16 * 16 * 64 * 2 * 16 * 3 * 2 * 4
    assert L.qgprobe_mfma_flops(7, 2, 3) == 0
    assert L.qgprobe_mfma_i8(FAKE, 0, 1, None) == 1


def test_status_strings():
    L = qg.lib()
    for s in range(6):
        assert L.qg_status_string(s)
    assert L.qg_status_string(99) == b"unknown status"


def _w4a16(M=16, N=1024, K=1024, g=128, A=FAKE, W=FAKE, S=FAKE, D=None, C=FAKE, flags=0,
           ws=None, wsb=0):
    return qg.lib().qgemm_w4a16(A, W, S, D, C, M, N, K, g, flags, ws, wsb, None)


@pytest.mark.parametrize("kw,rc", [
    (dict(K=1000), qg.QG_ERR_WORKSPACE),               # tails: A padded / C cropped in the workspace
    (dict(N=1000), qg.QG_ERR_WORKSPACE),
    (dict(K=1000, D=FAKE, flags=qg.QG_CORR_SEPARATE), qg.QG_ERR_UNSUPPORTED),
    (dict(K=1000, g=384), qg.QG_ERR_WORKSPACE),        # a partial last group
    (dict(M=0), qg.QG_ERR_INVALID_ARG),
    (dict(g=100), qg.QG_ERR_INVALID_ARG),
    (dict(g=48, K=1152), qg.QG_ERR_UNSUPPORTED),       # divides K, but not 32, 64 or 128k
    (dict(g=16), qg.QG_ERR_UNSUPPORTED),
    (dict(K=1000, g=64), qg.QG_ERR_WORKSPACE),         # groups of 64 with a K tail
    (dict(A=None), qg.QG_ERR_INVALID_ARG),
    (dict(C=None), qg.QG_ERR_INVALID_ARG),
    (dict(A=P(0x10002)), qg.QG_ERR_INVALID_ARG),
    (dict(W=P(0x10008)), qg.QG_ERR_INVALID_ARG),
    (dict(flags=8), qg.QG_ERR_INVALID_ARG),
    (dict(D=FAKE, flags=qg.QG_CORR_SEPARATE), qg.QG_ERR_WORKSPACE),
    (dict(D=FAKE, flags=qg.QG_CORR_SEPARATE, ws=FAKE, wsb=16), qg.QG_ERR_WORKSPACE),
])
def test_w4a16_validation(kw, rc):
    assert _w4a16(**kw) == rc
    assert qg.lib().qg_last_error()


def test_valid_arguments_reach_the_device_check():
    # large M needs no workspace: with no GPU the call must stop at the device check
    rc = _w4a16(M=256)
    assert rc == qg.QG_ERR_DEVICE
    assert b"device" in qg.lib().qg_last_error()
    rc = _w4a16(M=256, g=-1)
    assert rc == qg.QG_ERR_DEVICE
    for g in (32, 64):                     # groups of 32 and 64 are served
        assert _w4a16(M=256, g=g) == qg.QG_ERR_DEVICE


def test_split_k_workspace_is_required_and_sized():
    n = qg.qg_workspace_bytes(qg.QG_OP_W4A16, 16, 5120, 17408, 128)
    assert n >= 0
    if n > 0:
        assert _w4a16(M=16, N=5120, K=17408) == qg.QG_ERR_WORKSPACE
        assert _w4a16(M=16, N=5120, K=17408, ws=FAKE, wsb=n - 1) == qg.QG_ERR_WORKSPACE
        assert _w4a16(M=16, N=5120, K=17408, ws=P(0x10080), wsb=n) == qg.QG_ERR_INVALID_ARG  # alignment
        assert _w4a16(M=16, N=5120, K=17408, ws=FAKE, wsb=n) == qg.QG_ERR_DEVICE


def test_pack_validation():
    L = qg.lib()
    assert L.pack_int4_weights(FAKE, FAKE, FAKE, 1024, 1024, 128, 1, FAKE, FAKE, None, None) == qg.QG_ERR_INVALID_ARG
    # N tail: the padded scale_out cannot alias scale
    assert L.pack_int4_weights(FAKE, FAKE, None, 1024, 1000, 128, 1, FAKE, FAKE, None, None) == qg.QG_ERR_INVALID_ARG
    assert b"alias" in L.qg_last_error()
    # groups of 64 over K = 1025: the pack holds 18 groups (K padded to 1152),
    # the input scale 17 rows -- scale_out cannot alias it either
    assert L.pack_int4_weights(FAKE, FAKE, None, 1025, 1024, 64, 1, FAKE, FAKE, None, None) == qg.QG_ERR_INVALID_ARG
    assert b"alias" in L.qg_last_error()
    kp, np_, gg = qg.padded_shape(1025, 1024, 64)
    assert (kp, np_, gg) == (1152, 1024, 18)
    assert qg.padded_shape(1025, 1024, 32) == (1152, 1024, 36)
    assert L.pack_int4_weights(FAKE, FAKE, None, 1024, 1024, 64, 1, FAKE, FAKE, None, None) == qg.QG_ERR_DEVICE
    assert L.pack_int4_weights(FAKE, FAKE, None, 1024, 1000, 100, 1, FAKE, P(0x20000), None, None) == qg.QG_ERR_INVALID_ARG
    assert L.pack_int4_weights(FAKE, FAKE, None, 1024, 1024, 128, 4, FAKE, FAKE, None, None) == qg.QG_ERR_INVALID_ARG
    assert L.pack_int4_weights(None, FAKE, None, 1024, 1024, 128, 1, FAKE, FAKE, None, None) == qg.QG_ERR_INVALID_ARG


def test_w4a8_validation():
    L = qg.lib()
    args = lambda **kw: [kw.get("A", FAKE), FAKE, FAKE, FAKE, kw.get("D", None), kw.get("off", None), kw.get("E", 1),
                         kw.get("M", 64), kw.get("mr", 64), 1024, kw.get("K", 1024), 128, FAKE,
                         None, None, 0, kw.get("flags", 0), None]
    assert L.qgemm_w4a8(*args(E=2)) == qg.QG_ERR_INVALID_ARG          # offsets needed
    assert L.qgemm_w4a8(*args(mr=0)) == qg.QG_ERR_INVALID_ARG
    assert L.qgemm_w4a8(*args(mr=32)) == qg.QG_ERR_INVALID_ARG        # one expert must cover all rows
    assert L.qgemm_w4a8(*args(flags=1)) == qg.QG_ERR_INVALID_ARG
    assert L.qgemm_w4a8(*args(A=P(0x10004))) == qg.QG_ERR_INVALID_ARG
    assert L.qgemm_w4a8(*args(K=1000)) == qg.QG_ERR_WORKSPACE        # tails: A_q padded in the workspace
    tail_acc = args(K=1000)
    tail_acc[13] = FAKE                                                # acc_debug with a tail
    tail_acc[14], tail_acc[15] = P(0x100000), 1 << 30
    assert L.qgemm_w4a8(*tail_acc) == qg.QG_ERR_UNSUPPORTED
    assert L.qgemm_w4a8(*args(D=P(0x10001))) == qg.QG_ERR_INVALID_ARG  # misaligned deltas
    for g in (32, 64):                                                 # served
        gs = args()
        gs[11] = g
        assert L.qgemm_w4a8(*gs) == qg.QG_ERR_DEVICE
        assert qg.qg_workspace_bytes(qg.QG_OP_W4A8, 64, 1024, 1024, g, 1) == 0
    g48 = args(K=1152)
    g48[11] = 48                                                       # divides K, not 32, 64 or 128k
    assert L.qgemm_w4a8(*g48) == qg.QG_ERR_UNSUPPORTED


def test_group_sum_correction_validation():
    L = qg.lib()
    assert L.group_sum_correction(FAKE, FAKE, FAKE, 4, 1024, 1024, 128, None, 0, None) == qg.QG_ERR_WORKSPACE
    assert L.group_sum_correction(FAKE, FAKE, FAKE, 4, 1024, 1024, 128, FAKE, 4 * 8 * 4 - 1, None) == qg.QG_ERR_WORKSPACE
    assert L.group_sum_correction(None, FAKE, FAKE, 4, 1024, 1024, 128, FAKE, 4096, None) == qg.QG_ERR_INVALID_ARG


CTR = 65536   # QG_W4A16_WS_COUNTER_BYTES


def test_decode_workspace_size():
    # the fixed counter region + fp32 partials (16 rows per m-tile x 64
    # columns per split per 64-column group).  Splits: the most that keep <= 512
    # workgroups (two per CU) when that fills >= 448 of them, else the smallest
    # power of two giving >= 512 workgroups; >= 2 k-tiles per split.  A small
    # remainder over whole rounds of 256 CUs is balanced: at N = 17408 the
    # first 256 column groups keep 2 splits and the last 16 take 8 (M > 8,
    # splits of >= 5 k-tiles) or 4 (M <= 8, >= 10 k-tiles), one slot each.
    assert qg.qg_workspace_bytes(qg.QG_OP_W4A16, 16, 17408, 5120, 128) == CTR + (256 * 2 + 16 * 8) * 4096
    assert qg.qg_workspace_bytes(qg.QG_OP_W4A16, 4, 17408, 5120, 128) == CTR + (256 * 2 + 16 * 4) * 4096
    # unsplit grids with such a remainder split only their last column groups:
    # the gate/up pair's 34816 columns (512 + 32 groups, K = 5120) and a
    # 50304-column head (768 + 18)
    assert qg.qg_workspace_bytes(qg.QG_OP_W4A16, 16, 34816, 5120, 128) == CTR + 32 * 8 * 4096
    assert qg.qg_workspace_bytes(qg.QG_OP_W4A16, 1, 34816, 5120, 128) == CTR + 32 * 4 * 4096
    assert qg.qg_workspace_bytes(qg.QG_OP_W4A16, 16, 50304, 5120, 128) == CTR + 18 * 8 * 4096
    assert qg.qg_workspace_bytes(qg.QG_OP_W4A16, 9, 5120, 17408, 128) == CTR + 80 * 6 * 4096
    assert qg.qg_workspace_bytes(qg.QG_OP_W4A16, 16, 4096, 16384, 128) == CTR + 64 * 8 * 4096
    # short decode splits lose to the skinny kernel, which needs none
    assert qg.qg_workspace_bytes(qg.QG_OP_W4A16, 16, 4096, 4096, 128) == 0
    assert qg.qg_workspace_bytes(qg.QG_OP_W4A16, 16, 12288, 4096, 128) == CTR + 192 * 4 * 4096
    # at K = 17408, N = 5120 the decode kernel runs at every M <= 16 (splits
    # of 22-23 k-tiles); small problems run the skinny kernel
    assert qg.qg_workspace_bytes(qg.QG_OP_W4A16, 8, 5120, 17408, 128) == CTR + 80 * 6 * 4096
    assert qg.qg_workspace_bytes(qg.QG_OP_W4A16, 16, 1024, 1024, 128) == 0
    # 17 <= M <= 80: the decode kernel with 16-row m-tiles (partials of 16 per
    # m-tile rows) for two m-tiles, and for more on weights of > 2^24
    # elements (any group size); otherwise the skinny kernel
    assert qg.qg_workspace_bytes(qg.QG_OP_W4A16, 17, 5120, 17408, 128) == CTR + 80 * 6 * 8192
    assert qg.qg_workspace_bytes(qg.QG_OP_W4A16, 32, 4096, 4096, 128) == CTR + 64 * 8 * 8192
    assert qg.qg_workspace_bytes(qg.QG_OP_W4A16, 48, 17408, 5120, 128) == CTR + (256 * 2 + 16 * 8) * 12288
    assert qg.qg_workspace_bytes(qg.QG_OP_W4A16, 80, 17408, 5120, 128) == CTR + (256 * 2 + 16 * 8) * 20480
    assert qg.qg_workspace_bytes(qg.QG_OP_W4A16, 64, 4096, 4096, 128) == 0
    assert qg.qg_workspace_bytes(qg.QG_OP_W4A16, 32, 4096, 4096, 64) == CTR + 64 * 8 * 8192
    assert qg.qg_workspace_bytes(qg.QG_OP_W4A16, 64, 4096, 4096, 32) == 0
    assert qg.qg_workspace_bytes(qg.QG_OP_W4A16, 81, 17408, 5120, 128) == 0     # tiled from 81
    # a K range too short to split needs none
    assert qg.qg_workspace_bytes(qg.QG_OP_W4A16, 16, 1024, 256, 128) == 0
    # the correction's group sums always come after the counter region
    assert qg.qg_workspace_bytes(qg.QG_OP_W4A16, 256, 1024, 1024, 128, 1,
                                 qg.QG_CORR_SEPARATE) == CTR + 256 * 8 * 4
    assert qg.qg_workspace_bytes(qg.QG_OP_W4A16, 16, 1024, 1024, 128, 1, qg.QG_CORR_SEPARATE) == \
        CTR + 16 * 8 * 4
    assert qg.qg_workspace_bytes(qg.QG_OP_W4A16, 16, 17408, 5120, 128, 1, qg.QG_CORR_SEPARATE) == \
        CTR + (256 * 2 + 16 * 8) * 4096 + 16 * 40 * 4


def test_workspace_bytes():
    assert qg.qg_workspace_bytes(qg.QG_OP_W4A16, 256, 1024, 1024, 128) == 0
    base = qg.qg_workspace_bytes(qg.QG_OP_W4A16, 16, 1024, 1024, 128)
    sep = qg.qg_workspace_bytes(qg.QG_OP_W4A16, 16, 1024, 1024, 128, 1, qg.QG_CORR_SEPARATE)
    assert sep >= base + 16 * 8 * 4
    assert qg.qg_workspace_bytes(qg.QG_OP_GROUP_SUM_CORRECTION, 3, 1024, 1024, -1) == 3 * 4
    assert qg.qg_workspace_bytes(qg.QG_OP_W4A8, 64, 7168, 2048, 128, 8) == 0
    with pytest.raises(qg.QGemmError):
        qg.qg_workspace_bytes(qg.QG_OP_W4A16, 16, 1024, 1000, 100)     # 100 neither divides K nor is a multiple of 128
    al = lambda n: (n + 255) // 256 * 256
    # the counter region first (never written by W4A8), then A_q and C padded
    assert qg.qg_workspace_bytes(qg.QG_OP_W4A8, 16, 1000, 1000, 128, 2) == CTR + al(16 * 1024) + 16 * 1024 * 2
    with pytest.raises(qg.QGemmError):
        qg.qg_workspace_bytes(99, 16, 1024, 1024, 128)


def test_layout_spec_is_a_permutation():
    from tests.layout_unpack import layout_is_permutation
    assert layout_is_permutation()


def test_product_path_does_not_import_the_oracle():
    pkg = os.path.join(ROOT, "int4_weight_only_uint32_amd")
    for dp, _, fs in os.walk(pkg):
        for f in fs:
            if f.endswith((".py", ".hip", ".cpp", ".h")):
                txt = open(os.path.join(dp, f)).read()
                assert "import oracle" not in txt and "from oracle" not in txt, f
                assert "qgemm_oracle" not in txt and "liboracle" not in txt, f


def test_quantize_rows_validation():
    # every case fails validation, before the device check and any launch
    L = qg.lib()
    assert L.quantize_rows_int8(None, 4, 1024, FAKE, FAKE, None) == qg.QG_ERR_INVALID_ARG
    assert L.quantize_rows_int8(FAKE, 4, 1024, None, FAKE, None) == qg.QG_ERR_INVALID_ARG
    assert L.quantize_rows_int8(FAKE, 0, 1024, FAKE, FAKE, None) == qg.QG_ERR_INVALID_ARG
    assert L.quantize_rows_int8(FAKE, 4, 0, FAKE, FAKE, None) == qg.QG_ERR_INVALID_ARG
    assert L.quantize_rows_int8(FAKE, 4, 1020, FAKE, FAKE, None) == qg.QG_ERR_UNSUPPORTED
    assert L.quantize_rows_int8(P(0x10008), 4, 1024, FAKE, FAKE, None) == qg.QG_ERR_INVALID_ARG
    assert L.quantize_rows_int8(FAKE, 4, 1024, P(0x10004), FAKE, None) == qg.QG_ERR_INVALID_ARG
    assert L.quantize_rows_int8(FAKE, 4, 1024, FAKE, P(0x10002), None) == qg.QG_ERR_INVALID_ARG
    assert b"quantize_rows_int8" in L.qg_last_error()


def test_swiglu_validation():
    # every case fails validation, before the device check and any launch
    L = qg.lib()
    ok = lambda **kw: [kw.get("A", FAKE), FAKE, FAKE, None, kw.get("H", FAKE), kw.get("M", 64), kw.get("N", 1024),
                       kw.get("K", 1024), 128, kw.get("flags", 0), kw.get("ws", FAKE), kw.get("wsb", 1 << 30), None]
    assert L.qgemm_w4a16_swiglu(*ok(A=None)) == qg.QG_ERR_INVALID_ARG
    assert L.qgemm_w4a16_swiglu(*ok(H=P(0x10008))) == qg.QG_ERR_INVALID_ARG      # H 16-byte aligned
    assert L.qgemm_w4a16_swiglu(*ok(flags=1)) == qg.QG_ERR_INVALID_ARG
    assert L.qgemm_w4a16_swiglu(*ok(N=1000)) == qg.QG_ERR_UNSUPPORTED
    # every batch is one fused launch: only the decode kernel's split-K (here
    # M = 16, K 17408 -> N 5120 per half: 3 splits; M = 17, two m-tiles over
    # the 2048-column pair, 4 splits; the 34816-column pair at K 5120, whose
    # last 32 column groups take 8 splits to balance the grid) takes a workspace
    for M in (64, 256, 4096):
        assert qg.qg_workspace_bytes(qg.QG_OP_W4A16_SWIGLU, M, 1024, 1024, 128, 1, 0) == 0
    assert qg.qg_workspace_bytes(qg.QG_OP_W4A16_SWIGLU, 17, 1024, 1024, 128, 1, 0) == CTR + 32 * 4 * 8192
    assert qg.qg_workspace_bytes(qg.QG_OP_W4A16_SWIGLU, 16, 17408, 5120, 128, 1, 0) == CTR + 32 * 8 * 4096
    need = qg.qg_workspace_bytes(qg.QG_OP_W4A16_SWIGLU, 16, 5120, 17408, 128, 1, 0)
    assert need == CTR + 160 * 3 * 4096
    split = lambda **kw: ok(M=16, N=5120, K=17408, **kw)
    assert L.qgemm_w4a16_swiglu(*split(ws=None, wsb=0)) == qg.QG_ERR_WORKSPACE
    assert L.qgemm_w4a16_swiglu(*split(wsb=need - 1)) == qg.QG_ERR_WORKSPACE


def test_padded_shape():
    assert qg.padded_shape(5120, 17408, 128) == (5120, 17408, 40)
    assert qg.padded_shape(5120, 50257, 128) == (5120, 50304, 40)
    assert qg.padded_shape(1000, 300, 128) == (1024, 384, 8)
    assert qg.padded_shape(1000, 300, -1) == (1024, 384, 1)
    assert qg.padded_shape(1000, 128, 384) == (1152, 128, 3)
    assert qg.padded_shape(130, 1, 128) == (256, 128, 2)
    with pytest.raises(qg.QGemmError):
        qg.padded_shape(1000, 300, 100)


def test_tail_workspace_sizes():
    # counters, then A padded (K tail), then the padded product (N tail)
    al = lambda n: (n + 255) // 256 * 256
    ws = lambda M, N, K, g: qg.qg_workspace_bytes(qg.QG_OP_W4A16, M, N, K, g, 1, 0)
    assert ws(300, 1000, 1024, 128) == CTR + 300 * 1024 * 2
    assert ws(300, 1024, 1000, 128) == CTR + al(300 * 1024 * 2)
    assert ws(300, 1000, 1000, 128) == CTR + al(300 * 1024 * 2) + 300 * 1024 * 2
    with pytest.raises(qg.QGemmError):
        qg.qg_workspace_bytes(qg.QG_OP_W4A16, 4, 1000, 1000, 128, 1, qg.QG_CORR_SEPARATE)


def test_binding_refuses_undersized_tensors():
    """The Python layer checks element counts before any call: a tensor too
    small for the sizes passed would be read or written out of bounds."""
    import torch
    t = lambda n, dt=torch.float16: torch.zeros(n, dtype=dt)
    with pytest.raises(ValueError, match="C holds"):
        qg.qgemm_w4a16(t(16 * 1024), t(1024 * 1024 // 8, torch.int32), t(8 * 1024), None,
                       t(16 * 1024 - 1), 16, 1024, 1024, 128)
    with pytest.raises(ValueError, match="w_packed"):
        qg.qgemm_w4a16(t(16 * 1000), t(1000 * 1000 // 8, torch.int32), t(8 * 1024), None,
                       t(16 * 1000), 16, 1000, 1000, 128)    # the padded pack is 1024 x 1024
    with pytest.raises(ValueError, match="a_scale"):
        qg.quantize_rows_int8(t(4 * 64), 4, 64, t(4 * 64, torch.int8), t(3, torch.float32))
    with pytest.raises(ValueError, match="acc_debug"):
        qg.qgemm_w4a8(t(64 * 1024, torch.int8), t(64, torch.float32), t(1024 * 1024 // 8, torch.int32),
                      t(8 * 1024), None, 1, 64, 64, 1024, 1024, 128, t(64 * 1024),
                      acc_debug=t(10, torch.int32))
    with pytest.raises(ValueError, match="H holds"):
        qg.qgemm_w4a16_swiglu(t(16 * 1024), t(1024 * 2048 // 8, torch.int32), t(8 * 2048), None,
                              t(16 * 1023), 16, 1024, 1024, 128)


def test_offset_limits_refused():
    # shapes whose 32-bit in-kernel offsets would overflow are refused on the host
    with pytest.raises(qg.QGemmError):
        qg.qg_workspace_bytes(qg.QG_OP_W4A16, 16, 1024, 1 << 22, 128)
    with pytest.raises(qg.QGemmError):
        qg.qg_workspace_bytes(qg.QG_OP_W4A16, 16, 1 << 20, 1 << 18, 128)   # 2048 groups x 2^20 columns
    assert qg.qg_workspace_bytes(qg.QG_OP_W4A16, 16, 262144, 65536, 128) >= 0


def test_noalloc_refuses_shapes_beyond_the_scratch():
    """qgemm_w4a16_noalloc refuses a call needing more scratch than the
    library's static array holds, on the host, before any device call (the
    pointers are never dereferenced), naming the sizes."""
    L = qg.lib()
    M, K, N = 8192, 1000, 2000        # a tail shape: padded A and C need ~48 MB
    need = qg.qg_workspace_bytes(qg.QG_OP_W4A16, M, N, K, 128)
    assert need > qg.QG_NOALLOC_SCRATCH_BYTES
    assert L.qgemm_w4a16_noalloc(FAKE, FAKE, FAKE, None, FAKE, M, N, K, 128, 0, None) == \
        qg.QG_ERR_WORKSPACE
    assert b"static scratch" in L.qg_last_error()
    # the other host checks come first, as for qgemm_w4a16
    assert L.qgemm_w4a16_noalloc(None, FAKE, FAKE, None, FAKE, 16, 1024, 1024, 128, 0, None) == \
        qg.QG_ERR_INVALID_ARG
    assert L.qgemm_w4a16_noalloc(FAKE, FAKE, FAKE, None, FAKE, 16, 1024, 1024, 16, 0, None) == \
        qg.QG_ERR_UNSUPPORTED
    assert L.qgemm_w4a16_noalloc(FAKE, FAKE, FAKE, None, FAKE, 16, 1024, 1024, 128, 4, None) == \
        qg.QG_ERR_INVALID_ARG
