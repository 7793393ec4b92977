"""GPU parity: the HIP library, called through its C ABI, against the CPU
oracle on the same seeded inputs.

Bars: packing is bit-exact (codes, folded scales, delta); W4A16 relative
Frobenius error <= 2e-3 plus an elementwise guard; W4A8 int32 accumulators
bit-exact and output relative error <= 1e-2 plus the guard; integer-valued
cases bit-exact."""
import numpy as np
import pytest
import torch

import int4_weight_only_uint32_amd as qg
import oracle
import synth
from tests.gpu_util import dev, elementwise_guard, host, note, pack_case, rel_fro, run_w4a16
from tests.layout_unpack import unpack_codes

pytestmark = pytest.mark.gpu

W4A16_TOL = 2e-3
W4A8_TOL = 1e-2


@pytest.fixture(scope="module", autouse=True)
def _device():
    assert torch.cuda.is_available()
    assert qg.qg_device_supported(0), "GPU visible but not gfx950"
    oracle.build(force=False)


# ------------------------------------------------------------------ pack --
@pytest.mark.parametrize("K,N,g,asym,signed", [
    (256, 384, 128, False, True),
    (512, 256, 256, False, True),
    (1024, 128, -1, False, True),
    (256, 384, 128, True, False),
    (384, 256, 128, True, True),
    (128, 128, 128, False, False),
])
def test_pack_bit_exact(K, N, g, asym, signed):
    note(f"pack K={K} N={N} g={g} asym={asym}")
    gg = K if g == -1 else g
    c = synth.w4a16_case(1, K, N, gg, asym=asym, signed_scales=signed, stream=80, case_id=K + N)
    s = c.s.copy()
    if signed:
        s[0, :4] = np.float16(-0.0)          # negative zero: not folded
    q = c.q.copy()
    q[:gg, 0] = 0                            # a fully negative-scale group with code 0 -> clamp
    s[0, 0] = np.float16(-0.5) if signed else s[0, 0]
    pw = qg.pack(dev(q), dev(s), dev(c.z) if asym else None, g, fold=True)
    torch.cuda.synchronize()
    got_q = unpack_codes(host(pw.w), K, N)
    got_s = host(pw.scale).view(np.uint16)
    if asym:
        assert np.array_equal(got_q, q)
        assert np.array_equal(got_s, s.view(np.uint16))
        _, dh = oracle.delta(s, c.z)
        assert np.array_equal(host(pw.delta).view(np.uint16), dh)
    else:
        qf, sf, n = oracle.fold_negative_scales(q, s, gg)
        assert np.array_equal(got_q, qf)
        assert np.array_equal(got_s, sf)
        if signed:
            assert n > 0
    # no fold requested: codes and scales pass through unchanged
    pw2 = qg.pack(dev(q), dev(s), None, g, fold=False)
    torch.cuda.synchronize()
    assert np.array_equal(unpack_codes(host(pw2.w), K, N), q)
    assert np.array_equal(host(pw2.scale).view(np.uint16), s.view(np.uint16))


def test_pack_structured_codes():
    K, N = 512, 256
    k = np.arange(K)[:, None]
    n = np.arange(N)[None, :]
    q = ((k + 3 * n) % 16).astype(np.uint8)
    s = np.full((K // 128, N), 0.01, np.float16)
    pw = qg.pack(dev(q), dev(s), None, 128, fold=True)
    torch.cuda.synchronize()
    assert np.array_equal(unpack_codes(host(pw.w), K, N), q)


# ----------------------------------------------------------------- W4A16 --
def _check_w4a16(case, flags=0, fold=True, tol=W4A16_TOL):
    note(f"w4a16 {case.name} M={case.M} K={case.K} N={case.N} g={case.g} "
         f"asym={case.z is not None} flags={flags}")
    got, _ = run_w4a16(case, flags=flags, fold=fold)
    ref = oracle.w4a16(case.A, case.q, case.s, case.z, case.g, fold=fold)
    err = rel_fro(got, ref)
    assert np.all(np.isfinite(got))
    assert err <= tol, err
    assert elementwise_guard(got, ref) <= 0
    return err


@pytest.mark.parametrize("M", [1, 3, 16, 17, 33, 64, 100, 130])
@pytest.mark.parametrize("K,N,g,asym", [
    (1024, 1024, 128, True),
    (2048, 256, 256, True),
    (512, 384, -1, True),
    (1024, 512, 128, False),
])
def test_w4a16_ragged_shapes(M, K, N, g, asym):
    gg = K if g == -1 else g
    c = synth.w4a16_case(M, K, N, gg, asym=asym, signed_scales=not asym, stream=81,
                         case_id=M * 7 + K + N, name="ragged")
    _check_w4a16(c)


# Shapes chosen to reach each kernel path (the dispatch rules live in
# csrc/qg_w4a16.hip): the decode kernel split 8 ways (16 k-tiles per split)
# with every group size and both weight kinds; the decode kernel unsplit (wide
# N: one split already gives enough workgroups); the 64x128 tiled
# configuration with the fused delta; the 128x256 tiles with the row split
# (two launches).
@pytest.mark.parametrize("M", [9, 16])
@pytest.mark.parametrize("g,asym", [(128, True), (256, True), (-1, True), (128, False), (256, False)])
def test_w4a16_decode_kernel_splits(M, g, asym):
    K, N = 16384, 4096
    gg = K if g == -1 else g
    c = synth.w4a16_case(M, K, N, gg, asym=asym, signed_scales=not asym, stream=85,
                         case_id=M * 31 + gg + asym, name="decode-split8")
    _check_w4a16(c)


# N = 5120: 80 workgroup column groups, split 6 ways (480 workgroups, at most
# two per CU) with uneven k-ranges (16 or 17 k-tiles at K = 12800, 17 or 18 at
# 13312)
@pytest.mark.parametrize("M,K", [(16, 12800), (9, 13312)])
@pytest.mark.parametrize("g,asym", [(128, True), (256, False), (-1, True)])
def test_w4a16_decode_kernel_six_splits(M, K, g, asym):
    N = 5120
    gg = K if g == -1 else g
    note(f"decode six splits M={M} K={K} N={N} g={gg} asym={asym}")
    c = synth.w4a16_case(M, K, N, gg, asym=asym, signed_scales=not asym, stream=93,
                         case_id=M * 7 + K + gg, name="decode-split6")
    _check_w4a16(c)


@pytest.mark.parametrize("M,asym", [(1, False), (5, True), (16, True)])
def test_w4a16_decode_kernel_unsplit(M, asym):
    c = synth.w4a16_case(M, 1024, 32768, 128, asym=asym, signed_scales=not asym, stream=86,
                         case_id=M, name="decode-unsplit")
    _check_w4a16(c)


def test_w4a16_tiled_64x128_fused_delta():
    c = synth.w4a16_case(512, 1024, 8192, 128, asym=True, stream=87, case_id=0, name="tiled-64x128")
    _check_w4a16(c)


def test_w4a16_tiled_row_split():
    # M = 2048, N = 17408: 128 x 256 tiles on the first 1920 rows, the rest in
    # a second launch; checked on sampled rows across both parts
    M, K, N, g = 2048, 512, 17408, 128
    c = synth.w4a16_case(M, K, N, g, asym=True, stream=88, case_id=0, name="row-split")
    note(f"w4a16 row split M={M} K={K} N={N}")
    got, _ = run_w4a16(c)
    rows = np.array([0, 1, 127, 128, 1000, 1919, 1920, 1921, 2000, 2047])
    ref = oracle.w4a16(c.A[rows], c.q, c.s, c.z, c.g)
    assert rel_fro(got[rows], ref) <= W4A16_TOL
    assert elementwise_guard(got[rows], ref) <= 0


@pytest.mark.parametrize("g,asym,flags", [(128, False, 0), (-1, False, 0), (128, True, 1)])
def test_w4a16_tiled_128x256_symmetric(g, asym, flags):
    # M = 1000 (ragged last tile), N = 16256 (the last workgroup's upper two
    # waves have no columns), K = 640 (an odd number of k-tiles): 8 x 64 =
    # 512 tiles of 128 x 256, one launch.  Symmetric weights, or asymmetric
    # ones with the two-kernel correction, take the hand-ordered kernel.
    M, K, N = 1000, 640, 16256
    gg = K if g == -1 else g
    c = synth.w4a16_case(M, K, N, gg, asym=asym, signed_scales=not asym, stream=89,
                         case_id=gg + 2 * asym, name="tiled-128x256-sym")
    _check_w4a16(c, flags=qg.QG_CORR_SEPARATE if flags else 0)


@pytest.mark.parametrize("K,g,asym", [(256, 128, True), (384, 128, False), (640, -1, True),
                                       (256, -1, False), (512, 256, True), (768, 256, False),
                                       (1280, 256, True), (1024, 512, True)])
def test_w4a16_mid_kernel_short_k(K, g, asym):
    # M = 200 on N = 1024 takes the 64 x 64 mid kernel, whose pipeline keeps
    # several k-tiles in flight: fewer k-tiles (2, 3, 5) than its stages, or a
    # few more (6, 10), plus a ragged last row tile; per-k-tile scaling
    # (g = 128, 512), two-k-tile groups (g = 256: one group, one full pipeline
    # round, a round plus a one-group tail, two rounds plus a one-group tail)
    # and one group over all of K
    M, N = 200, 1024
    gg = K if g == -1 else g
    c = synth.w4a16_case(M, K, N, gg, asym=asym, signed_scales=not asym, stream=90,
                         case_id=K + gg + asym, name="mid-short-k")
    _check_w4a16(c)


@pytest.mark.parametrize("g,asym", [(128, True), (256, True), (384, True), (512, False), (1536, True)])
def test_w4a16_mid2_group_forms(g, asym):
    # M = 256 on N = 8192 takes the 8-wave mid kernel (K split between two
    # k-groups inside the workgroup), 12 k-tiles; every way a k-tile finds
    # its weight group: the k-tile itself (g = 128), a shift (g = 256), a
    # division (g = 384: groups of three k-tiles, scaled per k-tile; g = 512),
    # one group over all of K (g = K)
    M, K, N = 256, 1536, 8192
    c = synth.w4a16_case(M, K, N, g, asym=asym, signed_scales=not asym, stream=90,
                         case_id=5000 + g + asym, name="mid2-group-forms")
    _check_w4a16(c)


def test_w4a16_small_asym():
    c = synth.workload("w4a16-small-asym-M16-K1024-N1024-g128")
    _check_w4a16(c)
    _check_w4a16(c, flags=qg.QG_CORR_SEPARATE)


@pytest.mark.parametrize("name", synth.names("w4a16-decode"))
def test_w4a16_decode(name):
    _check_w4a16(synth.workload(name))


@pytest.mark.parametrize("name", synth.names("w4a16-midbatch"))
def test_w4a16_midbatch(name):
    c = synth.workload(name)
    _check_w4a16(c)
    _check_w4a16(c, flags=qg.QG_CORR_SEPARATE)


def test_w4a16_prefill_every_tile():
    """Full prefill shape (M=4096, K=5120, N=17408, random-sign scales, fold on)
    in the benchmark's launch shape: 128x256 tiles over rows 0..3839 and a
    second launch of 64x128 tiles over the last 256 rows.  Against the oracle:
    (a) one row of every 16-row m-tile crossed with one column of every
    16-column n-tile (row 16i + i%16, column 16j + j%16), 256 x 1088 cells:
    128 in every 128x256 output tile, at least one in every 16x16 MFMA tile of
    every wave, at varying positions inside it; (b) the first and the last
    128 rows densely over all N (every n-tile of both launches, the full
    40 k-tiles)."""
    c = synth.workload("w4a16-prefill-M4096-K5120-N17408-g128-sym-signed")
    note(f"w4a16 prefill M={c.M} K={c.K} N={c.N}")
    got, _ = run_w4a16(c)
    assert np.all(np.isfinite(got))
    i = np.arange(c.M // 16)
    j = np.arange(c.N // 16)
    rows = 16 * i + i % 16
    cols = 16 * j + j % 16
    ref = oracle.w4a16(c.A[rows], c.q[:, cols], c.s[:, cols],
                       None, c.g, fold=True)
    g = got[np.ix_(rows, cols)]
    assert rel_fro(g, ref) <= W4A16_TOL
    assert elementwise_guard(g, ref) <= 0
    for band in (np.arange(0, 128), np.arange(c.M - 128, c.M)):
        note(f"w4a16 prefill dense rows {band[0]}..{band[-1]}")
        ref = oracle.w4a16(c.A[band], c.q, c.s, None, c.g, fold=True)
        assert rel_fro(got[band], ref) <= W4A16_TOL
        assert elementwise_guard(got[band], ref) <= 0
    # the fold matters at this distribution: the unfolded product is far off
    r = np.random.default_rng(5)
    rr, cc = r.integers(0, c.M, 500), r.integers(0, c.N, 500)
    ref_f = oracle.w4a16_cells(c.A, c.q, c.s, None, c.g, rr, cc, fold=True)
    ref_nofold = oracle.w4a16_cells(c.A, c.q, c.s, None, c.g, rr, cc, fold=False)
    assert rel_fro(ref_nofold, ref_f) > 10 * W4A16_TOL


def test_w4a16_prefill_dense_slice():
    """A 256-row slice of the prefill case checked densely."""
    c = synth.workload("w4a16-prefill-M4096-K5120-N17408-g128-sym-signed")
    sl = synth.W4A16Case(A=c.A[:256], q=c.q[:, :2048], s=c.s[:, :2048], z=None, g=c.g,
                         name="prefill-slice")
    _check_w4a16(sl)


def test_w4a16_integer_exact():
    """Integer data: every product and sum is exact, so the fp16 output must be
    bit-identical to the exact result."""
    r = np.random.default_rng(11)
    M, K, N = 37, 256, 384
    A = r.integers(-1, 2, (M, K)).astype(np.float16)
    q = r.integers(0, 16, (K, N), dtype=np.uint8)
    s = np.ones((2, N), np.float16)
    z = np.full((2, N), -8.0, np.float16)
    z[1] = -3.0
    for zz in (None, z):
        case = synth.W4A16Case(A=A, q=q, s=s, z=zz, g=128, name="int-exact")
        got, _ = run_w4a16(case)
        ref = oracle.w4a16(A, q, s, zz, 128, fold=False)
        assert np.abs(ref).max() <= 2048
        assert np.array_equal(got, ref)


def test_w4a16_degenerate_values():
    r = np.random.default_rng(12)
    M, K, N = 16, 256, 128
    A = r.standard_normal((M, K)).astype(np.float16)
    q = np.full((K, N), 8, np.uint8)
    s = r.uniform(1e-3, 2e-2, (2, N)).astype(np.float16)
    got, _ = run_w4a16(synth.W4A16Case(A=A, q=q, s=s, z=None, g=128))
    # the kernel forms s*sum(A*q) - 8s*sum(A): with q == 8 the two fp32 terms
    # cancel up to their rounding, a few ulp of |8 s a_sum| (<= 8 here)
    a_sum = np.abs(A.astype(np.float64).reshape(M, 2, 128).sum(axis=2)).max()
    assert np.max(np.abs(got)) <= 8 * 2.0 ** -23 * 8 * 0.02 * a_sum * 2
    A0 = np.zeros((M, K), np.float16)
    c = synth.w4a16_case(M, K, N, 128, asym=True, stream=82, case_id=1)
    got, _ = run_w4a16(synth.W4A16Case(A=A0, q=c.q, s=c.s, z=c.z, g=128))
    assert np.all(got == 0.0)


def test_w4a16_fold_off_matches_unfolded():
    c = synth.w4a16_case(16, 1024, 512, 128, asym=False, signed_scales=True, stream=83,
                         case_id=0)
    _check_w4a16(c, fold=False)


def test_w4a16_decode_workspace_returns_to_zero():
    # the split-K counters must be zero after every call, so one zero-filled
    # workspace serves calls of different shapes in sequence
    cases = [synth.workload("w4a16-decode-M16-K5120-N17408-g128-asym"),
             synth.workload("w4a16-decode-M16-K17408-N5120-g128-asym"),
             synth.workload("w4a16-decode-M4-K17408-N5120-g128-asym"),
             synth.workload("w4a16-small-asym-M16-K1024-N1024-g128")]
    nbytes = max(qg.qg_workspace_bytes(qg.QG_OP_W4A16, c.M, c.N, c.K, c.g) for c in cases)
    assert nbytes > 0
    ws = torch.zeros(nbytes, dtype=torch.uint8, device="cuda")
    for rep in range(2):
        for c in cases:
            note(f"w4a16 shared workspace {c.name} rep {rep}")
            pw = pack_case(c)
            C = qg.w4a16(dev(c.A), pw, workspace=ws)
            torch.cuda.synchronize()
            ncounters = c.N // 64
            assert int(torch.count_nonzero(ws[: 4 * ncounters])) == 0
            got = host(C).astype(np.float64)
            ref = oracle.w4a16(c.A, c.q, c.s, c.z, c.g)
            assert rel_fro(got, ref) <= W4A16_TOL
            assert elementwise_guard(got, ref) <= 0


def test_w4a16_deterministic():
    c = synth.workload("w4a16-decode-M16-K5120-N17408-g128-asym")
    a, _ = run_w4a16(c)
    b, _ = run_w4a16(c)
    assert np.array_equal(a, b)


# ------------------------------------------------------ correction stage --
# rows in blocks of 4 (M < 256) or 16 (M >= 256), ragged last blocks; the
# groups in LDS chunks of 64 (G = 65, 72: a second chunk) and runs of 4 (G = 9,
# 65: a remainder of one)
@pytest.mark.parametrize("M,K,N,g", [(5, 1024, 256, 128), (64, 4096, 384, 4096), (130, 512, 128, 256),
                                     (17, 1152, 128, 128), (300, 8320, 256, 128), (257, 2304, 128, 32)])
def test_group_sum_correction(M, K, N, g):
    note(f"group_sum_correction M={M} K={K} N={N} g={g}")
    c = synth.w4a16_case(M, K, N, g, asym=True, stream=84, case_id=M)
    _, dh = oracle.delta(c.s, c.z)
    r = np.random.default_rng(M)
    Cin = r.standard_normal((M, N)).astype(np.float16)
    Ct = dev(Cin)
    qg.correct(dev(c.A), dev(dh.view(np.float16)), Ct, g)
    torch.cuda.synchronize()
    got = host(Ct).astype(np.float64)
    ref = oracle.group_sum_correction(c.A, dh, Cin, g)
    # fp32 accumulation then one fp16 rounding: within 2 fp16 ulps of the exact value
    ulp = np.spacing(np.abs(ref).astype(np.float16)).astype(np.float64)
    assert np.all(np.abs(got - ref) <= 2 * np.maximum(ulp, 2.0 ** -24) + 1e-6 * np.abs(ref) + 1e-7)


# ------------------------------------------------------------------ W4A8 --
def _pack_w4a8(case, fold=True):
    """Stacked packs of the experts' weights: (W, S, D), D None if symmetric."""
    ws, ss, ds = [], [], []
    for e in range(case.E):
        z = dev(case.z[e]) if case.z is not None else None
        pw = qg.pack(dev(case.q[e]), dev(case.s[e]), z, case.g, fold=fold)
        ws.append(pw.w)
        ss.append(pw.scale)
        ds.append(pw.delta)
    D = torch.stack(ds).contiguous() if case.z is not None else None
    return torch.stack(ws).contiguous(), torch.stack(ss).contiguous(), D


def _run_w4a8(case, max_rows=None, offsets=True, fold=True, debug=True):
    E, K, N, g = case.E, case.K, case.N, case.g
    W, S, D = _pack_w4a8(case, fold)
    G = K // g
    acc = torch.full((case.M_total, G, N), -7, dtype=torch.int32, device="cuda") if debug else None
    off = dev(case.offsets) if offsets else None
    mr = max_rows if max_rows is not None else int(np.max(np.diff(case.offsets)))
    C = qg.w4a8(dev(case.Aq), dev(case.a_scale), W, S, off, E, max(mr, 1), N, g, acc_debug=acc,
                w_delta=D)
    torch.cuda.synchronize()
    return host(C).astype(np.float64), host(acc) if debug else None


def _check_w4a8(case, **kw):
    note(f"w4a8 {case.name} E={case.E} rows={np.diff(case.offsets).tolist()} K={case.K} N={case.N}"
         f" asym={case.z is not None}")
    got, acc = _run_w4a8(case, **kw)
    ref, ref_acc = oracle.w4a8(case.Aq, case.a_scale, case.q, case.s, case.offsets, case.g, fold=True,
                               z=case.z)
    assert np.array_equal(acc.astype(np.int64), ref_acc)
    err = rel_fro(got, ref)
    assert err <= W4A8_TOL, err
    assert elementwise_guard(got, ref) <= 0
    return err


def test_w4a8_moe():
    c = synth.workload("w4a8-moe-E8x64-K2048-N7168-g128")
    err = _check_w4a8(c)
    note(f"w4a8 moe rel_fro vs same-int8 oracle = {err:.3e}")


def test_w4a8_ragged_experts_and_fold():
    c = synth.w4a8_case(5, 0, 512, 256, 128, signed_scales=True, stream=85, case_id=0,
                        rows=[0, 17, 64, 3, 100])
    _check_w4a8(c)


def test_w4a8_single_expert_no_offsets():
    c = synth.w4a8_case(1, 40, 1024, 384, 256, stream=85, case_id=1)
    _check_w4a8(c, offsets=False)
    c2 = synth.w4a8_case(1, 7, 768, 128, 768, stream=85, case_id=2)
    _check_w4a8(c2, offsets=False)


# ------------------------------------------------ W4A8 with zero-points --
def test_w4a8_moe_asym():
    """The expert-batch workload with AWQ-style zero-points (the same A, codes
    and scales): exact accumulators, the output within the W4A8 tolerance of
    the oracle (which uses the zeros themselves, not the fp16 deltas), and the
    accumulator-debug and plain instantiations bit-identical."""
    c = synth.w4a8_case(8, 64, 2048, 7168, 128, stream=4, case_id=0, asym=True,
                        name="w4a8-moe-asym")
    err = _check_w4a8(c)
    note(f"w4a8 moe asym rel_fro = {err:.3e}")
    plain, _ = _run_w4a8(c, debug=False)
    dbg, _ = _run_w4a8(c, debug=True)
    assert np.array_equal(plain, dbg)


def test_w4a8_asym_ragged_group256_signed():
    """Group 256 (two k-tiles per group: the sums carry across tiles), ragged
    experts, and negative scales that an asymmetric weight never folds."""
    c = synth.w4a8_case(4, 0, 1024, 256, 256, signed_scales=True, stream=85, case_id=2,
                        rows=[33, 0, 70, 5], asym=True, name="w4a8-asym-g256")
    _check_w4a8(c)
    plain, _ = _run_w4a8(c, debug=False)
    dbg, _ = _run_w4a8(c, debug=True)
    assert np.array_equal(plain, dbg)


def test_w4a8_asym_zero_delta_equals_symmetric():
    """z = -8s makes every delta exactly 0: the asymmetric call returns the
    symmetric call's output."""
    c = synth.w4a8_case(2, 48, 512, 256, 128, stream=85, case_id=3, asym=True)
    z8 = (-8.0 * c.s.astype(np.float64)).astype(np.float16)
    assert np.array_equal(z8.astype(np.float64), -8.0 * c.s.astype(np.float64))
    c.z = z8
    got_a, acc_a = _run_w4a8(c)
    c.z = None
    got_s, acc_s = _run_w4a8(c, fold=False)
    assert np.array_equal(acc_a, acc_s)
    assert np.array_equal(got_a, got_s)


def test_w4a8_asym_integer_exact():
    """Scale 1, integer zero-points, unit token scales and sparse +-1
    activations: every output is an integer below 2048, which the fp32
    arithmetic and the fp16 store represent exactly -- the GPU must match the
    oracle bit for bit, both instantiations."""
    c = synth.w4a8_case(2, 40, 256, 128, 128, stream=85, case_id=4, asym=True)
    rng = np.random.default_rng(9)
    c.s = np.ones_like(c.s)
    c.z = rng.integers(-8, 8, size=c.z.shape).astype(np.float16)
    Aq = rng.choice(np.array([-1, 0, 0, 0, 0, 0, 0, 0, 1], np.int8), size=c.Aq.shape)
    c.Aq = Aq
    c.a_scale = np.ones_like(c.a_scale)
    ref, _ = oracle.w4a8(c.Aq, c.a_scale, c.q, c.s, c.offsets, c.g, z=c.z)
    assert np.all(np.abs(ref) < 2048) and np.array_equal(ref, np.round(ref))
    for debug in (True, False):
        got, _ = _run_w4a8(c, debug=debug)
        assert np.array_equal(got, ref)


@pytest.mark.parametrize("asym", [False, True])
def test_w4a8_large_ragged_experts(asym):
    """Experts of 700 and 300 rows: many 64-row blocks per expert, a ragged
    last block, the grid sized by the larger expert."""
    c = synth.w4a8_case(2, 0, 1024, 512, 128, signed_scales=not asym, stream=85, case_id=6,
                        rows=[700, 300], asym=asym, name="w4a8-large")
    _check_w4a8(c)


@pytest.mark.parametrize("max_rows", [1, 64, 300])
def test_w4a8_understated_row_bound(max_rows):
    """max_rows_per_expert below the true row count (700 and 300 rows): the
    bound only sizes the launch, every row of every expert is still computed
    (C starts as NaN so a row left unwritten fails)."""
    c = synth.w4a8_case(2, 0, 1024, 512, 128, stream=85, case_id=7, rows=[700, 300],
                        name="w4a8-understated")
    note(f"w4a8 understated bound max_rows={max_rows} rows=[700, 300]")
    W, S, _ = _pack_w4a8(c)
    C = torch.full((c.M_total, c.N), float("nan"), dtype=torch.float16, device="cuda")
    acc = torch.full((c.M_total, c.K // c.g, c.N), -7, dtype=torch.int32, device="cuda")
    qg.w4a8(dev(c.Aq), dev(c.a_scale), W, S, dev(c.offsets), c.E, max_rows, c.N, c.g, C=C,
            acc_debug=acc)
    torch.cuda.synchronize()
    ref, ref_acc = oracle.w4a8(c.Aq, c.a_scale, c.q, c.s, c.offsets, c.g)
    got = host(C).astype(np.float64)
    assert np.all(np.isfinite(got))
    assert np.array_equal(host(acc).astype(np.int64), ref_acc)
    assert rel_fro(got, ref) <= W4A8_TOL
    assert elementwise_guard(got, ref) <= 0


def test_w4a8_output_only_two_byte_aligned():
    """C may be any 2-byte aligned pointer: a C that is not 16-byte aligned
    (a view two bytes into a buffer) gets the same bits as an aligned one
    (the kernel writes whole 16-byte row pieces only when it can)."""
    c = synth.w4a8_case(3, 0, 1024, 384, 128, stream=85, case_id=8, rows=[70, 5, 64])
    note("w4a8 output at a 2-byte offset")
    W, S, _ = _pack_w4a8(c)
    mr = int(np.max(np.diff(c.offsets)))
    A_q, a_sc, off = dev(c.Aq), dev(c.a_scale), dev(c.offsets)
    C = qg.w4a8(A_q, a_sc, W, S, off, c.E, mr, c.N, c.g)
    buf = torch.full((c.M_total * c.N + 8,), float("nan"), dtype=torch.float16, device="cuda")
    C2 = buf[1:1 + c.M_total * c.N].view(c.M_total, c.N)
    assert C2.data_ptr() % 16 == 2
    qg.w4a8(A_q, a_sc, W, S, off, c.E, mr, c.N, c.g, C=C2)
    torch.cuda.synchronize()
    assert torch.equal(C, C2)
    assert torch.isnan(buf[0]) and torch.isnan(buf[1 + c.M_total * c.N:]).all()


# The 8-wave mid-batch kernel (K split between two groups of waves inside the
# workgroup; taken when (N/128) * ceil(M/64) >= 256): every group form, both
# weight kinds, k-tile counts that split unevenly (9: 5 + 4; 10 with groups
# of two k-tiles: 6 + 4; 5 per-column: 3 + 2), the shortest K it takes (4
# k-tiles), and ragged rows.
@pytest.mark.parametrize("M,K,N,g,asym", [
    (256, 1152, 8192, 128, True),
    (256, 1280, 8192, 256, True),
    (256, 640, 8192, -1, True),
    (200, 512, 8192, 128, False),
    (256, 1536, 8192, 256, False),
    (130, 1024, 16384, 512, True),
])
def test_w4a16_mid_kernel_ksplit(M, K, N, g, asym):
    gg = K if g == -1 else g
    c = synth.w4a16_case(M, K, N, gg, asym=asym, signed_scales=not asym, stream=96,
                         case_id=M + K + gg + asym, name="mid-ksplit")
    _check_w4a16(c)
