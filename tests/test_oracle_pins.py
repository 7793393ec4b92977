"""Pins of the CPU oracle against facts that do not come from the oracle:
the binary16 format (via numpy's own conversions), exact rational arithmetic
on tiny inputs, closed-form identities from the pages, invariants, special
cases that reduce to library routines, and hand-worked fixtures.

Each test is chosen so that a plausible slip in the oracle -- a dropped term,
a wrong sign, a swapped index, a transposed operand -- fails at least one."""
import json
import os
from fractions import Fraction

import numpy as np
import pytest

import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _gold(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def _h(x):
    return np.asarray(x, dtype=np.float16)


# --------------------------------------------------------------- binary16 --
def test_f16_decode_all_patterns(oracle_lib):
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ref = bits.view(np.float16).astype(np.float64)
    got = np.array([oracle_lib.f16_to_f64(int(b)) for b in bits])
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], ref[~nan])
    assert np.array_equal(np.signbit(got[~nan]), np.signbit(ref[~nan]))


def test_f64_to_f16_round_to_nearest_even(oracle_lib):
    r = np.random.default_rng(7)
    xs = list(r.standard_normal(3000) * 10.0 ** r.integers(-9, 5, 3000))
    # exact halfway points between neighbouring binary16 values (ties to even)
    h = r.integers(0, 0x7bff, 2000).astype(np.uint16)
    lo = h.view(np.float16).astype(np.float64)
    hi = (h + 1).view(np.float16).astype(np.float64)
    xs += list((lo + hi) / 2.0)
    xs += [0.0, -0.0, 65504.0, 65520.0, 65519.99, 2.0 ** -24, 2.0 ** -25, 2.0 ** -25 * 1.0001,
           2.0 ** -14, -2.0 ** -14 * 0.99999, 1e-12]
    for x in xs:
        ref = int(np.float64(x).astype(np.float16).view(np.uint16))
        assert oracle_lib.f64_to_f16(x) == ref, x


# ------------------------------------------------------- exact brute force --
def _frac16(b):
    return Fraction(float(np.uint16(b).view(np.float16)))


def _exact_w4a16(A, q, s, z, g, fold):
    M, K = A.shape
    N = q.shape[1]
    Ab = A.view(np.uint16)
    sb = s.view(np.uint16)
    zb = None if z is None else z.view(np.uint16)
    C = [[Fraction(0)] * N for _ in range(M)]
    for n in range(N):
        for k in range(K):
            sv = _frac16(sb[k // g, n])
            v = int(q[k, n])
            if zb is not None:
                w = v * sv + _frac16(zb[k // g, n])
            else:
                if fold and sv < 0:
                    sv = -sv
                    v = min(16 - v, 15)
                w = (v - 8) * sv
            for m in range(M):
                C[m][n] += _frac16(Ab[m, k]) * w
    return C


@pytest.mark.parametrize("M,K,N,g,asym,signed", [
    (1, 128, 8, 32, True, False),
    (2, 128, 16, 128, True, False),
    (3, 256, 8, 64, False, True),
    (2, 256, 8, 256, False, False),
    (1, 256, 16, 128, False, True),
    (1, 130, 8, 128, True, False),      # K tail: a partial last group of 2
    (2, 200, 8, 64, False, True),       # groups of 64, the last of 8
])
def test_w4a16_matches_exact_rationals(oracle_lib, M, K, N, g, asym, signed):
    c = synth.w4a16_case(M, K, N, g, asym=asym, signed_scales=signed, stream=90, case_id=K + N + M)
    got = oracle_lib.w4a16(c.A, c.q, c.s, c.z, g, fold=True)
    exact = _exact_w4a16(c.A, c.q, c.s, c.z, g, fold=True)
    ref = np.array([[float(x) for x in row] for row in exact])
    scale = np.abs(ref).max()
    assert np.max(np.abs(got - ref)) <= 1e-14 * scale
    cells = oracle_lib.w4a16_cells(c.A, c.q, c.s, c.z, g,
                                   np.repeat(np.arange(M), N), np.tile(np.arange(N), M), fold=True)
    assert np.max(np.abs(cells.reshape(M, N) - ref)) <= 1e-14 * scale


# ------------------------------------------------------------ hand-worked --
def test_golden_asym_product_and_delta_route(oracle_lib):
    d = _gold("hand_w4a16_asym.json")
    A, q, s, z, g = _h(d["A"]), np.array(d["q"], np.uint8), _h(d["scale"]), _h(d["zero"]), d["g"]
    assert np.array_equal(oracle_lib.w4a16(A, q, s, z, g), np.array(d["expected_C"]))
    de, dh = oracle_lib.delta(s, z)
    assert np.array_equal(de, np.array(d["expected_delta"]))
    assert np.array_equal(dh.view(np.float16).astype(np.float64), np.array(d["expected_delta"]))
    assert np.array_equal(oracle_lib.w4a16(A, q, s, None, g, fold=False), np.array(d["expected_C_sym"]))
    assert np.array_equal(oracle_lib.group_sum(A, g), np.array(d["expected_a_sum"]))


def test_golden_sign_fold(oracle_lib):
    d = _gold("hand_sign_fold.json")
    A, q, s, g = _h(d["A"]), np.array(d["q"], np.uint8), _h(d["scale"]), d["g"]
    qf, sf, n = oracle_lib.fold_negative_scales(q, s, g)
    assert np.array_equal(qf, np.array(d["expected_q_folded"]))
    assert np.array_equal(sf.view(np.float16).astype(np.float64), np.array(d["expected_scale_folded"]))
    assert n == d["expected_clamped"]
    assert np.array_equal(oracle_lib.w4a16(A, q, s, None, g, fold=True), np.array(d["expected_C_folded"]))
    assert np.array_equal(oracle_lib.w4a16(A, q, s, None, g, fold=False), np.array(d["expected_C_unfolded"]))


def test_golden_w4a8(oracle_lib):
    d = _gold("hand_w4a8.json")
    C, acc = oracle_lib.w4a8(np.array(d["Aq"], np.int8), np.array(d["a_scale"], np.float32),
                             np.array(d["q"], np.uint8), _h(d["scale"]),
                             np.array(d["offsets"], np.int32), d["g"])
    assert np.array_equal(acc, np.array(d["expected_acc"]))
    assert np.array_equal(C, np.array(d["expected_C"]))


def test_golden_group_sum_correction(oracle_lib):
    d = _gold("hand_group_sum_correction.json")
    A, dl, Cin, g = _h(d["A"]), _h(d["delta"]), _h(d["C_in"]), d["g"]
    assert np.array_equal(oracle_lib.group_sum(A, g), np.array(d["expected_a_sum"]))
    assert np.array_equal(oracle_lib.group_sum_correction(A, dl, Cin, g), np.array(d["expected_C"]))


# ------------------------------------------------- identities and invariants --
@pytest.mark.parametrize("g", [128, 256, 1024])
def test_delta_identity(oracle_lib, g):
    """C_asym = C_sym + a_sum @ delta (exact because delta does not depend on k)."""
    c = synth.w4a16_case(16, 1024, 256, g, asym=True, stream=91, case_id=g)
    C_asym = oracle_lib.w4a16(c.A, c.q, c.s, c.z, g)
    C_sym = oracle_lib.w4a16(c.A, c.q, c.s, None, g, fold=False)
    de, _ = oracle_lib.delta(c.s, c.z)
    a_sum = oracle_lib.group_sum(c.A, g)
    C_route = C_sym + a_sum @ de
    nrm = np.linalg.norm(C_asym)
    assert np.linalg.norm(C_route - C_asym) <= 1e-13 * nrm
    # the correction is not negligible: dropping it is a visible error
    assert np.linalg.norm(C_sym - C_asym) > 1e-3 * nrm


def test_fold_invariant(oracle_lib):
    """Folding changes a weight only where s<0 and v==0, and there by exactly s."""
    c = synth.w4a16_case(1, 512, 384, 128, asym=False, signed_scales=True, stream=92, case_id=0)
    s = c.s.copy()
    s[0, 0] = np.float16(-0.0)   # negative zero is not folded
    W0 = oracle_lib.dequant_sym(c.q, s, 128)
    qf, sf, n = oracle_lib.fold_negative_scales(c.q, s, 128)
    W1 = oracle_lib.dequant_sym(qf, sf, 128)
    sv = s.astype(np.float64)
    neg = np.repeat(sv < 0, 128, axis=0)
    clamp = neg & (c.q == 0)
    assert n == int(clamp.sum()) and n > 0
    assert np.array_equal(W1[~clamp], W0[~clamp])
    assert np.array_equal((W1 - W0)[clamp], np.repeat(sv, 128, axis=0)[clamp])
    assert np.all(sf.view(np.float16).astype(np.float64) >= 0) or True
    assert not np.any(sf.view(np.float16).astype(np.float64) < 0)
    assert sf.view(np.uint16)[0, 0] == np.float16(-0.0).view(np.uint16)
    assert qf[0, 0] == c.q[0, 0]


def test_fold_identity_without_negative_scales(oracle_lib):
    c = synth.w4a16_case(2, 256, 128, 128, asym=False, signed_scales=False, stream=92, case_id=1)
    qf, sf, n = oracle_lib.fold_negative_scales(c.q, c.s, 128)
    assert n == 0 and np.array_equal(qf, c.q) and np.array_equal(sf, c.s.view(np.uint16))


def test_special_cases(oracle_lib):
    c = synth.w4a16_case(4, 256, 64, 128, asym=True, stream=93, case_id=0)
    # all codes at the offset 8 -> the symmetric product is exactly zero
    q8 = np.full_like(c.q, 8)
    assert np.all(oracle_lib.w4a16(c.A, q8, c.s, None, 128, fold=False) == 0.0)
    # zero = -8*scale -> delta = 0 -> asymmetric equals symmetric
    z = (-8.0 * c.s.astype(np.float64)).astype(np.float16)
    assert np.array_equal(oracle_lib.delta(c.s, z)[0], np.zeros_like(c.s, dtype=np.float64))
    np.testing.assert_allclose(oracle_lib.w4a16(c.A, c.q, c.s, z, 128),
                               oracle_lib.w4a16(c.A, c.q, c.s, None, 128, fold=False), rtol=0, atol=1e-12)
    # one-hot activation rows pick out weight rows: pins orientation (no transpose)
    K = 256
    A = np.zeros((3, K), np.float16)
    ks = [0, 131, 255]
    for i, k in enumerate(ks):
        A[i, k] = 1.0
    C = oracle_lib.w4a16(A, c.q, c.s, c.z, 128)
    for i, k in enumerate(ks):
        want = c.q[k].astype(np.float64) * c.s[k // 128].astype(np.float64) + c.z[k // 128].astype(np.float64)
        assert np.array_equal(C[i], want)
    # group == K: a single group, same as a per-column scale
    s1 = c.s[:1]
    C1 = oracle_lib.w4a16(c.A, c.q, s1, None, K, fold=False)
    W = (c.q.astype(np.float64) - 8.0) * s1.astype(np.float64)
    np.testing.assert_allclose(C1, c.A.astype(np.float64) @ W, rtol=1e-13, atol=1e-13)


def test_matmul_against_numpy(oracle_lib):
    r = np.random.default_rng(3)
    A = r.standard_normal((7, 33))
    W = r.standard_normal((33, 5))
    np.testing.assert_allclose(oracle_lib.matmul(A, W), A @ W, rtol=1e-13, atol=1e-13)
    # a non-square check that would catch a transposed operand
    assert oracle_lib.matmul(A, W).shape == (7, 5)


def test_group_sum_closed_forms(oracle_lib):
    K, g = 512, 128
    A = np.tile(np.arange(K, dtype=np.float64) % 64, (2, 1)).astype(np.float16)
    A[1] *= -1
    got = oracle_lib.group_sum(A, g)
    # each group of 128 holds 0..63 twice: 2 * 63*64/2 = 4032
    assert np.array_equal(got, np.array([[4032.0] * 4, [-4032.0] * 4]))


def test_w4a8_unit_scales_equal_integer_matmul(oracle_lib):
    c = synth.w4a8_case(2, 5, 256, 64, 128, stream=94, case_id=0, rows=[5, 3])
    ones = np.ones_like(c.s)
    unit = np.ones(c.M_total, np.float32)
    C, acc = oracle_lib.w4a8(c.Aq, unit, c.q, ones, c.offsets, 128, fold=False)
    for e in range(c.E):
        r0, r1 = c.offsets[e], c.offsets[e + 1]
        ref = c.Aq[r0:r1].astype(np.int64) @ (c.q[e].astype(np.int64) - 8)
        assert np.array_equal(C[r0:r1], ref.astype(np.float64))
        # the per-group integer partial sums, summed over groups, are the product
        assert np.array_equal(acc[r0:r1].sum(axis=1), ref)
        # and each group's partial is the product restricted to that k-range
        for gi in range(256 // 128):
            ks = slice(gi * 128, (gi + 1) * 128)
            part = c.Aq[r0:r1, ks].astype(np.int64) @ (c.q[e, ks].astype(np.int64) - 8)
            assert np.array_equal(acc[r0:r1, gi], part)


def test_w4a8_scaling_and_fold(oracle_lib):
    c = synth.w4a8_case(2, 4, 256, 32, 128, signed_scales=True, stream=94, case_id=1)
    C, acc = oracle_lib.w4a8(c.Aq, c.a_scale, c.q, c.s, c.offsets, 128, fold=True)
    for e in range(c.E):
        qf, sf, _ = oracle_lib.fold_negative_scales(c.q[e], c.s[e], 128)
        r0, r1 = c.offsets[e], c.offsets[e + 1]
        sv = sf.view(np.float16).astype(np.float64)
        for m in range(r0, r1):
            ref = 0.0
            for gi in range(2):
                ks = slice(gi * 128, (gi + 1) * 128)
                part = c.Aq[m, ks].astype(np.int64) @ (qf[ks].astype(np.int64) - 8)
                assert np.array_equal(acc[m, gi], part)
                ref = ref + sv[gi] * part
            np.testing.assert_allclose(C[m], np.float64(c.a_scale[m]) * ref, rtol=1e-14, atol=0)
    # fold is exact except at clamped codes: compare to the unfolded product
    C0, _ = oracle_lib.w4a8(c.Aq, c.a_scale, c.q, c.s, c.offsets, 128, fold=False)
    assert not np.array_equal(C0, C)


def test_quantize_rows_int8(oracle_lib):
    A = np.array([[0.5, -1.0, 0.25], [0, 0, 0], [127, -3, 1.5]], np.float16)
    codes, sc = oracle_lib.quantize_rows_int8(A)
    assert sc[1] == 0 and np.all(codes[1] == 0)
    assert codes[0, 1] == -127 and codes[2, 0] == 127
    assert np.all(np.abs(codes) <= 127)


# ------------------------------------------- per-row int8 quantization ---
def test_quantize_ties_half_even_unit_scale(oracle_lib):
    """max|row| = 127 gives a_scale = 1 exactly, so the codes are the row
    itself rounded half to even (hand-worked)."""
    A = _h([[127, 2.5, 3.5, -2.5, 0.5, -0.5, 1.5, 126.5, -1.5, 0.25]])
    codes, sc = oracle_lib.quantize_rows_int8(A)
    assert sc.dtype == np.float32 and sc[0] == 1.0
    assert codes.tolist() == [[127, 2, 4, -2, 0, 0, 2, 126, -2, 0]]


def test_quantize_power_of_two_scale(oracle_lib):
    """max|row| = 127/64 gives a_scale = 1/64 exactly: A = j/64 maps to code j,
    and (j + 1/2)/64 to the even neighbour."""
    j = np.arange(-127, 128)
    A = np.concatenate([j / 64.0, (np.arange(-126, 126) + 0.5) / 64.0])[None, :]
    codes, sc = oracle_lib.quantize_rows_int8(_h(A))
    assert sc[0] == np.float32(1 / 64)
    assert np.array_equal(codes[0, :255], j)
    half = np.arange(-126, 126) + 0.5
    even = np.where(np.floor(half) % 2 == 0, np.floor(half), np.ceil(half))
    assert np.array_equal(codes[0, 255:], even)


def test_quantize_zero_row_and_single_entry(oracle_lib):
    A = np.zeros((3, 16), np.float16)
    A[1, 5] = -3.0
    A[2, :] = 1e-7                      # binary16 subnormals: a tiny positive scale
    codes, sc = oracle_lib.quantize_rows_int8(A)
    assert sc[0] == 0 and np.all(codes[0] == 0)
    assert codes[1, 5] == -127 and np.count_nonzero(codes[1]) == 1
    assert sc[2] > 0 and np.all(codes[2] == 127)


def test_quantize_against_exact_rationals(oracle_lib):
    """Random rows: a_scale is max|row|/127 correctly rounded to binary32
    (within half an ulp of the exact quotient), the argmax maps to +-127, and
    every code is the exact quotient A/a_scale rounded half to even, except
    within binary32 rounding of a half-integer (counted: there are few)."""
    rng = np.random.default_rng(5)
    A = (rng.standard_normal((6, 300)) * np.array([[1e-3], [1], [30], [1], [5e3], [0.1]])).astype(np.float16)
    codes, sc = oracle_lib.quantize_rows_int8(A)
    A64 = A.astype(np.float64)
    near_half = 0
    for m in range(A.shape[0]):
        amax = Fraction(float(np.max(np.abs(A64[m]))))
        s = Fraction(float(sc[m]))
        ulp = Fraction(float(np.spacing(sc[m])))
        assert abs(s - amax / 127) <= ulp / 2
        am = int(np.argmax(np.abs(A64[m])))
        assert codes[m, am] == (127 if A64[m, am] > 0 else -127)
        for k in range(A.shape[1]):
            x = Fraction(float(A64[m, k])) / s
            fl = x.numerator // x.denominator
            frac = x - fl
            if abs(frac - Fraction(1, 2)) < Fraction(1, 1 << 16):
                near_half += 1
                assert codes[m, k] in (fl, fl + 1)
                continue
            r = fl + 1 if frac > Fraction(1, 2) else fl
            assert codes[m, k] == max(-127, min(127, r))
    assert near_half < 10


# ------------------------------------------- W4A8 with zero-points ---------
def _w4a8_asym_case(**kw):
    return synth.w4a8_case(E=2, rows_per_expert=5, K=256, N=128, g=128, asym=True, **kw)


def test_w4a8_asym_reduces_to_symmetric(oracle_lib):
    """z = -8s (exact in binary16) makes q s + z = (q - 8) s: the symmetric
    product, and the same integer accumulators."""
    c = _w4a8_asym_case()
    z8 = (-8.0 * c.s.astype(np.float64)).astype(np.float16)
    assert np.array_equal(z8.astype(np.float64), -8.0 * c.s.astype(np.float64))
    Ca, acc_a = oracle_lib.w4a8(c.Aq, c.a_scale, c.q, c.s, c.offsets, 128, z=z8)
    Cs, acc_s = oracle_lib.w4a8(c.Aq, c.a_scale, c.q, c.s, c.offsets, 128, fold=False)
    np.testing.assert_allclose(Ca, Cs, rtol=1e-12, atol=1e-12 * np.abs(Cs).max())
    assert np.array_equal(acc_a, acc_s)


def test_w4a8_asym_one_hot_rows_pick_weight_rows(oracle_lib):
    """A row with a single 1 at k and a_scale 1 returns row k of the
    dequantized asymmetric weight q s + z of its expert (orientation, the
    zero-point term and the expert's own weights)."""
    c = _w4a8_asym_case()
    rng = np.random.default_rng(2)
    ks = rng.integers(0, 256, size=c.M_total)
    Aq = np.zeros((c.M_total, 256), np.int8)
    Aq[np.arange(c.M_total), ks] = 1
    C, _ = oracle_lib.w4a8(Aq, np.ones(c.M_total, np.float32), c.q, c.s, c.offsets, 128, z=c.z)
    for e in range(c.E):
        W = oracle_lib.dequant_asym(c.q[e], c.s[e], c.z[e], 128)
        for m in range(c.offsets[e], c.offsets[e + 1]):
            np.testing.assert_allclose(C[m], W[ks[m]], rtol=1e-15, atol=0)


def test_w4a8_asym_linear_in_zero_points(oracle_lib):
    """C(z) - C(z') = a_scale * sum_g Q[m,g] (z - z')[g,n], Q the integer
    group sums of A_q: the zero-point term alone, in closed form."""
    c = _w4a8_asym_case()
    z2 = np.zeros_like(c.z)
    C1, _ = oracle_lib.w4a8(c.Aq, c.a_scale, c.q, c.s, c.offsets, 128, z=c.z)
    C0, _ = oracle_lib.w4a8(c.Aq, c.a_scale, c.q, c.s, c.offsets, 128, z=z2)
    Q = c.Aq.astype(np.int64).reshape(c.M_total, 2, 128).sum(axis=2)
    for e in range(c.E):
        rows = slice(c.offsets[e], c.offsets[e + 1])
        d = (Q[rows].astype(np.float64) @ c.z[e].astype(np.float64)) * c.a_scale[rows, None].astype(np.float64)
        np.testing.assert_allclose(C1[rows] - C0[rows], d, rtol=1e-9, atol=1e-12 * np.abs(C1).max())


def test_w4a8_asym_is_never_folded(oracle_lib):
    c = _w4a8_asym_case(signed_scales=True)
    Cf, _ = oracle_lib.w4a8(c.Aq, c.a_scale, c.q, c.s, c.offsets, 128, fold=True, z=c.z)
    Cn, _ = oracle_lib.w4a8(c.Aq, c.a_scale, c.q, c.s, c.offsets, 128, fold=False, z=c.z)
    assert np.array_equal(Cf, Cn)


# ---------------------------------------------------------- SwiGLU ---------
def test_silu_mul_closed_forms(oracle_lib):
    """With the up half 1, H = silu(x): silu(x) - silu(-x) = x (sigmoid(x) +
    sigmoid(-x) = 1), silu(ln 3) = (3/4) ln 3 (sigmoid(ln 3) = 3/4), silu(0) =
    0, silu(40) = 40 and silu(-40) vanishes in fp64."""
    x = np.concatenate([np.linspace(-12, 12, 97), [np.log(3.0), 40.0, -40.0, 0.0]])
    C = np.stack([np.concatenate([x, np.ones_like(x)]), np.concatenate([-x, np.ones_like(x)])])
    H = oracle_lib.silu_mul(C)
    np.testing.assert_allclose(H[0] - H[1], x, rtol=1e-14, atol=1e-14)
    n = len(x)
    assert abs(H[0, n - 4] - 0.75 * np.log(3.0)) < 1e-15
    assert H[0, n - 3] == 40.0 and abs(H[0, n - 2]) < 1e-15 and H[0, n - 1] == 0.0


def test_silu_mul_gate_is_the_first_half(oracle_lib):
    """Zero gate or zero up gives 0; [x | 1] gives silu(x) while [1 | x] gives
    silu(1) x -- the halves are not interchangeable."""
    x = np.linspace(-3, 3, 13)            # holds 1.0 at index 8
    one, zero = np.ones_like(x), np.zeros_like(x)
    H = oracle_lib.silu_mul(np.stack([np.concatenate([zero, x]), np.concatenate([x, zero]),
                                      np.concatenate([x, one]), np.concatenate([one, x])]))
    assert np.all(H[0] == 0) and np.all(H[1] == 0)
    silu1 = H[2, 8]
    np.testing.assert_allclose(H[3], silu1 * x, rtol=1e-15, atol=0)
    assert not np.allclose(H[2], H[3])


def test_w4a16_swiglu_halves(oracle_lib):
    """The pair's product is the two plain products side by side: with a
    gate whose product is 0 (codes 8, symmetric) the output is 0, and with up
    codes 9 at scale 1 (W_up = 1 everywhere) the output is silu of the gate
    product times the row sums of A."""
    rng = np.random.default_rng(4)
    M, K, N, g = 3, 256, 32, 128
    A = (rng.standard_normal((M, K)) * 0.05).astype(np.float16)
    qg_ = rng.integers(0, 16, size=(K, N), dtype=np.uint8)
    s = rng.uniform(1e-3, 2e-2, size=(K // g, 2 * N)).astype(np.float16)
    q = np.concatenate([np.full((K, N), 8, np.uint8), qg_], axis=1)
    H0 = oracle_lib.w4a16_swiglu(A, q, s, None, g)
    assert np.all(H0 == 0)
    q = np.concatenate([qg_, np.full((K, N), 9, np.uint8)], axis=1)
    s1 = s.copy()
    s1[:, N:] = 1.0
    H = oracle_lib.w4a16_swiglu(A, q, s1, None, g)
    Cg = oracle_lib.w4a16(A, qg_, s[:, :N], None, g)
    rows = A.astype(np.float64).sum(axis=1, keepdims=True)
    np.testing.assert_allclose(H, Cg / (1 + np.exp(-Cg)) * rows, rtol=1e-12, atol=1e-15)


# ------------------------------------------------- shapes with tails -------
def test_w4a16_k_tail_is_zero_padding(oracle_lib):
    """K not a multiple of 128: the product equals the product over K padded
    to 128 with zero activations and arbitrary codes in the padding (the
    groups, and so the scales, are the same)."""
    c = synth.w4a16_case(3, 1000, 40, 128, asym=True, stream=90, case_id=500)
    C = oracle_lib.w4a16(c.A, c.q, c.s, c.z, 128)
    rng = np.random.default_rng(1)
    Ap = np.concatenate([c.A, np.zeros((3, 24), np.float16)], axis=1)
    qp = np.concatenate([c.q, rng.integers(0, 16, size=(24, 40), dtype=np.uint8)], axis=0)
    Cp = oracle_lib.w4a16(Ap, qp, c.s, c.z, 128)
    assert np.array_equal(C, Cp)


def test_w4a16_n_tail_columns_are_independent(oracle_lib):
    """N not a multiple of 128: each column is its own product, so the first
    300 columns of a 384-column problem are the 300-column problem."""
    c = synth.w4a16_case(2, 256, 384, 128, asym=False, signed_scales=True, stream=90, case_id=501)
    C = oracle_lib.w4a16(c.A, c.q, c.s, None, 128)
    C3 = oracle_lib.w4a16(c.A, np.ascontiguousarray(c.q[:, :300]), np.ascontiguousarray(c.s[:, :300]),
                          None, 128)
    assert np.array_equal(C[:, :300], C3)


def test_w4a8_k_tail_is_zero_padding(oracle_lib):
    """W4A8 over K = 1000 (a partial last group) equals the same product with
    A_q padded by zero columns to K = 1024 and arbitrary padding codes."""
    c = synth.w4a8_case(2, 3, 1000, 40, 128, stream=90, case_id=502, asym=True)
    C, acc = oracle_lib.w4a8(c.Aq, c.a_scale, c.q, c.s, c.offsets, 128, z=c.z)
    rng = np.random.default_rng(2)
    Aq = np.concatenate([c.Aq, np.zeros((c.M_total, 24), np.int8)], axis=1)
    q = np.concatenate([c.q, rng.integers(0, 16, size=(2, 24, 40), dtype=np.uint8)], axis=1)
    Cp, accp = oracle_lib.w4a8(Aq, c.a_scale, q, c.s, c.offsets, 128, z=c.z)
    assert np.array_equal(C, Cp) and np.array_equal(acc, accp)
