"""CPU oracle for the packed-int4 weight GEMM -- test infrastructure only.

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  The product path (the HIP library and its
Python binding) never imports, links or runs anything here.

The arithmetic lives in ``qgemm_oracle.c`` (plain C, fp64, naive loops); this
module only builds it with gcc and marshals numpy arrays through ctypes.
"""
import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "qgemm_oracle.c")
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
_lib = None


def build(force=True):
    """Compile the oracle with gcc (OpenMP, fp64).  Always recompiles when force."""
    if force or not os.path.exists(_LIB_PATH):
        tmp = _LIB_PATH + ".tmp"
        subprocess.check_call(["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-std=c99",
                               "-D_DEFAULT_SOURCE", _SRC, "-o", tmp, "-lm"])
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            build(force=True)
        lib = ctypes.CDLL(_LIB_PATH)
        P = ctypes.c_void_p
        I = ctypes.c_int
        lib.oracle_f16_to_f64.restype = ctypes.c_double
        lib.oracle_f16_to_f64.argtypes = [ctypes.c_uint16]
        lib.oracle_f64_to_f16.restype = ctypes.c_uint16
        lib.oracle_f64_to_f16.argtypes = [ctypes.c_double]
        lib.oracle_fold_negative_scales.restype = ctypes.c_long
        lib.oracle_fold_negative_scales.argtypes = [P, P, I, I, I]
        lib.oracle_dequant_sym.restype = None
        lib.oracle_dequant_sym.argtypes = [P, P, I, I, I, P]
        lib.oracle_dequant_asym.restype = None
        lib.oracle_dequant_asym.argtypes = [P, P, P, I, I, I, P]
        lib.oracle_delta.restype = None
        lib.oracle_delta.argtypes = [P, P, I, I, P, P]
        lib.oracle_matmul.restype = None
        lib.oracle_matmul.argtypes = [P, P, I, I, I, P]
        lib.oracle_w4a16.restype = I
        lib.oracle_w4a16.argtypes = [P, P, P, P, I, I, I, I, I, P]
        lib.oracle_w4a16_cells.restype = I
        lib.oracle_w4a16_cells.argtypes = [P, P, P, P, I, I, I, I, I, I, P, P, P]
        lib.oracle_group_sum.restype = None
        lib.oracle_group_sum.argtypes = [P, I, I, I, P]
        lib.oracle_group_sum_correction.restype = I
        lib.oracle_group_sum_correction.argtypes = [P, P, P, I, I, I, I, P]
        lib.oracle_w4a8.restype = I
        lib.oracle_w4a8.argtypes = [P, P, P, P, P, P, I, I, I, I, I, I, P, P]
        lib.oracle_quantize_rows_int8.restype = None
        lib.oracle_silu_mul.restype = None
        lib.oracle_silu_mul.argtypes = [P, I, I, P]
        lib.oracle_quantize_rows_int8.argtypes = [P, I, I, P, P]
        _lib = lib
    return _lib


def _c(a, dtype):
    a = np.ascontiguousarray(a, dtype=dtype)
    return a, a.ctypes.data_as(ctypes.c_void_p)


def _bits16(a):
    """Accept float16 arrays or their uint16 bit patterns."""
    a = np.asarray(a)
    if a.dtype == np.float16:
        a = a.view(np.uint16)
    return np.ascontiguousarray(a, dtype=np.uint16)


def f16_to_f64(bits):
    return _load().oracle_f16_to_f64(int(bits))


def f64_to_f16(x):
    return _load().oracle_f64_to_f16(float(x))


def fold_negative_scales(q, s, g):
    """Return (q_folded, s_folded_bits, n_clamped) -- copies; inputs untouched."""
    q2, pq = _c(np.array(q, dtype=np.uint8, copy=True), np.uint8)
    s2 = _bits16(s).copy()
    s2, ps = _c(s2, np.uint16)
    K, N = q2.shape
    n = _load().oracle_fold_negative_scales(pq, ps, K, N, int(g))
    return q2, s2, int(n)


def dequant_sym(q, s, g):
    q, pq = _c(q, np.uint8)
    s, ps = _c(_bits16(s), np.uint16)
    K, N = q.shape
    W = np.empty((K, N), dtype=np.float64)
    _load().oracle_dequant_sym(pq, ps, K, N, int(g), W.ctypes.data_as(ctypes.c_void_p))
    return W


def dequant_asym(q, s, z, g):
    q, pq = _c(q, np.uint8)
    s, ps = _c(_bits16(s), np.uint16)
    z, pz = _c(_bits16(z), np.uint16)
    K, N = q.shape
    W = np.empty((K, N), dtype=np.float64)
    _load().oracle_dequant_asym(pq, ps, pz, K, N, int(g), W.ctypes.data_as(ctypes.c_void_p))
    return W


def delta(s, z):
    """(delta_exact fp64 [G,N], delta_f16 bits [G,N])."""
    s, ps = _c(_bits16(s), np.uint16)
    z, pz = _c(_bits16(z), np.uint16)
    G, N = s.shape
    de = np.empty((G, N), dtype=np.float64)
    dh = np.empty((G, N), dtype=np.uint16)
    _load().oracle_delta(ps, pz, G, N, de.ctypes.data_as(ctypes.c_void_p),
                         dh.ctypes.data_as(ctypes.c_void_p))
    return de, dh


def matmul(A, W):
    A, pa = _c(A, np.float64)
    W, pw = _c(W, np.float64)
    M, K = A.shape
    K2, N = W.shape
    assert K == K2
    C = np.empty((M, N), dtype=np.float64)
    _load().oracle_matmul(pa, pw, M, N, K, C.ctypes.data_as(ctypes.c_void_p))
    return C


def w4a16(A, q, s, z, g, fold=True):
    """C = A . W in fp64 (z None -> symmetric, folded when fold)."""
    A, pa = _c(_bits16(A), np.uint16)
    q, pq = _c(q, np.uint8)
    s, ps = _c(_bits16(s), np.uint16)
    M, K = A.shape
    N = q.shape[1]
    if z is None:
        pz = None
    else:
        z, pz = _c(_bits16(z), np.uint16)
    C = np.empty((M, N), dtype=np.float64)
    rc = _load().oracle_w4a16(pa, pq, ps, pz, M, N, K, int(g), int(bool(fold)),
                              C.ctypes.data_as(ctypes.c_void_p))
    if rc != 0:
        raise MemoryError("oracle_w4a16 allocation failed")
    return C


def w4a16_cells(A, q, s, z, g, rows, cols, fold=True):
    A, pa = _c(_bits16(A), np.uint16)
    q, pq = _c(q, np.uint8)
    s, ps = _c(_bits16(s), np.uint16)
    M, K = A.shape
    N = q.shape[1]
    pz = None
    if z is not None:
        z, pz = _c(_bits16(z), np.uint16)
    rows, pr = _c(rows, np.int32)
    cols, pc = _c(cols, np.int32)
    out = np.empty(rows.shape[0], dtype=np.float64)
    _load().oracle_w4a16_cells(pa, pq, ps, pz, M, N, K, int(g), int(bool(fold)),
                               int(rows.shape[0]), pr, pc, out.ctypes.data_as(ctypes.c_void_p))
    return out


def group_sum(A, g):
    A, pa = _c(_bits16(A), np.uint16)
    M, K = A.shape
    out = np.empty((M, -(-K // g)), dtype=np.float64)
    _load().oracle_group_sum(pa, M, K, int(g), out.ctypes.data_as(ctypes.c_void_p))
    return out


def group_sum_correction(A, delta_bits, C_in, g):
    A, pa = _c(_bits16(A), np.uint16)
    d, pd = _c(_bits16(delta_bits), np.uint16)
    c, pc = _c(_bits16(C_in), np.uint16)
    M, K = A.shape
    N = d.shape[1]
    out = np.empty((M, N), dtype=np.float64)
    rc = _load().oracle_group_sum_correction(pa, pd, pc, M, N, K, int(g),
                                             out.ctypes.data_as(ctypes.c_void_p))
    if rc != 0:
        raise MemoryError("oracle_group_sum_correction allocation failed")
    return out


def w4a8(Aq, a_scale, q, s, offsets, g, fold=True, want_acc=True, z=None):
    """Grouped W4A8.  q: [E,K,N] u8, s: [E,G,N] fp16 bits, offsets: [E+1];
    z: [E,G,N] fp16 zeros for asymmetric weights (never folded), or None.
    Returns (C fp64 [M_total,N], acc int64 [M_total,G,N] or None)."""
    Aq, pa = _c(Aq, np.int8)
    a_scale, psc = _c(a_scale, np.float32)
    q, pq = _c(q, np.uint8)
    s, ps = _c(_bits16(s), np.uint16)
    pz = None
    if z is not None:
        z, pz = _c(_bits16(z), np.uint16)
    offsets, po = _c(offsets, np.int32)
    E, K, N = q.shape
    M_total = Aq.shape[0]
    G = -(-K // g)
    C = np.empty((M_total, N), dtype=np.float64)
    acc = np.zeros((M_total, G, N), dtype=np.int64) if want_acc else None
    pacc = acc.ctypes.data_as(ctypes.c_void_p) if want_acc else None
    rc = _load().oracle_w4a8(pa, psc, pq, ps, pz, po, E, M_total, N, K, int(g), int(bool(fold)),
                             pacc, C.ctypes.data_as(ctypes.c_void_p))
    if rc != 0:
        raise MemoryError("oracle_w4a8 allocation failed")
    return C, acc


def quantize_rows_int8(A):
    """Per-row int8 codes of fp16 activations [M,K] (float16 or uint16 bits).
    Returns (codes int8 [M,K], a_scale float32 [M])."""
    A, pa = _c(_bits16(A), np.uint16)
    M, K = A.shape
    codes = np.empty((M, K), dtype=np.int8)
    sc = np.empty(M, dtype=np.float32)
    _load().oracle_quantize_rows_int8(pa, M, K, codes.ctypes.data_as(ctypes.c_void_p),
                                      sc.ctypes.data_as(ctypes.c_void_p))
    return codes, sc


def silu_mul(C):
    """H = silu(C[:, :N]) * C[:, N:] for C fp64 [M, 2N]."""
    C, pc = _c(C, np.float64)
    M, N2 = C.shape
    H = np.empty((M, N2 // 2), dtype=np.float64)
    _load().oracle_silu_mul(pc, M, N2 // 2, H.ctypes.data_as(ctypes.c_void_p))
    return H


def w4a16_swiglu(A, q, s, z, g, fold=True):
    """SwiGLU of a gate/up pair held as one weight [K, 2N] (gate columns
    first): silu(A . W_gate) * (A . W_up), fp64 [M, N]."""
    return silu_mul(w4a16(A, q, s, z, g, fold=fold))
