"""Python binding of the packed-int4 weight GEMM library (libqgemm.so, gfx950).

Argument marshalling only: each function checks that it was given device
tensors of the right dtype and of at least the sizes the call touches, passes
their pointers and the current HIP stream to the C ABI declared in
include/qgemm.h, and raises QGemmError on a non-zero status.  Every step of the
computation runs in the library's HIP kernels; there is no fallback of any
kind -- if libqgemm.so is missing, importing works but every call raises.

Names follow the C ABI: pack_int4_weights, qgemm_w4a16, qgemm_w4a16_noalloc,
qgemm_w4a16_swiglu, group_sum_correction, quantize_rows_int8, qgemm_w4a8 (plus
qg_device_supported, qg_workspace_bytes, qg_padded_shape); pack, w4a16,
w4a16_swiglu, correct, quantize_rows and w4a8 are the same calls with
torch-allocated outputs.
"""
import ctypes
import os
from dataclasses import dataclass
from typing import Optional

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libqgemm.so")
DEBUG_SYNC_LIB_PATH = os.path.join(_HERE, "libqgemm_debugsync.so")

QG_OK = 0
QG_ERR_INVALID_ARG = 1
QG_ERR_UNSUPPORTED = 2
QG_ERR_WORKSPACE = 3
QG_ERR_DEVICE = 4
QG_ERR_LAUNCH = 5

QG_PACK_FOLD_NEG_SCALES = 0x1
QG_CORR_SEPARATE = 0x1

QG_W4A16_WS_COUNTER_BYTES = 65536
QG_NOALLOC_SCRATCH_BYTES = 33554432

QG_OP_W4A16 = 1
QG_OP_W4A8 = 2
QG_OP_GROUP_SUM_CORRECTION = 3
QG_OP_PACK = 4
QG_OP_W4A16_SWIGLU = 5

EXPORTED = ("qg_device_supported", "qg_status_string", "qg_last_error", "qg_workspace_bytes",
            "pack_int4_weights", "qgemm_w4a16", "group_sum_correction", "qgemm_w4a8",
            "quantize_rows_int8", "qgemm_w4a16_swiglu", "qg_padded_shape",
            "qgemm_w4a16_noalloc")


class QGemmError(RuntimeError):
    def __init__(self, status, detail):
        super().__init__(f"qgemm status {status}: {detail}")
        self.status = status


_lib = None
_debug_lib = None


def lib():
    """Load libqgemm.so (built by __graft_entry__.build() or build.py)."""
    global _lib
    if _lib is None:
        _lib = open_library(LIB_PATH)
    return _lib


def debug_sync_lib():
    """libqgemm_debugsync.so: the same entry points built with QG_DEBUG_SYNC=1
    (every pipeline stage waits for all outstanding memory operations, every
    call waits for its kernels), for race checks against lib()."""
    global _debug_lib
    if _debug_lib is None:
        _debug_lib = open_library(DEBUG_SYNC_LIB_PATH)
    return _debug_lib


def open_library(path):
    """A built library with the argument types of every entry point set."""
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is missing: build it first "
                           "(python int4_weight_only_uint32_amd/build.py)")
    L = ctypes.CDLL(path)
    P, I, U, Z = ctypes.c_void_p, ctypes.c_int, ctypes.c_uint, ctypes.c_size_t
    L.qg_device_supported.restype = I
    L.qg_device_supported.argtypes = [I]
    L.qg_status_string.restype = ctypes.c_char_p
    L.qg_status_string.argtypes = [I]
    L.qg_last_error.restype = ctypes.c_char_p
    L.qg_last_error.argtypes = []
    L.qg_workspace_bytes.restype = Z
    L.qg_workspace_bytes.argtypes = [I, I, I, I, I, I, U]
    L.pack_int4_weights.restype = I
    L.pack_int4_weights.argtypes = [P, P, P, I, I, I, U, P, P, P, P]
    L.qgemm_w4a16.restype = I
    L.qgemm_w4a16.argtypes = [P, P, P, P, P, I, I, I, I, U, P, Z, P]
    L.qgemm_w4a16_noalloc.restype = I
    L.qgemm_w4a16_noalloc.argtypes = [P, P, P, P, P, I, I, I, I, U, P]
    L.group_sum_correction.restype = I
    L.group_sum_correction.argtypes = [P, P, P, I, I, I, I, P, Z, P]
    L.qgemm_w4a8.restype = I
    L.qgemm_w4a8.argtypes = [P, P, P, P, P, P, I, I, I, I, I, I, P, P, P, Z, U, P]
    L.qg_padded_shape.restype = I
    L.qg_padded_shape.argtypes = [I, I, I, P, P, P]
    L.qgemm_w4a16_swiglu.restype = I
    L.qgemm_w4a16_swiglu.argtypes = [P, P, P, P, P, I, I, I, I, U, P, Z, P]
    L.quantize_rows_int8.restype = I
    L.quantize_rows_int8.argtypes = [P, I, I, P, P, P]
    return L


def _check(rc):
    if rc != QG_OK:
        raise QGemmError(rc, lib().qg_last_error().decode())


def _ptr(t: Optional[torch.Tensor], dtype=None, name="tensor"):
    if t is None:
        return None
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be a device tensor")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return ctypes.c_void_p(t.data_ptr())


def _need(t: Optional[torch.Tensor], n: int, name: str):
    """Element count a call will touch: a smaller tensor would be read or
    written out of bounds on the device, so it is refused here."""
    if t is not None and isinstance(t, torch.Tensor) and t.numel() < n:
        raise ValueError(f"{name} holds {t.numel()} elements, the call needs {n}")


def _groups(K: int, group_size: int) -> int:
    g = K if group_size == -1 else group_size
    return -(-K // g) if g > 0 else 0


def _stream(t: torch.Tensor):
    return ctypes.c_void_p(torch.cuda.current_stream(t.device).cuda_stream)


def qg_device_supported(device: int = 0) -> bool:
    return bool(lib().qg_device_supported(int(device)))


def qg_workspace_bytes(op, M, N, K, group_size, num_experts=1, flags=0) -> int:
    n = lib().qg_workspace_bytes(op, M, N, K, group_size, num_experts, flags)
    if n == ctypes.c_size_t(-1).value:
        raise QGemmError(QG_ERR_INVALID_ARG, lib().qg_last_error().decode())
    return int(n)


@dataclass
class PackedWeight:
    w: torch.Tensor                 # int32 [K*N/8] (uint32 bit patterns)
    scale: torch.Tensor             # fp16 [G, N] (folded)
    delta: Optional[torch.Tensor]   # fp16 [G, N] or None (symmetric)
    K: int
    N: int
    group_size: int


def pack_int4_weights(q, scale, zero, K, N, group_size, flags, w_packed, scale_out, delta_out):
    """Same arguments as the C entry point, as device tensors (zero/delta_out may be None)."""
    Kp, Np, G = padded_shape(K, N, group_size)
    _need(q, K * N, "q")
    for t, nm in ((scale, "scale"), (zero, "zero")):
        _need(t, _groups(K, group_size) * N, nm)
    _need(w_packed, Kp * Np // 8, "w_packed")
    for t, nm in ((scale_out, "scale_out"), (delta_out, "delta_out")):
        _need(t, G * Np, nm)
    _check(lib().pack_int4_weights(_ptr(q, torch.uint8, "q"), _ptr(scale, torch.float16, "scale"),
                                   _ptr(zero, torch.float16, "zero"), K, N, group_size, flags,
                                   _ptr(w_packed, torch.int32, "w_packed"),
                                   _ptr(scale_out, torch.float16, "scale_out"),
                                   _ptr(delta_out, torch.float16, "delta_out"), _stream(q)))


def padded_shape(K: int, N: int, group_size: int):
    """(K_padded, N_padded, groups) of a pack of [K, N] codes."""
    kp, np_, gs = ctypes.c_int(0), ctypes.c_int(0), ctypes.c_int(0)
    _check(lib().qg_padded_shape(K, N, group_size, ctypes.byref(kp), ctypes.byref(np_),
                                 ctypes.byref(gs)))
    return kp.value, np_.value, gs.value


def pack(q: torch.Tensor, scale: torch.Tensor, zero: Optional[torch.Tensor] = None,
         group_size: int = 128, fold: bool = True) -> PackedWeight:
    """Allocate outputs (torch) and run pack_int4_weights (any K, N: shapes
    with tails get a padded pack, see qg_padded_shape)."""
    K, N = q.shape
    g = K if group_size == -1 else group_size
    Kp, Np, G = padded_shape(K, N, group_size)
    w = torch.empty(Kp * Np // 8, dtype=torch.int32, device=q.device)
    s_out = torch.empty((G, Np), dtype=torch.float16, device=q.device)
    d_out = torch.empty((G, Np), dtype=torch.float16, device=q.device) if zero is not None else None
    pack_int4_weights(q, scale, zero, K, N, group_size,
                      QG_PACK_FOLD_NEG_SCALES if fold else 0, w, s_out, d_out)
    return PackedWeight(w=w, scale=s_out, delta=d_out, K=K, N=N, group_size=g)


def qgemm_w4a16(A, w_packed, scale, delta, C, M, N, K, group_size, flags=0, workspace=None):
    Kp, Np, G = padded_shape(K, N, group_size)
    _need(A, M * K, "A")
    _need(C, M * N, "C")
    _need(w_packed, Kp * Np // 8, "w_packed")
    _need(scale, G * Np, "scale")
    _need(delta, G * Np, "delta")
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(lib().qgemm_w4a16(_ptr(A, torch.float16, "A"), _ptr(w_packed, torch.int32, "w_packed"),
                             _ptr(scale, torch.float16, "scale"),
                             _ptr(delta, torch.float16, "delta"), _ptr(C, torch.float16, "C"),
                             M, N, K, group_size, flags, _ptr(workspace, None, "workspace"),
                             ws_bytes, _stream(A)))


def qgemm_w4a16_noalloc(A, w_packed, scale, delta, C, M, N, K, group_size, flags=0):
    """qgemm_w4a16 with the library's static scratch instead of a workspace
    (no device allocation; calls that overlap on one GPU race)."""
    Kp, Np, G = padded_shape(K, N, group_size)
    _need(A, M * K, "A")
    _need(C, M * N, "C")
    _need(w_packed, Kp * Np // 8, "w_packed")
    _need(scale, G * Np, "scale")
    _need(delta, G * Np, "delta")
    _check(lib().qgemm_w4a16_noalloc(_ptr(A, torch.float16, "A"),
                                     _ptr(w_packed, torch.int32, "w_packed"),
                                     _ptr(scale, torch.float16, "scale"),
                                     _ptr(delta, torch.float16, "delta"),
                                     _ptr(C, torch.float16, "C"), M, N, K, group_size, flags,
                                     _stream(A)))


_workspaces = {}


def workspace_for(device: torch.device, nbytes: int) -> torch.Tensor:
    """A workspace of at least `nbytes`, cached per (device, current stream).
    Calls that share it must be ordered (one stream): each call overwrites it."""
    key = (device.index, torch.cuda.current_stream(device).cuda_stream)
    ws = _workspaces.get(key)
    if ws is None or ws.numel() < nbytes:
        ws = torch.zeros(max(nbytes, 256), dtype=torch.uint8, device=device)
        _workspaces[key] = ws
    return ws


def w4a16(A: torch.Tensor, pw: PackedWeight, C: Optional[torch.Tensor] = None, flags: int = 0,
          workspace: Optional[torch.Tensor] = None) -> torch.Tensor:
    M, K = A.shape
    if C is None:
        C = torch.empty((M, pw.N), dtype=torch.float16, device=A.device)
    if workspace is None:
        n = qg_workspace_bytes(QG_OP_W4A16, M, pw.N, K, pw.group_size, 1,
                               flags if pw.delta is not None else 0)
        if n > 0:
            workspace = workspace_for(A.device, n)
    qgemm_w4a16(A, pw.w, pw.scale, pw.delta, C, M, pw.N, K, pw.group_size, flags, workspace)
    return C


def group_sum_correction(A, delta, C, M, N, K, group_size, workspace):
    _need(A, M * K, "A")
    _need(delta, _groups(K, group_size) * N, "delta")
    _need(C, M * N, "C")
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(lib().group_sum_correction(_ptr(A, torch.float16, "A"), _ptr(delta, torch.float16, "delta"),
                                      _ptr(C, torch.float16, "C"), M, N, K, group_size,
                                      _ptr(workspace, None, "workspace"), ws_bytes, _stream(A)))


def correct(A: torch.Tensor, delta: torch.Tensor, C: torch.Tensor, group_size: int) -> torch.Tensor:
    """C += a_sum @ delta in place (allocates its fp32 workspace with torch)."""
    M, K = A.shape
    N = C.shape[1]
    n = qg_workspace_bytes(QG_OP_GROUP_SUM_CORRECTION, M, N, K, group_size)
    ws = torch.empty(max(n, 4), dtype=torch.uint8, device=A.device)
    group_sum_correction(A, delta, C, M, N, K, group_size, ws)
    return C


def qgemm_w4a8(A_q, a_scale, w_packed, w_scale, expert_offsets, num_experts, M_total,
               max_rows_per_expert, N, K, group_size, C, acc_debug=None, flags=0, w_delta=None,
               workspace=None):
    Kp, Np, G = padded_shape(K, N, group_size)
    _need(A_q, M_total * K, "A_q")
    _need(a_scale, M_total, "a_scale")
    _need(w_packed, num_experts * Kp * Np // 8, "w_packed")
    _need(w_scale, num_experts * G * Np, "w_scale")
    _need(w_delta, num_experts * G * Np, "w_delta")
    _need(expert_offsets, num_experts + 1, "expert_offsets")
    _need(C, M_total * N, "C")
    _need(acc_debug, M_total * G * N, "acc_debug")
    _check(lib().qgemm_w4a8(_ptr(A_q, torch.int8, "A_q"), _ptr(a_scale, torch.float32, "a_scale"),
                            _ptr(w_packed, torch.int32, "w_packed"),
                            _ptr(w_scale, torch.float16, "w_scale"),
                            _ptr(w_delta, torch.float16, "w_delta"),
                            _ptr(expert_offsets, torch.int32, "expert_offsets"), num_experts,
                            M_total, max_rows_per_expert, N, K, group_size,
                            _ptr(C, torch.float16, "C"), _ptr(acc_debug, torch.int32, "acc_debug"),
                            _ptr(workspace, None, "workspace"),
                            workspace.numel() * workspace.element_size() if workspace is not None else 0,
                            flags, _stream(A_q)))


def w4a8(A_q: torch.Tensor, a_scale: torch.Tensor, w_packed: torch.Tensor, w_scale: torch.Tensor,
         expert_offsets: Optional[torch.Tensor], num_experts: int, max_rows_per_expert: int,
         N: int, group_size: int, C: Optional[torch.Tensor] = None,
         acc_debug: Optional[torch.Tensor] = None,
         w_delta: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Grouped W4A8; w_delta (stacked deltas of asymmetric packs) or None."""
    M_total, K = A_q.shape
    if C is None:
        C = torch.empty((M_total, N), dtype=torch.float16, device=A_q.device)
    ws = None
    n = qg_workspace_bytes(QG_OP_W4A8, M_total, N, K, group_size, num_experts, 0)
    if n > 0:
        ws = workspace_for(A_q.device, n)
    qgemm_w4a8(A_q, a_scale, w_packed, w_scale, expert_offsets, num_experts, M_total,
               max_rows_per_expert, N, K, group_size, C, acc_debug, w_delta=w_delta, workspace=ws)
    return C


def quantize_rows_int8(A, M, K, A_q, a_scale):
    _need(A, M * K, "A")
    _need(A_q, M * K, "A_q")
    _need(a_scale, M, "a_scale")
    _check(lib().quantize_rows_int8(_ptr(A, torch.float16, "A"), M, K, _ptr(A_q, torch.int8, "A_q"),
                                    _ptr(a_scale, torch.float32, "a_scale"), _stream(A)))


def quantize_rows(A: torch.Tensor, A_q: Optional[torch.Tensor] = None,
                  a_scale: Optional[torch.Tensor] = None):
    """Per-row int8 codes and fp32 scales of fp16 activations [M,K]."""
    M, K = A.shape
    if A_q is None:
        A_q = torch.empty((M, K), dtype=torch.int8, device=A.device)
    if a_scale is None:
        a_scale = torch.empty((M,), dtype=torch.float32, device=A.device)
    if tuple(A_q.shape) != (M, K) or tuple(a_scale.shape) != (M,):
        raise ValueError(f"A_q must be [{M},{K}] and a_scale [{M}]")
    quantize_rows_int8(A, M, K, A_q, a_scale)
    return A_q, a_scale


def qgemm_w4a16_swiglu(A, w_packed, scale, delta, H, M, N, K, group_size, flags=0, workspace=None):
    G = _groups(K, group_size)
    _need(A, M * K, "A")
    _need(w_packed, K * 2 * N // 8, "w_packed")
    _need(scale, G * 2 * N, "scale")
    _need(delta, G * 2 * N, "delta")
    _need(H, M * N, "H")
    nbytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    _check(lib().qgemm_w4a16_swiglu(_ptr(A, torch.float16, "A"), _ptr(w_packed, torch.int32, "w_packed"),
                                    _ptr(scale, torch.float16, "scale"), _ptr(delta, torch.float16, "delta"),
                                    _ptr(H, torch.float16, "H"), M, N, K, group_size, flags,
                                    _ptr(workspace, None, "workspace"), nbytes, _stream(A)))


def w4a16_swiglu(A: torch.Tensor, pair: PackedWeight, H: Optional[torch.Tensor] = None,
                 workspace: Optional[torch.Tensor] = None) -> torch.Tensor:
    """silu(A . W_gate) * (A . W_up) for a gate/up pair packed as one [K, 2N]
    weight (gate columns first)."""
    M, K = A.shape
    N = pair.N // 2
    if H is None:
        H = torch.empty((M, N), dtype=torch.float16, device=A.device)
    if tuple(H.shape) != (M, N):
        raise ValueError(f"H must be [{M},{N}]")
    if workspace is None:
        n = qg_workspace_bytes(QG_OP_W4A16_SWIGLU, M, N, K, pair.group_size, 1, 0)
        if n > 0:
            workspace = workspace_for(A.device, n)
    qgemm_w4a16_swiglu(A, pair.w, pair.scale, pair.delta, H, M, N, K, pair.group_size, 0, workspace)
    return H
