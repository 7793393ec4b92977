"""Achievable-peak probes (libqgprobe.so, declared in include/qgprobe.h) used
by the benchmark to price the GEMM kernels against what this GPU sustains in
the same run, beside the published peaks: an fp16 MFMA loop and an HBM
streaming read.  Not part of the GEMM library."""
import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(os.path.dirname(_HERE), "libqgprobe.so")
EXPORTED = ("qgprobe_hbm_read", "qgprobe_mfma_f16", "qgprobe_mfma_flops", "qgprobe_mfma_i8")

_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it first "
                               "(python int4_weight_only_uint32_amd/build.py)")
        L = ctypes.CDLL(LIB_PATH)
        P, I, Z = ctypes.c_void_p, ctypes.c_int, ctypes.c_size_t
        L.qgprobe_mfma_f16.restype = I
        L.qgprobe_mfma_f16.argtypes = [I, P, I, I, P]
        L.qgprobe_mfma_i8.restype = I
        L.qgprobe_mfma_i8.argtypes = [P, I, I, P]
        L.qgprobe_mfma_flops.restype = ctypes.c_longlong
        L.qgprobe_mfma_flops.argtypes = [I, I, I]
        L.qgprobe_hbm_read.restype = I
        L.qgprobe_hbm_read.argtypes = [P, Z, P, I, I, P]
        _lib = L
    return _lib


def _events_ms(launch, reps):
    """Average ms of `launch()` over `reps` back-to-back launches, HIP events
    on torch's current stream (the stream the probes are launched on)."""
    st = torch.cuda.current_stream()
    for _ in range(2):
        launch()
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record(st)
    for _ in range(reps):
        launch()
    e1.record(st)
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / reps


def mfma_f16_tflops(shape, workgroups, iters, reps=10):
    """Sustained dense fp16 MFMA TFLOP/s of the loop probe."""
    L = lib()
    out = torch.empty(workgroups * 256, dtype=torch.float32, device="cuda")
    st = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)

    def launch():
        rc = L.qgprobe_mfma_f16(shape, ctypes.c_void_p(out.data_ptr()), workgroups, iters, st)
        if rc:
            raise RuntimeError(f"qgprobe_mfma_f16 status {rc}")
    ms = _events_ms(launch, reps)
    return L.qgprobe_mfma_flops(shape, workgroups, iters) / (ms * 1e-3) / 1e12


def mfma_i8_tops(workgroups, iters, reps=10):
    """Sustained dense int8 MFMA TOP/s of the loop probe."""
    L = lib()
    out = torch.empty(workgroups * 256, dtype=torch.int32, device="cuda")
    st = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)

    def launch():
        rc = L.qgprobe_mfma_i8(ctypes.c_void_p(out.data_ptr()), workgroups, iters, st)
        if rc:
            raise RuntimeError(f"qgprobe_mfma_i8 status {rc}")
    ms = _events_ms(launch, reps)
    return L.qgprobe_mfma_flops(64, workgroups, iters) / (ms * 1e-3) / 1e12


def hbm_read_gbps(buffers, workgroups, unroll, reps=20):
    """Sustained HBM read GB/s of the streaming probe, rotating over
    `buffers` (device uint8 tensors) so no read is served from cache."""
    L = lib()
    out = torch.empty(workgroups * 256, dtype=torch.int32, device="cuda")
    st = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    nbytes = buffers[0].numel() // 1024 * 1024
    k = [0]

    def launch():
        b = buffers[k[0] % len(buffers)]
        k[0] += 1
        rc = L.qgprobe_hbm_read(ctypes.c_void_p(b.data_ptr()), nbytes, ctypes.c_void_p(out.data_ptr()),
                                workgroups, unroll, st)
        if rc:
            raise RuntimeError(f"qgprobe_hbm_read status {rc}")
    ms = _events_ms(launch, reps)
    return nbytes / (ms * 1e-3) / 1e9
