// Achievable-peak probes for the measurement harness (not part of the GEMM
// path): a matrix-core loop and an HBM streaming read, each timed by the
// caller.  Declared in include/qgprobe.h.
#include <hip/hip_runtime.h>
#include <cstddef>
#include <cstdint>

#include "qgprobe.h"

namespace {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef float float4v __attribute__((ext_vector_type(4)));
typedef float float16v __attribute__((ext_vector_type(16)));
typedef unsigned int uint4v __attribute__((ext_vector_type(4)));

// Every wave runs `iters` rounds of CH independent MFMA chains.  The MFMAs
// are written as asm so the accumulators stay in place (the compiler
// otherwise shuttles some of them between register files every round); the
// chains are CH instructions apart, far more than any dependency needs, and
// the s_nops after the loop cover the last results before they are read.
template <int CH>
__global__ __launch_bounds__(256) void mfma16_loop(float *out, int iters, float seed)
{
    half8 a, b;
    for (int i = 0; i < 8; ++i) {
        a[i] = (_Float16)(seed * (float)(threadIdx.x + i));
        b[i] = (_Float16)(seed * (float)i);
    }
    float4v acc[CH];
    for (int j = 0; j < CH; ++j) acc[j] = float4v{0.f, 0.f, 0.f, 0.f};
    asm volatile("s_nop 4" ::: "memory"); // operands written by VALU just before
    for (int it = 0; it < iters; ++it) {
#pragma unroll
        for (int j = 0; j < CH; ++j)
            asm volatile("v_mfma_f32_16x16x32_f16 %0, %1, %2, %0" : "+v"(acc[j]) : "v"(a), "v"(b));
    }
    asm volatile("s_nop 7\n s_nop 7\n s_nop 7" ::: "memory");
    float s = 0.f;
    for (int j = 0; j < CH; ++j) s += acc[j][0] + acc[j][1] + acc[j][2] + acc[j][3];
    out[(size_t)blockIdx.x * 256 + threadIdx.x] = s;
}

template <int CH>
__global__ __launch_bounds__(256) void mfma32_loop(float *out, int iters, float seed)
{
    half8 a, b;
    for (int i = 0; i < 8; ++i) {
        a[i] = (_Float16)(seed * (float)(threadIdx.x + i));
        b[i] = (_Float16)(seed * (float)i);
    }
    float16v acc[CH];
    for (int j = 0; j < CH; ++j)
        for (int r = 0; r < 16; ++r) acc[j][r] = 0.f;
    asm volatile("s_nop 4" ::: "memory"); // operands written by VALU just before
    for (int it = 0; it < iters; ++it) {
#pragma unroll
        for (int j = 0; j < CH; ++j)
            asm volatile("v_mfma_f32_32x32x16_f16 %0, %1, %2, %0" : "+v"(acc[j]) : "v"(a), "v"(b));
    }
    asm volatile("s_nop 7\n s_nop 7\n s_nop 7" ::: "memory");
    float s = 0.f;
    for (int j = 0; j < CH; ++j)
        for (int r = 0; r < 16; ++r) s += acc[j][r];
    out[(size_t)blockIdx.x * 256 + threadIdx.x] = s;
}

typedef int int4v __attribute__((ext_vector_type(4)));

// int8 16x16x64 MFMA loop, sixteen independent chains per wave, as above.
template <int CH>
__global__ __launch_bounds__(256) void mfma_i8_loop(int *out, int iters, int seed)
{
    int4v a, b;
    for (int i = 0; i < 4; ++i) {
        a[i] = seed * (int)(threadIdx.x + i);
        b[i] = seed * i;
    }
    int4v acc[CH];
    for (int j = 0; j < CH; ++j) acc[j] = int4v{0, 0, 0, 0};
    asm volatile("s_nop 4" ::: "memory"); // operands written by VALU just before
    for (int it = 0; it < iters; ++it) {
#pragma unroll
        for (int j = 0; j < CH; ++j)
            asm volatile("v_mfma_i32_16x16x64_i8 %0, %1, %2, %0" : "+v"(acc[j]) : "v"(a), "v"(b));
    }
    asm volatile("s_nop 7\n s_nop 7\n s_nop 7" ::: "memory");
    int s = 0;
    for (int j = 0; j < CH; ++j) s += acc[j][0] + acc[j][1] + acc[j][2] + acc[j][3];
    out[(size_t)blockIdx.x * 256 + threadIdx.x] = s;
}

// Each wave reads its own contiguous run of 1 KiB blocks (one 16-byte load
// per lane per block) in batches of U blocks, the next batch issued before
// the current one is consumed.  Loads past the run are clamped to its last
// block (unconditional loads keep the compiler's wait counts exact); every
// byte loaded feeds the result.
template <int U>
__global__ __launch_bounds__(256) void stream_read(const uint4v *__restrict__ src, unsigned *__restrict__ out,
                                                   long long nblk, long long per_wave)
{
    const int lane = threadIdx.x & 63;
    const long long wave = (long long)blockIdx.x * 4 + (threadIdx.x >> 6);
    const long long b0 = wave * per_wave;
    long long b1 = b0 + per_wave;
    b1 = b1 < nblk ? b1 : nblk;
    unsigned acc = 0;
    if (b0 < b1) {
        uint4v v0[U], v1[U];
        auto issue = [&](long long c, uint4v (&v)[U]) {
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const long long b = c + u < b1 ? c + u : b1 - 1;
                v[u] = src[b * 64 + lane];
            }
        };
        auto use = [&](long long c, const uint4v (&v)[U]) {
#pragma unroll
            for (int u = 0; u < U; ++u)
                if (c + u < b1) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
        };
        issue(b0, v0);
        // the scheduling barriers keep each batch's loads issued before the
        // previous batch is waited for
        for (long long c = b0; c < b1; c += 2 * U) {
            issue(c + U, v1);
            __builtin_amdgcn_sched_barrier(0);
            use(c, v0);
            __builtin_amdgcn_sched_barrier(0);
            issue(c + 2 * U, v0);
            __builtin_amdgcn_sched_barrier(0);
            use(c + U, v1);
            __builtin_amdgcn_sched_barrier(0);
        }
    }
    out[wave * 64 + lane] = acc;
}

} // namespace

extern "C" int qgprobe_mfma_f16(int shape, float *out, int workgroups, int iters, void *stream)
{
    if (!out || workgroups < 1 || iters < 1 || (shape != 16 && shape != 32)) return 1;
    hipStream_t st = static_cast<hipStream_t>(stream);
    if (shape == 16)
        hipLaunchKernelGGL(mfma16_loop<16>, dim3(workgroups), dim3(256), 0, st, out, iters, 1e-3f);
    else
        hipLaunchKernelGGL(mfma32_loop<4>, dim3(workgroups), dim3(256), 0, st, out, iters, 1e-3f);
    return hipGetLastError() == hipSuccess ? 0 : 5;
}

extern "C" int qgprobe_mfma_i8(int *out, int workgroups, int iters, void *stream)
{
    if (!out || workgroups < 1 || iters < 1) return 1;
    hipLaunchKernelGGL(mfma_i8_loop<16>, dim3(workgroups), dim3(256), 0, static_cast<hipStream_t>(stream), out,
                       iters, 3);
    return hipGetLastError() == hipSuccess ? 0 : 5;
}

extern "C" long long qgprobe_mfma_flops(int shape, int workgroups, int iters)
{
    // operations one launch performs: 16 / 32 = qgprobe_mfma_f16 of that
    // shape, 64 = qgprobe_mfma_i8; 0 for any other shape
    long long per = 0;
    if (shape == 16) per = 16LL * 16 * 32 * 2 * 16;
    if (shape == 32) per = 32LL * 32 * 16 * 2 * 4;
    if (shape == 64) per = 16LL * 16 * 64 * 2 * 16;
    return per * iters * (long long)workgroups * 4;
}

extern "C" int qgprobe_hbm_read(const void *buf, size_t bytes, unsigned *out, int workgroups, int unroll,
                                void *stream)
{
    if (!buf || !out || workgroups < 1 || bytes < 1024 || (unroll != 1 && unroll != 2 && unroll != 4 && unroll != 8 && unroll != 16)) return 1;
    const long long nblk = (long long)(bytes / 1024);
    const long long waves = (long long)workgroups * 4;
    const long long per_wave = (nblk + waves - 1) / waves;
    hipStream_t st = static_cast<hipStream_t>(stream);
    const uint4v *src = static_cast<const uint4v *>(buf);
    switch (unroll) {
    case 1: hipLaunchKernelGGL(stream_read<1>, dim3(workgroups), dim3(256), 0, st, src, out, nblk, per_wave); break;
    case 2: hipLaunchKernelGGL(stream_read<2>, dim3(workgroups), dim3(256), 0, st, src, out, nblk, per_wave); break;
    case 4: hipLaunchKernelGGL(stream_read<4>, dim3(workgroups), dim3(256), 0, st, src, out, nblk, per_wave); break;
    case 8: hipLaunchKernelGGL(stream_read<8>, dim3(workgroups), dim3(256), 0, st, src, out, nblk, per_wave); break;
    case 16: hipLaunchKernelGGL(stream_read<16>, dim3(workgroups), dim3(256), 0, st, src, out, nblk, per_wave); break;
    default: return 1;
    }
    return hipGetLastError() == hipSuccess ? 0 : 5;
}
