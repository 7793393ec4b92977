// Load-time repack of 4-bit codes into the MFMA-operand tile layout, with the
// sign fold of negative group scales and the asymmetric delta.
//
// Sources: "Marlin INT4 on Ada - how it works", section "The pipeline, end to
// end" (a load-time pass that packs 8 codes per uint32 in the GEMM's operand
// order and computes delta = zero + 8*scale per group and column); the
// HyperQwen W4A8 article, negative group-scale section (scale -> -scale,
// code v -> 16 - v, clamped to 15 for v = 0).
#include "qg_device.h"
#include "qg_launch.h"

namespace qg {

// binary16 -> binary64, exact.
__device__ inline double f16_bits_to_f64(uint16_t b)
{
    unsigned e = (b >> 10) & 31u, f = b & 1023u;
    double mag;
    if (e == 0)
        mag = (double)f * 0x1p-24;
    else if (e == 31)
        mag = f ? __builtin_nan("") : __builtin_inf();
    else
        mag = (double)(1024u + f) * __builtin_ldexp(1.0, (int)e - 25);
    return (b & 0x8000) ? -mag : mag;
}

// binary64 -> binary16, round to nearest, ties to even (integer arithmetic on
// the significand, so there is exactly one rounding).
__device__ inline uint16_t f64_to_f16_rne(double x)
{
    uint64_t b = __builtin_bit_cast(uint64_t, x);
    uint16_t sign = (uint16_t)((b >> 48) & 0x8000u);
    int ex = (int)((b >> 52) & 0x7ff);
    uint64_t man = b & ((1ull << 52) - 1);
    if (ex == 0x7ff) return (uint16_t)(sign | (man ? 0x7e00u : 0x7c00u));
    if (ex == 0) return sign;                       // binary64 subnormal -> 0
    int e = ex - 1023;
    if (e > 15) return (uint16_t)(sign | 0x7c00u);
    uint64_t sig = (1ull << 52) | man;              // 53-bit significand
    int shift = 42 + (e < -14 ? (-14 - e) : 0);      // keep 10 fraction bits
    if (shift > 62) return sign;
    uint64_t r = sig >> shift;
    uint64_t rem = sig & ((1ull << shift) - 1);
    uint64_t halfway = 1ull << (shift - 1);
    if (rem > halfway || (rem == halfway && (r & 1))) ++r;
    if (e >= -14) {
        if (r == 2048) { r = 1024; ++e; }
        if (e > 15) return (uint16_t)(sign | 0x7c00u);
        return (uint16_t)(sign | (uint16_t)((e + 15) << 10) | (uint16_t)(r - 1024));
    }
    return (uint16_t)(sign | (uint16_t)r);          // subnormal (r == 1024 -> 2^-14)
}

// One thread per packed uint32 of the padded [Kp, Np] weight; codes outside
// the logical [K, N] are 8 (zero weight for a symmetric pack; the GEMM pads
// the activations with zeros and drops the extra columns anyway).
__global__ void pack_codes_kernel(const uint8_t *__restrict__ q, const uint16_t *__restrict__ s,
                                  int K, int N, int Kp, int g, int fold,
                                  uint32_t *__restrict__ out, size_t total)
{
    size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= total) return;
    size_t tile = i >> 8;
    int within = (int)(i & 255);
    int lane = within >> 2, j = within & 3;
    int KT = Kp / KTILE;
    int nt = (int)(tile / KT), kt = (int)(tile % KT);
    int n = nt * NTILE + (lane & 15);
    int kq = lane >> 4;
    uint32_t word = 0;
#pragma unroll
    for (int p = 0; p < 8; ++p) {
        int k = kt * KTILE + tile_k(kq, j, p);
        unsigned v = 8u;
        if (k < K && n < N) {
            v = q[(size_t)k * N + n] & 15u;
            if (fold && f16_is_negative(s[(size_t)(k / g) * N + n])) {
                v = 16u - v;
                if (v > 15u) v = 15u;
            }
        }
        word |= v << (4 * p);
    }
    out[i] = word;
}

// One thread per (group, column) of the padded [G, Np] outputs: folded scale
// and delta; 0 in the columns past N and in the groups past the Gin groups of
// the input (groups of 32 or 64 with K padded to a multiple of 128 can add
// whole groups that hold no k < K).
__global__ void pack_scales_kernel(const uint16_t *__restrict__ s, const uint16_t *__restrict__ z,
                                   int N, int Np, int Gin, int fold, uint16_t *s_out,
                                   uint16_t *__restrict__ d_out, size_t total)
{
    size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= total) return;
    const size_t gi = i / Np;
    const int n = (int)(i % Np);
    if (n >= N || gi >= (size_t)Gin) {
        if (z) d_out[i] = 0;
        s_out[i] = 0;
        return;
    }
    const size_t src = gi * N + n;
    uint16_t sb = s[src];
    if (z) d_out[i] = f64_to_f16_rne(f16_bits_to_f64(z[src]) + 8.0 * f16_bits_to_f64(sb));
    s_out[i] = (fold && f16_is_negative(sb)) ? (uint16_t)(sb ^ 0x8000u) : sb;
}

void padded_shape(int K, int N, int g, int *Kp, int *Np, int *gp)
{
    // g == K: one group per column, padded with K to a multiple of 128;
    // g = 32 or 64: K padded to a multiple of 128 (whole groups, whole tiles);
    // otherwise g is a multiple of 128 and K is padded to a whole group
    const int kp = (g == K || g < KTILE) ? (K + KTILE - 1) / KTILE * KTILE : (K + g - 1) / g * g;
    *Kp = kp;
    *Np = (N + 127) / 128 * 128;
    *gp = g == K ? kp : g;
}

hipError_t launch_pack(const uint8_t *q, const uint16_t *s, const uint16_t *z, int K, int N,
                       int g, bool fold, uint32_t *w, uint16_t *s_out, uint16_t *d_out,
                       hipStream_t st)
{
    // the fold only applies to symmetric weights
    int f = (fold && z == nullptr) ? 1 : 0;
    int Kp, Np, gp;
    padded_shape(K, N, g, &Kp, &Np, &gp);
    size_t total = (size_t)Kp * Np / 8;
    int bs = 256;
    // codes first: they read the original scales, which s_out may overwrite
    hipLaunchKernelGGL(pack_codes_kernel, dim3((unsigned)((total + bs - 1) / bs)), dim3(bs), 0, st,
                       q, s, K, N, Kp, g, f, w, total);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    size_t gt = (size_t)(Kp / gp) * Np;
    const int gin = (K + g - 1) / g;          // groups the input scale rows hold
    hipLaunchKernelGGL(pack_scales_kernel, dim3((unsigned)((gt + bs - 1) / bs)), dim3(bs), 0, st,
                       s, z, N, Np, gin, f, s_out, d_out, gt);
    return hipGetLastError();
}

} // namespace qg
