// Per-token (per-row) int8 quantization of fp16 activations, the input stage
// of the W4A8 path.
//
// Source: the HyperQwen W4A8 article, section "why int8 activation
// quantization (W4A8) is worth doing" (activations quantized per token to
// int8, weights kept 4-bit).  The rule is the plain symmetric absmax one:
//   a_scale[m] = max_k |A[m,k]| / 127
//   A_q[m,k]   = clamp(round_half_even(A[m,k] / a_scale[m]), -127, 127)
// with both divisions IEEE binary32 operations (round to nearest even); a row
// of zeros gets a_scale 0 and codes 0.
//
// HBM-bound at large M*K: each value is read once (a row of up to 16 chunks
// of 8 values per lane stays in registers between the absmax and the code
// pass) and its code written once; small batches are launch- and
// latency-bound.  One workgroup of four waves per row.
#include "qg_device.h"
#include "qg_launch.h"

namespace qg {
namespace {

// The code pass (`codes` below).  The int8 code of x at scale sc > 0 is
// clamp(rint(x / sc), -127, 127) with
// x / sc one correctly rounded binary32 division (sc == 0 only for a row of
// zeros: code 0).  The division is costly, so the code is first taken from
// y = x * inv, inv = 1 / sc correctly rounded: |y - x/sc| stays below 2^-15
// for |x| <= 128 sc (two roundings of relative size 2^-24 each), and the
// correctly rounded quotient is within 2^-18 of x/sc, so both round to the
// same integer unless y lies within 2^-15 + 2^-18 of a half-integer.  Only
// then (|y - rint(y)| within 2^-12 of 1/2, rare) is the division done.
// Rounding: y + 1.5 * 2^23 lands in [2^23, 2^24), where the spacing of
// binary32 is 1, so the sum is y rounded to an integer (nearest, ties to
// even) and its low significand byte is that integer's two's complement
// byte -- the code, taken from the bits without a float-to-int conversion.
// The clamp never acts: |x| <= max_k |A[m,k]| makes |x / sc| at most 127 (1 +
// 2^-23), so |rint| <= 127 on both routes.  The eight values of a chunk
// share one branch to the division fallback.

// WPR waves per row, 4 / WPR rows per 256-thread workgroup.  Each lane takes
// 16-byte chunks of 8 values, the waves of a row interleaved chunk by chunk.
// CPL > 0: the row fits in CPL chunks per lane, which stay in registers
// between the two passes (one HBM read per value); CPL == 0: the second pass
// reads the row again.
template <int WPR, int CPL>
__global__ __launch_bounds__(256) void quantize_rows_int8_kernel(
    const uint16_t *__restrict__ A, int8_t *__restrict__ Aq, float *__restrict__ a_scale,
    int M, int K)
{
    constexpr int RPW = 4 / WPR;
    constexpr int NR = CPL > 0 ? CPL : 1;
    __shared__ unsigned red[4];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int row = blockIdx.x * RPW + wave / WPR;
    const int part = wave % WPR;
    const bool live = row < M;
    // a row past M (last workgroup only) reads row M-1 and stores nothing, so
    // every wave reaches the barrier
    const int r = live ? row : M - 1;
    const uint4v *a = reinterpret_cast<const uint4v *>(A + (size_t)r * K);
    const int nch = K / 8;
    const int c0 = part * 64 + lane;
    constexpr int STEP = 64 * WPR;

    // max |x| as binary16 magnitude bits: for finite values the order of the
    // magnitudes is the integer order of the bits with the sign cleared
    unsigned mx = 0;
    auto absmax = [&](const uint4v &v) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            mx = __builtin_elementwise_max(mx, v[j] & 0x7fffu);
            mx = __builtin_elementwise_max(mx, (v[j] >> 16) & 0x7fffu);
        }
    };
    uint4v keep[NR];
    if (CPL > 0) {
#pragma unroll
        for (int i = 0; i < NR; ++i) {
            const int c = c0 + i * STEP;
            keep[i] = c < nch ? a[c] : uint4v{0u, 0u, 0u, 0u};
        }
#pragma unroll
        for (int i = 0; i < NR; ++i) absmax(keep[i]);
    } else {
#pragma unroll 4
        for (int c = c0; c < nch; c += STEP) absmax(a[c]);
    }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1)
        mx = __builtin_elementwise_max(mx, (unsigned)__shfl_xor((int)mx, o));
    if (WPR > 1) {
        if (lane == 0) red[wave] = mx;
        __syncthreads();
        const int w0 = (wave / WPR) * WPR;
#pragma unroll
        for (int i = 0; i < WPR; ++i) mx = __builtin_elementwise_max(mx, red[w0 + i]);
    }
    if (!live) return;

    const float sc = h2f((uint16_t)mx) / 127.0f;
    const float inv = sc > 0.0f ? 1.0f / sc : 0.0f;
    if (part == 0 && lane == 0) a_scale[row] = sc;
    uint2v *q = reinterpret_cast<uint2v *>(Aq + (size_t)row * K);
    auto codes = [&](const uint4v &v) {
        constexpr float MAGIC = 0x1.8p23f;
        float x[8], t[8];
        bool nd[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            x[j] = h2f((uint16_t)(v[j / 2] >> (16 * (j & 1))));
            const float y = x[j] * inv;
            t[j] = y + MAGIC;
            const float r = t[j] - MAGIC;
            nd[j] = __builtin_fabsf(__builtin_fabsf(y - r) - 0.5f) < 0x1p-12f;
        }
        if (nd[0] | nd[1] | nd[2] | nd[3] | nd[4] | nd[5] | nd[6] | nd[7]) {
#pragma unroll
            for (int j = 0; j < 8; ++j)
                if (nd[j]) t[j] = x[j] / sc + MAGIC;
        }
        unsigned out[2];
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const unsigned a0 = __builtin_bit_cast(unsigned, t[4 * h]), a1 = __builtin_bit_cast(unsigned, t[4 * h + 1]);
            const unsigned b0 = __builtin_bit_cast(unsigned, t[4 * h + 2]), b1 = __builtin_bit_cast(unsigned, t[4 * h + 3]);
            const unsigned pa = __builtin_amdgcn_perm(a1, a0, 0x0c0c0400u);
            const unsigned pb = __builtin_amdgcn_perm(b1, b0, 0x0c0c0400u);
            out[h] = __builtin_amdgcn_perm(pb, pa, 0x05040100u);
        }
        return uint2v{out[0], out[1]};
    };
    if (CPL > 0) {
#pragma unroll
        for (int i = 0; i < NR; ++i) {
            const int c = c0 + i * STEP;
            if (c < nch) q[c] = codes(keep[i]);
        }
    } else {
#pragma unroll 4
        for (int c = c0; c < nch; c += STEP) q[c] = codes(a[c]);
    }
}

template <int WPR>
hipError_t launch_quant(const uint16_t *A, int M, int K, int8_t *Aq, float *a_scale,
                        hipStream_t st)
{
    const int per_lane = (K / 8 + 64 * WPR - 1) / (64 * WPR);   // chunks per lane
    const dim3 grid((M + 4 / WPR - 1) / (4 / WPR)), block(256);
#define QG_QUANT(CPL) \
    hipLaunchKernelGGL((quantize_rows_int8_kernel<WPR, CPL>), grid, block, 0, st, A, Aq, a_scale, M, K)
    if (per_lane <= 1) QG_QUANT(1);
    else if (per_lane <= 2) QG_QUANT(2);
    else if (per_lane <= 4) QG_QUANT(4);
    else if (per_lane <= 8) QG_QUANT(8);
    else if (per_lane <= 16) QG_QUANT(16);
    else QG_QUANT(0);
#undef QG_QUANT
    return hipGetLastError();
}

} // namespace

hipError_t launch_quantize_rows_int8(const uint16_t *A, int M, int K, int8_t *Aq,
                                     float *a_scale, hipStream_t st)
{
    // four waves per row: faster than one wave per row at every size measured
    // (M = 16 .. 8192 rows, K = 2048 .. 5120; 16.5 against 19.7 us at
    // M = 4096, K = 5120), since the workgroups are then short enough for
    // one round of them to overlap the next one's loads
    return launch_quant<4>(A, M, K, Aq, a_scale, st);
}

} // namespace qg
