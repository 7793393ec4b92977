// Grouped W4A8 GEMM: 4-bit symmetric weights x per-token int8 activations on
// int8 MFMA with exact int32 accumulation per weight group, then per-group and
// per-token scaling in fp32.
//
// Method: the HyperQwen W4A8 article, section on why int8 activation
// quantization is worth doing (weights stay int4, activations are quantized per
// token to int8, the product runs on int8 matrix cores); the grouped layout
// (one weight matrix per expert, rows of each expert contiguous) follows the
// SGLang w4a8 MoE article's "task split" section.  That article's bug was a
// scale applied before the asynchronous matrix ops had finished; here the
// MFMA results are plain register values, and the compiler's dependency
// tracking orders every read of an accumulator after the MFMA that wrote it.
//
// Kernel.  A wave owns MT 16-row m-tiles x NT 16-column n-tiles of one expert
// and a range of whole weight groups.  Per 128-k tile and n-tile, one 128-bit
// word of codes per lane becomes two 16x16x64 int8 operands of 16*(v-8) by
// masking and an XOR; A's bytes are loaded in the same k order.  At the end of
// each group the int32 accumulator (exactly 16x the group's integer product)
// is shifted right by 4, optionally stored to acc_debug, and folded into the
// fp32 accumulator with the group scale.  The waves of a workgroup split the
// groups and are summed through LDS; the per-token scale is applied last.
#include "qg_device.h"
#include "qg_launch.h"

namespace qg {

template <int MT, int NT, int NWMAX>
__global__ __launch_bounds__(NWMAX * 64) void w4a8_kernel(
    const int8_t *__restrict__ Aq, const float *__restrict__ a_scale,
    const uint4v *__restrict__ Wall, const uint16_t *__restrict__ Sall,
    const int32_t *__restrict__ offsets, int M_total, int N, int K, int g,
    uint16_t *__restrict__ C, int32_t *__restrict__ acc_debug, int nw)
{
    extern __shared__ float red[];
    const int e = blockIdx.z;
    int r0 = 0, r1 = M_total;
    if (offsets) {
        r0 = offsets[e];
        r1 = offsets[e + 1];
        r0 = r0 < 0 ? 0 : (r0 > M_total ? M_total : r0);
        r1 = r1 < r0 ? r0 : (r1 > M_total ? M_total : r1);
    }
    const int m0 = r0 + blockIdx.y * 16 * MT;
    if (m0 >= r1) return;   // uniform over the workgroup, before any barrier

    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int c = lane & 15, kq = lane >> 4;
    const int KT = K / KTILE, G = K / g, kpg = g / KTILE;
    const int nt0 = blockIdx.x * NT;
    const uint4v *W = Wall + (size_t)e * KT * (N / NTILE) * 64;
    const uint16_t *S = Sall + (size_t)e * G * N;
    const int g_beg = (wave * G) / nw, g_end = ((wave + 1) * G) / nw;

    const int8_t *arow[MT];
    bool aok[MT];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
        int r = m0 + 16 * mt + c;
        aok[mt] = r < r1;
        arow[mt] = Aq + (size_t)(aok[mt] ? r : 0) * K + 8 * kq;
    }
    const uint4v *wp[NT];
    int col[NT];
#pragma unroll
    for (int t = 0; t < NT; ++t) {
        wp[t] = W + (size_t)(nt0 + t) * KT * 64 + lane;
        col[t] = (nt0 + t) * NTILE + c;
    }

    float4v accf[MT][NT];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int t = 0; t < NT; ++t) accf[mt][t] = float4v{0.f, 0.f, 0.f, 0.f};
    const int4v izero = {0, 0, 0, 0};

    for (int gi = g_beg; gi < g_end; ++gi) {
        int4v acci[MT][NT];
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
#pragma unroll
            for (int t = 0; t < NT; ++t) acci[mt][t] = izero;
        for (int kt = gi * kpg; kt < (gi + 1) * kpg; ++kt) {
            uint4v w[NT];
#pragma unroll
            for (int t = 0; t < NT; ++t) w[t] = wp[t][(size_t)kt * 64];
            int4v alo[MT], ahi[MT];
#pragma unroll
            for (int mt = 0; mt < MT; ++mt) {
                const int8_t *p = arow[mt] + kt * KTILE;
                uint2v q0 = {0u, 0u}, q1 = {0u, 0u}, q2 = {0u, 0u}, q3 = {0u, 0u};
                if (aok[mt]) {
                    q0 = *reinterpret_cast<const uint2v *>(p);
                    q1 = *reinterpret_cast<const uint2v *>(p + 32);
                    q2 = *reinterpret_cast<const uint2v *>(p + 64);
                    q3 = *reinterpret_cast<const uint2v *>(p + 96);
                }
                alo[mt] = int4v{(int)swap_mid_bytes(q0.x), (int)swap_mid_bytes(q0.y),
                                (int)swap_mid_bytes(q1.x), (int)swap_mid_bytes(q1.y)};
                ahi[mt] = int4v{(int)swap_mid_bytes(q2.x), (int)swap_mid_bytes(q2.y),
                                (int)swap_mid_bytes(q3.x), (int)swap_mid_bytes(q3.y)};
            }
#pragma unroll
            for (int t = 0; t < NT; ++t) {
                CodeOpsI8 b = split_codes_i8(w[t]);
#pragma unroll
                for (int mt = 0; mt < MT; ++mt) {
                    acci[mt][t] = mfma_i8(alo[mt], b.op[0], acci[mt][t]);
                    acci[mt][t] = mfma_i8(ahi[mt], b.op[1], acci[mt][t]);
                }
            }
        }
#pragma unroll
        for (int t = 0; t < NT; ++t) {
            const float s = h2f(S[(size_t)gi * N + col[t]]);
#pragma unroll
            for (int mt = 0; mt < MT; ++mt) {
                int4v qv = acci[mt][t] >> 4;   // exact: every term is a multiple of 16
                accf[mt][t] += s * __builtin_convertvector(qv, float4v);
                if (acc_debug) {
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        int row = m0 + 16 * mt + 4 * (lane >> 4) + r;
                        if (row < r1) acc_debug[((size_t)row * G + gi) * N + col[t]] = qv[r];
                    }
                }
            }
        }
    }

    constexpr int E4 = MT * NT * 4;
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int t = 0; t < NT; ++t)
#pragma unroll
            for (int r = 0; r < 4; ++r)
                red[((size_t)wave * E4 + (mt * NT + t) * 4 + r) * 64 + lane] = accf[mt][t][r];
    __syncthreads();
    for (int idx = threadIdx.x; idx < E4 * 64; idx += blockDim.x) {
        float v = 0.f;
        for (int w = 0; w < nw; ++w) v += red[(size_t)w * E4 * 64 + idx];
        const int ee = idx >> 6, l = idx & 63;
        const int r = ee & 3, t = (ee >> 2) % NT, mt = (ee >> 2) / NT;
        const int row = m0 + 16 * mt + 4 * (l >> 4) + r;
        const int cc = (nt0 + t) * NTILE + (l & 15);
        if (row < r1) C[(size_t)row * N + cc] = f2h(a_scale[row] * v);
    }
}

template <int MT, int NT, int NWMAX>
static hipError_t run_w4a8(const int8_t *Aq, const float *a_scale, const uint32_t *W,
                           const uint16_t *S, const int32_t *offsets, int E, int M_total,
                           int max_rows, int N, int K, int g, uint16_t *C, int32_t *acc_debug,
                           hipStream_t st)
{
    const int G = K / g;
    dim3 grid((unsigned)(N / NTILE / NT), (unsigned)((max_rows + 16 * MT - 1) / (16 * MT)),
              (unsigned)E);
    long blocks = (long)grid.x * grid.y * grid.z;
    int nw = 1;
    while (nw < NWMAX && blocks * nw * 2 <= 2560 && G / (nw * 2) >= 1) nw *= 2;
    size_t lds = (size_t)nw * MT * NT * 4 * 64 * sizeof(float);
    hipLaunchKernelGGL((w4a8_kernel<MT, NT, NWMAX>), grid, dim3(64 * nw), lds, st, Aq, a_scale,
                       reinterpret_cast<const uint4v *>(W), S, offsets, M_total, N, K, g, C,
                       acc_debug, nw);
    return hipGetLastError();
}

hipError_t launch_w4a8(const int8_t *Aq, const float *a_scale, const uint32_t *W,
                       const uint16_t *S, const int32_t *offsets, int E, int M_total,
                       int max_rows, int N, int K, int g, uint16_t *C, int32_t *acc_debug,
                       hipStream_t st)
{
    if (max_rows <= 16)
        return run_w4a8<1, 2, 16>(Aq, a_scale, W, S, offsets, E, M_total, max_rows, N, K, g, C,
                                  acc_debug, st);
    if (max_rows <= 32)
        return run_w4a8<2, 2, 8>(Aq, a_scale, W, S, offsets, E, M_total, max_rows, N, K, g, C,
                                 acc_debug, st);
    return run_w4a8<4, 2, 4>(Aq, a_scale, W, S, offsets, E, M_total, max_rows, N, K, g, C,
                             acc_debug, st);
}

} // namespace qg
