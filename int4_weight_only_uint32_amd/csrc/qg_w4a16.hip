// W4A16 GEMM kernels and the two-stage asymmetric correction.
//
// Method ("Marlin INT4 on Ada - how it works", section "The core mismatch:
// symmetric vs asymmetric"): with delta[g,n] = zero[g,n] + 8*scale[g,n],
//     C = A . W_sym + A_group_sum @ delta,  W_sym[k,n] = (q[k,n] - 8) scale[g,n]
// which is exact because delta does not depend on k.
//
// This file: the skinny kernel, the dispatch between the W4A16 kernels, the
// K/N tail path, the SwiGLU dispatch and the two-stage correction; the decode,
// mid-batch and tiled kernels have files of their own.
//
// Skinny kernel (M <= 80; for most shapes the decode kernel, which shares the
// activation tile between waves, is used instead: see use_decode_kernel).  A wave owns MT 16-row m-tiles x NT 16-column
// n-tiles and a contiguous range of 128-k tiles, with P tiles of codes and
// activations in flight in a register ring; the waves of a workgroup split K
// and are summed through LDS at the end (one launch, no workspace).
// Per 128-k tile and n-tile, a lane loads one 128-bit word of codes, turns it
// into four fp16 MFMA operands by masking alone (codes as exact fp16
// subnormals), and runs four 16x16x32 fp16 MFMAs that accumulate
//     X = sum_k A[m,k] * q[k,n]            (unsigned codes, up to 2^-20)
// The group scale is applied once per tile on the fp32 accumulator:
//     acc += scale * X + (delta - 8 scale) * a_sum        (asymmetric)
//     acc += scale * X - 8 scale * a_sum                   (symmetric)
// where a_sum = sum_k A[m,k] over the tile comes from four MFMAs against an
// all-ones operand (it lands in the accumulator layout, no shuffles).
#include "qg_device.h"
#include "qg_launch.h"

#include <cstdio>
#include <type_traits>

namespace qg {

// GPT: weight groups per 128-k tile (1 for g >= 128, 2 for g = 64, 4 for
// g = 32), as in the decode kernel: each 32-k MFMA step's products are scaled
// with the scale, delta and activation sum of the step's own group.
template <int MT, int NT, int P, int NWMAX, bool DELTA, bool GATED, int GPT = 1>
__global__ __launch_bounds__(NWMAX * 64) void w4a16_skinny_kernel(
    const uint16_t *__restrict__ A, const uint4v *__restrict__ W, const uint16_t *__restrict__ S,
    const uint16_t *__restrict__ D, uint16_t *__restrict__ C, int M, int N, int K, int g, int nw)
{
    // LDS: per wave, one k-tile of activations (16*MT rows x 128 k fp16,
    // 16-byte chunks swizzled by row); reused for the cross-wave sum.
    extern __shared__ __attribute__((aligned(16))) float red[];
    constexpr int SLOT_HALVES = MT * 16 * KTILE;
    const int lane = threadIdx.x & 63;
    // the wave index is uniform across a wave: keep it (and everything derived
    // from it) in scalar registers
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int c = lane & 15, kq = lane >> 4;
    const int KT = K / KTILE;
    const int nt0 = blockIdx.x * NT;
    // GATED: the NT (virtual) n-tiles are NT/2 gate/up pairs of the [K, N]
    // pair weight, and C is the [M, N/2] output
    const int Nh16 = N / (2 * NTILE);
    const int pt0 = GATED ? gated_tile(nt0, 0, Nh16) : nt0;   // first physical tile
    // physical tile of n-tile t, relative to pt0
    auto trel = [&](int t) { return GATED ? gated_tile(nt0, t, Nh16) - pt0 : t; };
    const int m0 = blockIdx.y * 16 * MT;
    const int kt_beg = (wave * KT) / nw, kt_end = ((wave + 1) * KT) / nw;
    const int n = kt_end - kt_beg;
    _Float16 *scratch = reinterpret_cast<_Float16 *>(red) + (size_t)wave * SLOT_HALVES;

    // Activations are fetched row-contiguously (load j covers rows 4j..4j+3,
    // 256 bytes each: lane i reads chunk i%16 of row 4j + i/16), which keeps a
    // wave's request to 8 whole cache lines, then rearranged through LDS into
    // the MFMA operand layout.  Rows past M read row M-1 (they only feed output
    // rows that are never stored).
    const uint4v *asrc[MT * 4];
    int adst[MT * 4];
#pragma unroll
    for (int j = 0; j < MT * 4; ++j) {
        const int r = 4 * j + (lane >> 4);
        int row = m0 + r;
        row = row < M ? row : M - 1;
        asrc[j] = reinterpret_cast<const uint4v *>(A + (size_t)row * K) + (lane & 15);
        adst[j] = r * KTILE + 8 * ((lane & 15) ^ (r & 15));
    }
    const uint4v *wbase = W + (size_t)pt0 * KT * 64 + lane;
    const int col0 = pt0 * NTILE + c;

    float4v acc[MT][NT];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int t = 0; t < NT; ++t) acc[mt][t] = float4v{0.f, 0.f, 0.f, 0.f};

    const half8 ones = {1, 1, 1, 1, 1, 1, 1, 1};
    const float4v fzero = {0.f, 0.f, 0.f, 0.f};

    // P-deep register ring.  Every slot is refilled unconditionally (tile
    // index clamped to the wave's last tile) so the loads in flight are the
    // same on every path and each wait only covers the slot being consumed.
    uint4v ra[P][MT * 4];
    uint4v rw[P][NT];
    // Scales and deltas are fetched as the aligned 32-bit pair holding this
    // lane's column (half c&1 of it): 16-bit ring registers get packed in
    // pairs by the compiler, and the packing waits for loads just issued.
    uint32_t rs[P][NT][GPT], rd[P][NT][GPT];
    const int sh = 16 * (c & 1);
    auto load = [&](int kt, uint4v (&a)[MT * 4], uint4v (&w)[NT], uint32_t (&sv)[NT][GPT],
                    uint32_t (&dv)[NT][GPT]) {
#pragma unroll
        for (int j = 0; j < MT * 4; ++j) a[j] = asrc[j][kt * (KTILE / 8)];
#pragma unroll
        for (int t = 0; t < NT; ++t) w[t] = wbase[((size_t)trel(t) * KT + kt) * 64];
        const int gi = (kt * KTILE) / g;
        const uint32_t *srow = reinterpret_cast<const uint32_t *>(S + (size_t)gi * N + (col0 & ~1));
#pragma unroll
        for (int t = 0; t < NT; ++t)
#pragma unroll
            for (int q = 0; q < GPT; ++q) sv[t][q] = srow[(size_t)q * (N / 2) + 8 * trel(t)];
        if (DELTA) {
            const uint32_t *drow = reinterpret_cast<const uint32_t *>(D + (size_t)gi * N + (col0 & ~1));
#pragma unroll
            for (int t = 0; t < NT; ++t)
#pragma unroll
                for (int q = 0; q < GPT; ++q) dv[t][q] = drow[(size_t)q * (N / 2) + 8 * trel(t)];
        }
    };
    // Consuming a slot happens in two halves: `stage` moves the slot's
    // activations into LDS and splits its codes into MFMA operands, after which
    // the slot's registers are free and the refill can be issued; `finish`
    // then does the MFMAs and the per-group scaling while the refill is in
    // flight.
    struct Staged {
        CodeOps ops[NT];
        float s[NT][GPT], d[NT][GPT];
    };
    auto stage = [&](const uint4v (&ar)[MT * 4], const uint4v (&w)[NT], const uint32_t (&sv)[NT][GPT],
                     const uint32_t (&dv)[NT][GPT], Staged &st) {
        debug_stage_sync();
#pragma unroll
        for (int j = 0; j < MT * 4; ++j) *reinterpret_cast<uint4v *>(scratch + adst[j]) = ar[j];
#pragma unroll
        for (int t = 0; t < NT; ++t) {
            st.ops[t] = split_codes(w[t]);
#pragma unroll
            for (int q = 0; q < GPT; ++q) {
                st.s[t][q] = h2f((uint16_t)(sv[t][q] >> sh));
                st.d[t][q] = DELTA ? h2f((uint16_t)(dv[t][q] >> sh)) : 0.f;
            }
        }
    };
    auto finish = [&](const Staged &st) {
        half8 a[MT][4];
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
            const int r = 16 * mt + c;
#pragma unroll
            for (int o = 0; o < 4; ++o)
                a[mt][o] = *reinterpret_cast<const half8 *>(scratch + r * KTILE + 8 * ((4 * o + kq) ^ c));
        }
        if (GPT > 1) {
            // groups of 64 or 32: per group, its steps' products and sums
            constexpr int SPG = 4 / GPT;                  // MFMA steps per group
            float4v asg[MT][GPT];
#pragma unroll
            for (int mt = 0; mt < MT; ++mt)
#pragma unroll
                for (int q = 0; q < GPT; ++q) {
                    asg[mt][q] = mfma_f16(a[mt][SPG * q], ones, fzero);
                    if (SPG == 2) asg[mt][q] = mfma_f16(a[mt][SPG * q + 1], ones, asg[mt][q]);
                }
#pragma unroll
            for (int t = 0; t < NT; ++t) {
                const half8 op[4] = {st.ops[t].lo[0], st.ops[t].lo[1], st.ops[t].hi[0], st.ops[t].hi[1]};
#pragma unroll
                for (int mt = 0; mt < MT; ++mt)
#pragma unroll
                    for (int q = 0; q < GPT; ++q) {
                        float4v x = mfma_f16(a[mt][SPG * q], op[SPG * q], fzero);
                        if (SPG == 2) x = mfma_f16(a[mt][SPG * q + 1], op[SPG * q + 1], x);
                        const float sq = st.s[t][q];
                        // steps 0, 1: low nibbles (2^-24 v); 2, 3: high ones (2^-20 v)
                        const float cx = sq * (SPG * q < 2 ? 0x1p24f : 0x1p20f);
                        const float c2 = DELTA ? (st.d[t][q] - 8.0f * sq) : (-8.0f * sq);
#pragma unroll
                        for (int r = 0; r < 4; ++r) {
                            const float v = __builtin_fmaf(cx, x[r], acc[mt][t][r]);
                            acc[mt][t][r] = __builtin_fmaf(c2, asg[mt][q][r], v);
                        }
                    }
            }
            return;
        }
        float4v as[MT];
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
            float4v y = mfma_f16(a[mt][0], ones, fzero);
            y = mfma_f16(a[mt][1], ones, y);
            y = mfma_f16(a[mt][2], ones, y);
            as[mt] = mfma_f16(a[mt][3], ones, y);
        }
#pragma unroll
        for (int t = 0; t < NT; ++t) {
            const float s = st.s[t][0];
            const float c1 = s * 0x1p20f, c16 = s * 0x1p24f;
            const float c2 = DELTA ? (st.d[t][0] - 8.0f * s) : (-8.0f * s);
#pragma unroll
            for (int mt = 0; mt < MT; ++mt) {
                float4v xl = mfma_f16(a[mt][0], st.ops[t].lo[0], fzero);
                xl = mfma_f16(a[mt][1], st.ops[t].lo[1], xl);
                float4v xh = mfma_f16(a[mt][2], st.ops[t].hi[0], fzero);
                xh = mfma_f16(a[mt][3], st.ops[t].hi[1], xh);
                // sum_k A q = 2^24 xl + 2^20 xh (exact powers of two)
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    float v = __builtin_fmaf(c16, xl[r], acc[mt][t][r]);
                    v = __builtin_fmaf(c1, xh[r], v);
                    acc[mt][t][r] = __builtin_fmaf(c2, as[mt][r], v);
                }
            }
        }
    };

    if (n > 0) {
        const int last = kt_end - 1;
#pragma unroll
        for (int i = 0; i < P; ++i) {
            const int kt = kt_beg + i;
            load(kt < last ? kt : last, ra[i], rw[i], rs[i], rd[i]);
        }
        int j = 0;
        for (; j + P <= n; j += P) {
#pragma unroll
            for (int i = 0; i < P; ++i) {
                Staged st;
                stage(ra[i], rw[i], rs[i], rd[i], st);
                const int kt = kt_beg + j + i + P;
                load(kt < last ? kt : last, ra[i], rw[i], rs[i], rd[i]);
                finish(st);
                // A memory clobber between each refill and the loop's back
                // edge: without one, the compiler folds "phi(prologue load,
                // refill load)" of the last slot into a single load at the
                // top of the loop, right before its use, and that slot loses
                // its prefetch distance.  The scheduling barrier keeps the
                // next slot's work (and so its wait) out of this step.
                asm volatile("" ::: "memory");
                __builtin_amdgcn_sched_barrier(0);
            }
        }
#pragma unroll
        for (int i = 0; i < P - 1; ++i)
            if (j + i < n) {
                Staged st;
                stage(ra[i], rw[i], rs[i], rd[i], st);
                finish(st);
            }
    }

    // sum the waves' partial products through LDS (the scratch is dead now)
    __syncthreads();
    constexpr int E4 = MT * NT * 4;
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int t = 0; t < NT; ++t)
#pragma unroll
            for (int r = 0; r < 4; ++r)
                red[((size_t)wave * E4 + (mt * NT + t) * 4 + r) * 64 + lane] = acc[mt][t][r];
    __syncthreads();
    for (int idx = threadIdx.x; idx < E4 * 64; idx += blockDim.x) {
        const int e = idx >> 6, l = idx & 63;
        const int r = e & 3, t = (e >> 2) % NT, mt = (e >> 2) / NT;
        if (GATED && (t & 1)) continue;                   // an up tile: read with its gate
        float v = 0.f;
        for (int w = 0; w < nw; ++w) v += red[(size_t)w * E4 * 64 + idx];
        const int row = m0 + 16 * mt + 4 * (l >> 4) + r;
        if (row >= M) continue;
        if (GATED) {
            float u = 0.f;   // the up element of the same output: tile t + 1
            for (int w = 0; w < nw; ++w) u += red[(size_t)w * E4 * 64 + idx + 4 * 64];
            C[(size_t)row * (N / 2) + (pt0 + trel(t)) * NTILE + (l & 15)] = f2h(silu_mul(v, u));
        } else {
            C[(size_t)row * N + (nt0 + t) * NTILE + (l & 15)] = f2h(v);
        }
    }
}

template <int MT, int NT, int P, int NWMAX, bool DELTA, bool GATED, int GPT>
static hipError_t run_skinny(const SkinnyCfg &cf, const uint16_t *A, const uint32_t *W,
                             const uint16_t *S, const uint16_t *D, uint16_t *C, int M, int N,
                             int K, int g, hipStream_t st)
{
    dim3 grid((unsigned)(N / (NTILE * NT)), (unsigned)((M + 16 * MT - 1) / (16 * MT)));
    const size_t ring = (size_t)cf.nw * MT * 16 * KTILE * sizeof(uint16_t);
    const size_t sum = (size_t)cf.nw * MT * NT * 4 * 64 * sizeof(float);
    const size_t lds = ring > sum ? ring : sum;
    if (lds > 160 * 1024) return hipErrorInvalidConfiguration;
    if (cf.nw < 1 || cf.nw > NWMAX) return hipErrorInvalidConfiguration;
    hipLaunchKernelGGL((w4a16_skinny_kernel<MT, NT, P, NWMAX, DELTA, GATED, GPT>), grid, dim3(64 * cf.nw), lds,
                       st, A, reinterpret_cast<const uint4v *>(W), S, D, C, M, N, K, g, cf.nw);
    return hipGetLastError();
}


// Heuristic choice of the skinny configuration (also sizes the workspace).
SkinnyCfg skinny_config(int M, int N, int K)
{
    SkinnyCfg c;
    const int KT = K / KTILE, NT16 = N / NTILE;
    if (M <= 16) {
        c.MT = 1; c.NT = 2; c.P = 2;
    } else if (M <= 32) {
        c.MT = 2; c.NT = 4; c.P = 2;
    } else {
        c.MT = 4; c.NT = 2; c.P = 2;
    }
    const int nwmax = (c.MT == 1) ? 8 : 4;
    c.S = 1;
    const long blocks = (long)(NT16 / c.NT) * ((M + 16 * c.MT - 1) / (16 * c.MT));
    // about 2500-4500 waves (measured best on MI355X for the decode shapes),
    // each with at least 2 k-tiles
    c.nw = 1;
    while (c.nw < nwmax && blocks * c.nw * 2 <= 4608 && KT / (c.nw * 2) >= 2) c.nw *= 2;
    return c;
}

size_t w4a16_workspace_bytes(int M, int N, int K, int g)
{
    // the decode kernel's split-K counters and partial sums (decode-size
    // batches, M <= 80); the skinny and tiled kernels need none
    return decode_workspace_bytes(M, N, K, g);
}

template <bool DELTA, bool GATED, int GPT>
static hipError_t dispatch_skinny_g(const SkinnyCfg &c, const uint16_t *A, const uint32_t *W,
                                    const uint16_t *S, const uint16_t *D, uint16_t *C, int M,
                                    int N, int K, int g, hipStream_t st)
{
    if (c.S != 1) return hipErrorInvalidConfiguration;
#define QG_SK(MT_, NT_, P_, NWMAX_)                                                             \
    if (c.MT == MT_ && c.NT == NT_ && c.P == P_ && c.nw <= NWMAX_)                              \
        return run_skinny<MT_, NT_, P_, NWMAX_, DELTA, GATED, GPT>(c, A, W, S, D, C, M, N, K, g, st);
    QG_SK(1, 2, 2, 8) QG_SK(2, 4, 2, 4) QG_SK(4, 2, 2, 4)
#undef QG_SK
    return hipErrorInvalidConfiguration;
}

// groups per k-tile: 1 (g >= 128), 2 (g = 64), 4 (g = 32)
template <bool DELTA, bool GATED>
static hipError_t dispatch_skinny(const SkinnyCfg &c, const uint16_t *A, const uint32_t *W,
                                  const uint16_t *S, const uint16_t *D, uint16_t *C, int M, int N,
                                  int K, int g, hipStream_t st)
{
    if (g >= KTILE) return dispatch_skinny_g<DELTA, GATED, 1>(c, A, W, S, D, C, M, N, K, g, st);
    if (g == KTILE / 2) return dispatch_skinny_g<DELTA, GATED, 2>(c, A, W, S, D, C, M, N, K, g, st);
    if (g == KTILE / 4) return dispatch_skinny_g<DELTA, GATED, 4>(c, A, W, S, D, C, M, N, K, g, st);
    return hipErrorInvalidValue;
}

hipError_t launch_w4a16_skinny_cfg(const SkinnyCfg &c, const uint16_t *A, const uint32_t *W,
                                   const uint16_t *S, const uint16_t *D, uint16_t *C, int M,
                                   int N, int K, int g, bool fuse_delta, void *ws,
                                   hipStream_t st, bool gated)
{
    (void)ws;
    const bool dl = D && fuse_delta;
    if (gated)
        return dl ? dispatch_skinny<true, true>(c, A, W, S, D, C, M, N, K, g, st)
                  : dispatch_skinny<false, true>(c, A, W, S, nullptr, C, M, N, K, g, st);
    return dl ? dispatch_skinny<true, false>(c, A, W, S, D, C, M, N, K, g, st)
              : dispatch_skinny<false, false>(c, A, W, S, nullptr, C, M, N, K, g, st);
}

hipError_t launch_w4a16(const uint16_t *A, const uint32_t *W, const uint16_t *S,
                        const uint16_t *D, uint16_t *C, int M, int N, int K, int g,
                        bool fuse_delta, void *ws, hipStream_t st)
{
    if (M >= TILED_MIN_M) return launch_w4a16_tiled(A, W, S, D, C, M, N, K, g, fuse_delta, st);
    if (use_decode_kernel(M, N, K, g))
        return launch_w4a16_decode(A, W, S, D, C, M, N, K, g, fuse_delta,
                                   decode_workspace_bytes(M, N, K, g) ? decode_splits(N, K, g) : 1, ws,
                                   st);
    return launch_w4a16_skinny_cfg(skinny_config(M, N, K), A, W, S, D, C, M, N, K, g,
                                   fuse_delta, ws, st);
}

// The kernels launch_w4a16 / launch_w4a16_swiglu run for a shape (K and N
// multiples of 128), in words, for the first-dispatch log line.
static const char *big_kernel(int M, int N, int K, int g, bool delta)
{
    if (g < KTILE) {
        if (g == KTILE / 2 && tiled_config(M, N) == 0 && use_mid2(M, N, K))
            return "mid 64x128 (K split in the workgroup)";
        return tiled_config(M, N) == 2 ? "tiled 128x256" : "tiled 64x128";
    }
    switch (tiled_config(M, N)) {
    case 0: return use_mid2(M, N, K) ? "mid 64x128 (K split in the workgroup)" : "mid 64x64";
    case 1: return "tiled 64x128";
    default: return delta ? "tiled 128x256" : "tiled 128x256 symmetric";
    }
}

void describe_w4a16(int M, int N, int K, int g, bool delta, bool gated, char *buf, size_t n)
{
    const int N2 = gated ? 2 * N : N;
    const char *gate = gated ? "gated " : "";
    if (gated ? swiglu_uses_decode(M, N, K, g) : (M < TILED_MIN_M && use_decode_kernel(M, N, K, g))) {
        snprintf(buf, n, "%sdecode, %d K-split(s)", gate,
                 decode_workspace_bytes(M, N2, K, g) ? decode_splits(N2, K, g) : 1);
    } else if (M < TILED_MIN_M) {
        snprintf(buf, n, "%sskinny", gate);
    } else if (tiled_config(M, N2) == 2 && tiled_row_split(M, N2) < M &&
               tiled_col_split(M, N2, g, gated) < N2) {
        const int n1 = tiled_col_split(M, N2, g, gated);
        snprintf(buf, n, "%s columns 0-%d, tiled 64x128 columns %d-%d",
                 big_kernel(M, n1, K, g, delta), n1 - 1, n1, N2 - 1);
    } else if (tiled_config(M, N2) == 2 && tiled_row_split(M, N2) < M) {
        const int m1 = tiled_row_split(M, N2);
        snprintf(buf, n, "%s%s rows 0-%d, %s rows %d-%d", gate, big_kernel(m1, N2, K, g, delta), m1 - 1,
                 big_kernel(M - m1, N2, K, g, delta), m1, M - 1);
    } else {
        snprintf(buf, n, "%s%s", gate, big_kernel(M, N2, K, g, delta));
    }
}

// ---- shapes with tails: K or N not a multiple of 128 (the pages' dispatcher
//      requires both; "Gaps and follow-ups" lists the head projection's N
//      as the gap) ----
// The pack pads the weight to [Kp, Np] (codes 8, scales 0); a call copies A
// into the workspace with zero columns up to Kp, runs the GEMM on the padded
// shape, and crops the padded product to C (the decode kernel instead stores
// C's logical columns directly).  All in the workspace after the counter
// region: [counters | GEMM workspace][A padded][C padded].
__global__ __launch_bounds__(256) void pad_cols_kernel(const uint16_t *__restrict__ A,
                                                       uint16_t *__restrict__ Ap, int M, int K,
                                                       int Kp)
{
    const size_t i = (size_t)blockIdx.x * 256 + threadIdx.x;
    if (i >= (size_t)M * Kp) return;
    const size_t m = i / Kp;
    const int k = (int)(i % Kp);
    Ap[i] = k < K ? A[m * K + k] : (uint16_t)0;
}

__global__ __launch_bounds__(256) void crop_cols_kernel(const uint16_t *__restrict__ Cp,
                                                        uint16_t *__restrict__ C, int M, int N,
                                                        int Np)
{
    const size_t i = (size_t)blockIdx.x * 256 + threadIdx.x;
    if (i >= (size_t)M * N) return;
    const size_t m = i / N;
    const int n = (int)(i % N);
    C[i] = Cp[m * Np + n];
}

static size_t al256(size_t n) { return (n + 255) / 256 * 256; }

hipError_t launch_crop_cols(const uint16_t *Cp, uint16_t *C, int M, int N, int Np, hipStream_t st)
{
    const size_t n = (size_t)M * N;
    hipLaunchKernelGGL(crop_cols_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st, Cp, C,
                       M, N, Np);
    return hipGetLastError();
}

bool is_tail_shape(int N, int K, int g)
{
    int Kp, Np, gp;
    padded_shape(K, N, g, &Kp, &Np, &gp);
    return Kp != K || Np != N;
}

size_t tail_workspace_bytes(int M, int N, int K, int g)
{
    int Kp, Np, gp;
    padded_shape(K, N, g, &Kp, &Np, &gp);
    const size_t gemm = w4a16_workspace_bytes(M, Np, Kp, gp);
    size_t off = al256(gemm > W4A16_WS_COUNTER_BYTES ? gemm : W4A16_WS_COUNTER_BYTES);
    if (Kp != K) off += al256((size_t)M * Kp * sizeof(uint16_t));
    if (Np != N) off += (size_t)M * Np * sizeof(uint16_t);
    return off;
}

hipError_t launch_w4a16_tail(const uint16_t *A, const uint32_t *W, const uint16_t *S,
                             const uint16_t *D, uint16_t *C, int M, int N, int K, int g,
                             bool fuse_delta, void *ws, hipStream_t st)
{
    if (!ws) return hipErrorInvalidValue;
    int Kp, Np, gp;
    padded_shape(K, N, g, &Kp, &Np, &gp);
    const size_t gemm = w4a16_workspace_bytes(M, Np, Kp, gp);
    char *p = static_cast<char *>(ws) + al256(gemm > W4A16_WS_COUNTER_BYTES ? gemm : W4A16_WS_COUNTER_BYTES);
    const uint16_t *Ause = A;
    if (Kp != K) {
        uint16_t *Ap = reinterpret_cast<uint16_t *>(p);
        p += al256((size_t)M * Kp * sizeof(uint16_t));
        const size_t n = (size_t)M * Kp;
        hipLaunchKernelGGL(pad_cols_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st, A,
                           Ap, M, K, Kp);
        Ause = Ap;
    }
    if (Np != N && M < TILED_MIN_M && use_decode_kernel(M, Np, Kp, gp)) {
        // the decode kernel stores the logical columns straight into C (no
        // padded product, no crop)
        const int ns = decode_workspace_bytes(M, Np, Kp, gp) ? decode_splits(Np, Kp, gp) : 1;
        hipError_t e = launch_w4a16_decode(Ause, W, S, D, C, M, Np, Kp, gp, fuse_delta, ns,
                                           gemm ? ws : nullptr, st, false, N, N);
        if (e != hipSuccess) return e;
        return hipGetLastError();
    }
    uint16_t *Cuse = Np != N ? reinterpret_cast<uint16_t *>(p) : C;
    hipError_t e = launch_w4a16(Ause, W, S, D, Cuse, M, Np, Kp, gp, fuse_delta, gemm ? ws : nullptr, st);
    if (e != hipSuccess) return e;
    if (Np != N) {
        const size_t n = (size_t)M * N;
        hipLaunchKernelGGL(crop_cols_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st, Cuse,
                           C, M, N, Np);
    }
    return hipGetLastError();
}

// ---- SwiGLU of a gate/up pair ("Gaps and follow-ups": mlp_gate and mlp_up
//      in one kernel) ----
// The pair is one packed [K, 2N] weight, gate columns first.  Every batch
// runs one launch whose kernel holds the gate and the up product of the same
// output columns in fp32 and stores silu(gate) * up once: the gated decode
// kernel (M <= 80 where it is chosen), otherwise the skinny, mid or tiled
// kernel with the gated epilogue (gated_tile pairs their n-tiles).

bool swiglu_uses_decode(int M, int N, int K, int g) { return use_decode_kernel(M, 2 * N, K, g); }

size_t swiglu_workspace_bytes(int M, int N, int K, int g)
{
    // only the decode kernel's split-K needs a workspace
    return swiglu_uses_decode(M, N, K, g) ? decode_workspace_bytes(M, 2 * N, K, g) : 0;
}

hipError_t launch_w4a16_swiglu(const uint16_t *A, const uint32_t *W, const uint16_t *S,
                               const uint16_t *D, uint16_t *H, int M, int N, int K, int g,
                               void *ws, hipStream_t st)
{
    const int N2 = 2 * N;
    if (swiglu_uses_decode(M, N, K, g)) {
        const int ns = decode_workspace_bytes(M, N2, K, g) ? decode_splits(N2, K, g) : 1;
        if (ns > 1 && !ws) return hipErrorInvalidValue;
        return launch_w4a16_decode(A, W, S, D, H, M, N2, K, g, true, ns, ws, st, true);
    }
    if (M >= TILED_MIN_M) return launch_w4a16_tiled(A, W, S, D, H, M, N2, K, g, true, st, true);
    return launch_w4a16_skinny_cfg(skinny_config(M, N2, K), A, W, S, D, H, M, N2, K, g, true,
                                   nullptr, st, true);
}

// ---- two-stage correction ("The pipeline, end to end": a_group_sum then
//      correction_accum) ----
// Stage 1: one wave per (row, group); lanes sum a strided slice in fp32 and
// the wave combines them with butterfly shuffles.
__global__ __launch_bounds__(64) void group_sum_kernel(const uint16_t *__restrict__ A, int K,
                                                       int g, int G, float *__restrict__ a_sum)
{
    const int cell = blockIdx.x;          // m * G + gi
    const int m = cell / G, gi = cell % G;
    const uint16_t *p = A + (size_t)m * K + (size_t)gi * g;
    float v = 0.f;
    for (int k = threadIdx.x; k < g; k += 64) v += h2f(p[k]);
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off, 64);
    if (threadIdx.x == 0) a_sum[cell] = v;
}

// Stage 2: C += sum_g a_sum[m,g] * delta[g,n].  A workgroup (one wave)
// takes 64 consecutive columns (one per lane) and R rows: each delta value is
// read once and applied to all R rows.  The rows' group sums, the same for
// every lane, are staged in LDS 64 groups at a time (coalesced loads) and read
// back four groups per 16-byte broadcast read.  Per output the sum runs over
// g in order, one fma each.  R = 16 for large M (delta re-read M/16 times),
// 4 below M = 256 (four times the waves for the same columns).
template <int R>
__global__ __launch_bounds__(64) void correction_accum_kernel(const float *__restrict__ a_sum,
                                                              const uint16_t *__restrict__ D,
                                                              uint16_t *__restrict__ C, int M,
                                                              int N, int G)
{
    constexpr int GCH = 64;                       // groups per LDS chunk
    __shared__ __attribute__((aligned(16))) float sa[R][GCH];
    const int lane = threadIdx.x;
    const int n = blockIdx.x * 64 + lane;
    const int m0 = blockIdx.y * R;
    const int rows = M - m0 < R ? M - m0 : R;
    const bool col_ok = n < N;                    // (every lane reaches the barriers)
    float corr[R];
#pragma unroll
    for (int r = 0; r < R; ++r) corr[r] = 0.f;
    for (int g0 = 0; g0 < G; g0 += GCH) {
        const int gn = G - g0 < GCH ? G - g0 : GCH;
        __syncthreads();                          // the previous chunk's reads are done
        for (int i = lane; i < R * GCH; i += 64) {
            const int r = i / GCH, gg = i % GCH;
            sa[r][gg] = (r < rows && gg < gn) ? a_sum[(size_t)(m0 + r) * G + g0 + gg] : 0.f;
        }
        __syncthreads();
        if (!col_ok) continue;
        int gg = 0;
        for (; gg + 4 <= gn; gg += 4) {
            float d[4];
#pragma unroll
            for (int u = 0; u < 4; ++u) d[u] = h2f(D[(size_t)(g0 + gg + u) * N + n]);
#pragma unroll
            for (int r = 0; r < R; ++r) {
                const float4v a4 = *reinterpret_cast<const float4v *>(&sa[r][gg]);
#pragma unroll
                for (int u = 0; u < 4; ++u)
                    if (r < rows) corr[r] = __builtin_fmaf(a4[u], d[u], corr[r]);
            }
        }
        for (; gg < gn; ++gg) {
            const float d = h2f(D[(size_t)(g0 + gg) * N + n]);
#pragma unroll
            for (int r = 0; r < R; ++r)
                if (r < rows) corr[r] = __builtin_fmaf(sa[r][gg], d, corr[r]);
        }
    }
    if (!col_ok) return;
#pragma unroll
    for (int r = 0; r < R; ++r)
        if (r < rows) {
            uint16_t *cp = C + (size_t)(m0 + r) * N + n;
            *cp = f2h(h2f(*cp) + corr[r]);
        }
}

hipError_t launch_group_sum_correction(const uint16_t *A, const uint16_t *D, uint16_t *C,
                                       int M, int N, int K, int g, float *a_sum,
                                       hipStream_t st)
{
    const int G = K / g;
    hipLaunchKernelGGL(group_sum_kernel, dim3((unsigned)((size_t)M * G)), dim3(64), 0, st, A, K,
                       g, G, a_sum);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    if (M >= 256)
        hipLaunchKernelGGL(correction_accum_kernel<16>, dim3((unsigned)((N + 63) / 64), (unsigned)((M + 15) / 16)),
                           dim3(64), 0, st, a_sum, D, C, M, N, G);
    else
        hipLaunchKernelGGL(correction_accum_kernel<4>, dim3((unsigned)((N + 63) / 64), (unsigned)((M + 3) / 4)),
                           dim3(64), 0, st, a_sum, D, C, M, N, G);
    return hipGetLastError();
}

} // namespace qg
