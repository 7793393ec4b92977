// W4A16 mid-batch kernels (64 x 64 tiles; 64 x 128 tiles with K split inside
// the workgroup).  Codes as exact fp16 subnormals, scale and delta applied
// once per weight group on the fp32 accumulators ("Marlin INT4 on Ada - how
// it works", "The core mismatch: symmetric vs asymmetric").
#include "qg_device.h"
#include "qg_launch.h"

#include <atomic>
#include <type_traits>

namespace qg {

// ---- mid kernel (mid-size M) ----
// Workgroup tile 64 rows x 64 columns, 4 waves in a 2 x 2 arrangement: wave
// (mw, nw) owns rows 32 mw .. 32 mw + 31 (2 m-tiles) and columns
// 32 nw .. 32 nw + 31 (2 n-tiles).  Small tiles keep two or more waves per
// SIMD at mid-size M, where one wave per SIMD left every LDS and memory
// latency exposed.  The arithmetic is the decode kernel's: codes enter the
// MFMAs as exact fp16 subnormals (no per-element dequantization, which would
// otherwise cost more VALU than the MFMAs take), the group sums of A come from
// MFMAs against an all-ones operand, and scale and delta are applied on the
// fp32 accumulators -- once per weight group: the MFMAs accumulate a group's
// raw sums (low-nibble, high-nibble and activation sums apart) across its
// k-tiles, so a group of 2 k-tiles (g = 256) costs half the scaling FMAs of
// per-k-tile scaling and one group over all of K (g = K) almost none (the
// loop is issue-bound: 24 MFMAs against ~110 VALU instructions per k-tile and
// wave with per-k-tile scaling).  GK selects the form: 1 = every k-tile is
// scaled on its own (g = 128), 3 = likewise for any other g, 2 = groups of
// two k-tiles (g = 256), 0 = one group (g = K); the forms also fix how a
// k-tile finds its group row (none, the k-tile itself, a shift; a division
// only for form 3).  Pipeline: MID_STAGES k-tiles in flight.
// A k-tile of A (64 rows, 16 KB) goes straight from global memory to one of
// MID_STAGES LDS buffers (wave w fills rows 16w .. 16w + 15; 16-byte chunk ch
// of row r lands at position ch ^ (r % 16)); codes, scales and deltas of the
// same k-tile go to the matching slot of a register ring.  Each k-tile starts
// with a wait that leaves the later k-tiles' loads in flight and one barrier,
// after which the slot used by the previous k-tile is refilled.
constexpr int MID_STAGES = 4;

// The weight group of k-tile k in form GK (see above).
template <int GK>
__device__ inline int mid_group(int k, int g)
{
    return GK == 0 ? 0 : GK == 1 ? k : GK == 2 ? (k >> 1) : GK == 4 ? 2 * k : (k * KTILE) / g;
}

template <int SG, bool DELTA, int GK, bool GATED>
__global__ __launch_bounds__(256, 2) void w4a16_mid_kernel(
    const uint16_t *__restrict__ A, const uint4v *__restrict__ W, const uint16_t *__restrict__ S,
    const uint16_t *__restrict__ D, uint16_t *__restrict__ C, int M, int N, int K, int g)
{
    constexpr int WM = 2, WN = 2, BM = 64, BN = 64;
    constexpr int L = 4 + WN + WN + (DELTA ? WN : 0);     // loads per thread and k-tile
    static_assert((SG - 2) * L < 64, "vmcnt holds 6 bits");
    extern __shared__ __attribute__((aligned(16))) _Float16 Asm[];   // [SG][BM * KTILE]

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int mw = wave >> 1, nw = wave & 1;
    const int c = lane & 15, kq = lane >> 4;
    const int KT = K / KTILE;
    const int m0 = blockIdx.y * BM;
    const int ntile0 = blockIdx.x * (BN / NTILE) + WN * nw;
    const int col0 = ntile0 * NTILE + c;
    const int sh = 16 * (c & 1);
    // GATED: the wave's two (virtual) n-tiles are the gate tile ntile0 / 2
    // and the up tile N / 32 + ntile0 / 2 of the [K, N] pair weight; each
    // takes its own resources (parity p of n-tile t = t & 1)
    const int Nh16 = N / (2 * NTILE);
    auto pbase = [&](int p) { return GATED ? gated_tile(ntile0, p, Nh16) : ntile0; };

    // Every load below is a buffer load: a workgroup-uniform resource (base
    // address), a fixed per-lane byte offset and the k-dependent byte offset
    // in a scalar register, so the k-loop does no per-lane address arithmetic.
    // The ranges cover the arrays from each base to their end.
    // A: direct global -> LDS loads, one wave instruction fills 1 KB = 4 rows;
    // rows past M read row M-1 (their results are never stored)
    const __amdgpu_buffer_rsrc_t a_rs = buffer_rsrc(A + (size_t)m0 * K, (size_t)(M - m0) * K * 2);
    unsigned a_off[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int r = (wave * 4 + i) * 4 + (lane >> 4);
        const int ch = (lane & 15) ^ (r & 15);
        const int row = m0 + r < M ? r : M - 1 - m0;
        a_off[i] = (unsigned)(row * K + ch * 8) * 2u;
    }
    auto load_a = [&](int kt, int st) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int blk = wave * 4 + i;
            __builtin_amdgcn_raw_ptr_buffer_load_lds(
                a_rs, (__attribute__((address_space(3))) void *)(Asm + st * BM * KTILE + blk * 4 * KTILE), 16,
                a_off[i], kt * KTILE * 2, 0, 0);
        }
    };
    // (plain variables of a fixed type: a target builtin given an argument
    // whose type depends on a template parameter loses the kernel's host
    // launch stub)
    const int pt0 = pbase(0), pt1 = pbase(1);
    const __amdgpu_buffer_rsrc_t w_rs0 = buffer_rsrc(W + (size_t)pt0 * KT * 64, (size_t)(N / NTILE - pt0) * KT * 1024);
    const __amdgpu_buffer_rsrc_t w_rs1 = buffer_rsrc(W + (size_t)pt1 * KT * 64, (size_t)(N / NTILE - pt1) * KT * 1024);
    const __amdgpu_buffer_rsrc_t s_rs0 = buffer_rsrc(S + pt0 * NTILE, ((size_t)(K / g) * N - pt0 * NTILE) * 2);
    const __amdgpu_buffer_rsrc_t s_rs1 = buffer_rsrc(S + pt1 * NTILE, ((size_t)(K / g) * N - pt1 * NTILE) * 2);
    const __amdgpu_buffer_rsrc_t d_rs0 = buffer_rsrc(DELTA ? D + pt0 * NTILE : S, DELTA ? ((size_t)(K / g) * N - pt0 * NTILE) * 2 : 4);
    const __amdgpu_buffer_rsrc_t d_rs1 = buffer_rsrc(DELTA ? D + pt1 * NTILE : S, DELTA ? ((size_t)(K / g) * N - pt1 * NTILE) * 2 : 4);
    // n-tile t: the up resources at tile 0 for odd t (GATED), else the first
    // resources at tile t
    auto odd = [](int t) { return GATED && (t & 1); };
    auto rel = [](int t) { return GATED ? 0 : t; };
    uint4v rw[SG][WN];
    uint32_t rs[SG][WN], rd[SG][WN];   // aligned scale / delta pairs (half c & 1)
    const unsigned w_off = (unsigned)lane * 16u;      // this lane's 16 bytes of a code tile
    const unsigned s_off = ((unsigned)c >> 1) * 4u;   // this lane's scale pair within 16 columns
    // every load of k-tile kt (clamped: the count per k-tile is fixed, which
    // the waits rely on)
    auto load = [&](int kt, int slot) {
        const int k = kt < KT ? kt : KT - 1;
        load_a(k, slot);
#pragma unroll
        for (int t = 0; t < WN; ++t) {
            const __amdgpu_buffer_rsrc_t wr = odd(t) ? w_rs1 : w_rs0;
            const int wo = (rel(t) * KT + k) * 1024;
            rw[slot][t] = __builtin_bit_cast(uint4v, __builtin_amdgcn_raw_buffer_load_b128(wr, w_off, wo, 0));
        }
        // byte offset of this k-tile's group row (opaque: one load per k-tile)
        const int gb = opaque_s(mid_group<GK>(k, g) * N * 2);
#pragma unroll
        for (int t = 0; t < WN; ++t) {
            const __amdgpu_buffer_rsrc_t sr = odd(t) ? s_rs1 : s_rs0;
            const int so = gb + 32 * rel(t);
            rs[slot][t] = __builtin_amdgcn_raw_buffer_load_b32(sr, s_off, so, 0);
        }
        if (DELTA) {
#pragma unroll
            for (int t = 0; t < WN; ++t) {
                const __amdgpu_buffer_rsrc_t dr = odd(t) ? d_rs1 : d_rs0;
                const int so = gb + 32 * rel(t);
                rd[slot][t] = __builtin_amdgcn_raw_buffer_load_b32(dr, s_off, so, 0);
            }
        }
    };

    // fp32 accumulators, and the raw sums of the current weight group (codes
    // as subnormals, low and high nibbles apart, and the activation sums);
    // the group's scale and delta are applied once, at its last k-tile
    float4v acc[WM][WN], xl[WM][WN], xh[WM][WN], asum[WM];
    const half8 ones = {1, 1, 1, 1, 1, 1, 1, 1};
    const float4v fzero = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int mt = 0; mt < WM; ++mt) {
        asum[mt] = fzero;
#pragma unroll
        for (int t = 0; t < WN; ++t) acc[mt][t] = xl[mt][t] = xh[mt][t] = fzero;
    }
    int kt_ = 0;   // the k-tile being computed

    // the group constants of the slot being computed (converted at every
    // k-tile, used at a group's last: every slot's registers are then
    // consumed at the same point of its step, which keeps the compiler's load
    // tracking exact)
    float k16[WN], k1[WN], k2[WN];
    // first: this k-tile starts its weight group (the raw sums restart)
    auto compute = [&](int slot, bool first) {
#pragma unroll
        for (int t = 0; t < WN; ++t) {
            const float s = h2f((uint16_t)(rs[slot][t] >> sh));
            const float d = DELTA ? h2f((uint16_t)(rd[slot][t] >> sh)) : 0.f;
            k16[t] = s * 0x1p24f;
            k1[t] = s * 0x1p20f;
            k2[t] = DELTA ? (d - 8.0f * s) : (-8.0f * s);
            pin(k16[t]); pin(k1[t]); pin(k2[t]);
        }
        load(kt_ + SG - 1, (slot + SG - 1) % SG);
        const _Float16 *as = Asm + slot * BM * KTILE;
#pragma unroll
        for (int mt = 0; mt < WM; ++mt) {
            const int r = 32 * mw + 16 * mt + c;
            half8 a[4];
#pragma unroll
            for (int o = 0; o < 4; ++o)
                a[o] = *reinterpret_cast<const half8 *>(as + r * KTILE + 8 * ((4 * o + kq) ^ c));
            asum[mt] = mfma_f16(a[0], ones, first ? fzero : asum[mt]);
            asum[mt] = mfma_f16(a[1], ones, asum[mt]);
            asum[mt] = mfma_f16(a[2], ones, asum[mt]);
            asum[mt] = mfma_f16(a[3], ones, asum[mt]);
#pragma unroll
            for (int t = 0; t < WN; ++t) {
                const CodeOps ops = split_codes(rw[slot][t]);
                xl[mt][t] = mfma_f16(a[0], ops.lo[0], first ? fzero : xl[mt][t]);
                xl[mt][t] = mfma_f16(a[1], ops.lo[1], xl[mt][t]);
                xh[mt][t] = mfma_f16(a[2], ops.hi[0], first ? fzero : xh[mt][t]);
                xh[mt][t] = mfma_f16(a[3], ops.hi[1], xh[mt][t]);
            }
        }
    };
    // end of a weight group: scale and delta applied to its raw sums
    auto apply = [&](bool clear) {
#pragma unroll
        for (int mt = 0; mt < WM; ++mt) {
#pragma unroll
            for (int t = 0; t < WN; ++t) {
#pragma unroll
                for (int r4 = 0; r4 < 4; ++r4) {
                    float v = __builtin_fmaf(k16[t], xl[mt][t][r4], acc[mt][t][r4]);
                    v = __builtin_fmaf(k1[t], xh[mt][t][r4], v);
                    acc[mt][t][r4] = __builtin_fmaf(k2[t], asum[mt][r4], v);
                }
                if (clear) xl[mt][t] = xh[mt][t] = fzero;
            }
            if (clear) asum[mt] = fzero;
        }
    };
    // tail: a step after the main loop.  Its loads (k-tiles past the end) are
    // never read, so the compiler keeps only the direct-to-LDS ones and fewer
    // than L follow each k-tile's loads there: those steps wait for every load
    // in flight instead of counting.
    auto step = [&](int kt, int slot, bool tail) {
        constexpr unsigned WAIT = waitcnt_vm((SG - 2) * L);
        if (tail)
            __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));
        else
            __builtin_amdgcn_s_waitcnt(WAIT);
        debug_stage_sync();
        asm volatile("" ::: "memory");
        __builtin_amdgcn_s_barrier();
        asm volatile("" ::: "memory");
        // nothing that reads this slot's registers moves above the wait
        __builtin_amdgcn_sched_barrier(0);
        kt_ = kt;
        if (GK == 1 || GK == 3) {
            compute(slot, true);
            apply(false);
        } else if (GK == 2) {
            // k-tiles come in slot order from a multiple of SG (even)
            compute(slot, (slot & 1) == 0);
            if (slot & 1) apply(false);
        } else {
            // GK == 0, one group over all of K: the raw sums start at zero
            // and are applied once, after the loop
            compute(slot, false);
        }
    };

#pragma unroll
    for (int i = 0; i < SG - 1; ++i) {
        load(i, i);
        __builtin_amdgcn_sched_barrier(0);   // k-tile by k-tile, as the loop refills
    }
    int kt = 0;
    for (; kt + SG <= KT; kt += SG) {
#pragma unroll
        for (int i = 0; i < SG; ++i) {
            step(kt + i, i, false);
            asm volatile("" ::: "memory");
            __builtin_amdgcn_sched_barrier(0);
        }
    }
#pragma unroll
    for (int i = 0; i < SG - 1; ++i)
        if (kt + i < KT) step(kt + i, i, true);
    if (GK == 0) apply(false);   // the single group (g = K) ends with the last k-tile
    __builtin_amdgcn_s_waitcnt(0);   // the last (unused) loads

#pragma unroll
    for (int mt = 0; mt < WM; ++mt)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int row = m0 + 32 * mw + 16 * mt + 4 * kq + r;
            if (row >= M) continue;
            if (GATED) {
                C[(size_t)row * (N / 2) + pbase(0) * NTILE + c] = f2h(silu_mul(acc[mt][0][r], acc[mt][1][r]));
            } else {
#pragma unroll
                for (int t = 0; t < WN; ++t) C[(size_t)row * N + col0 + 16 * t] = f2h(acc[mt][t][r]);
            }
        }
}

// ---- mid kernel with the K range split inside the workgroup (mid-size M
//      on wide N) ----
// Workgroup 64 rows x 128 columns, 8 waves: k-group kg = wave / 4 takes the
// k-tiles of one half of K, and wave wn = wave % 4 of it owns all 64 rows (4
// m-tiles) and columns 32 wn .. 32 wn + 31 (2 n-tiles).  Against the 2 x 2
// layout of the 64 x 64 kernel, every code word is split once for 4 m-tiles
// instead of twice for 2, and the group sums of A are taken once per k-group
// -- wave wn sums m-tile wn and shares the sums through LDS -- instead of
// twice; the two halves are added through LDS at the end.  Scale and delta
// are applied per weight group as in the 64 x 64 kernel (GK), except that
// the delta term, which needs the other waves' group sums, is added one
// k-tile after the group's end, once the next barrier has made those sums
// visible: acc += k16 xl + k1 xh at the end of the group, acc += k2 a_sum a
// k-tile later.  The LDS ring holds both k-groups' activation tiles of
// MID2_STAGES k-tile steps (one wait and one barrier per step).
constexpr int MID2_STAGES = 4;

template <int SG, bool DELTA, int GK, bool GATED>
__global__ __launch_bounds__(512) void w4a16_mid2_kernel(
    const uint16_t *__restrict__ A, const uint4v *__restrict__ W, const uint16_t *__restrict__ S,
    const uint16_t *__restrict__ D, uint16_t *__restrict__ C, int M, int N, int K, int g)
{
    constexpr int WM = 4, WN = 2, BM = 64;
    constexpr int NS = GK == 4 ? 2 : 1;                    // weight groups per k-tile
    constexpr int L = 4 + WN + NS * WN + (DELTA ? NS * WN : 0);   // loads per thread and step
    static_assert((SG - 2) * L < 64, "vmcnt holds 6 bits");
    static_assert(SG % 4 == 0, "group parities follow the ring slot");
    // LDS: the ring [SG][2 k-groups][BM * KTILE] fp16, then the group sums
    // shared within a k-group [2 k-groups][2 parities][NS][BM] fp32
    extern __shared__ __attribute__((aligned(16))) _Float16 Asm[];
    float *gx = reinterpret_cast<float *>(Asm + (size_t)SG * 2 * BM * KTILE);

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int kg = wave >> 2, wn = wave & 3;
    const int c = lane & 15, kq = lane >> 4;
    const int KT = K / KTILE;
    // half 0 takes KH k-tiles (whole two-k-tile groups when GK == 2), half 1
    // the rest; a k-group past its range reloads its last tile and computes
    // nothing (an empty half, K = 128: tile 0)
    const int KH = GK == 2 ? ((KT / 2 + 1) / 2) * 2 : (KT + 1) / 2;
    const int kbeg = kg ? KH : 0, kn = kg ? KT - KH : KH;
    const int klast = kn > 0 ? kbeg + kn - 1 : 0;
    const int m0 = blockIdx.y * BM;
    const int ntile0 = blockIdx.x * (4 * WN) + WN * wn;
    const int col0 = ntile0 * NTILE + c;
    const int sh = 16 * (c & 1);
    // GATED: the wave's two (virtual) n-tiles are a gate tile and its up tile
    const int Nh16 = N / (2 * NTILE);
    const int pt0 = GATED ? gated_tile(ntile0, 0, Nh16) : ntile0;
    const int pt1 = GATED ? gated_tile(ntile0, 1, Nh16) : ntile0;
    auto odd = [](int t) { return GATED && (t & 1); };
    auto rel = [](int t) { return GATED ? 0 : t; };

    // A: direct global -> LDS loads; wave wn of k-group kg fills rows
    // 16 wn .. 16 wn + 15 of the k-group's tile (4 blocks of 4 rows); rows
    // past M read row M-1 (their results are never stored)
    const __amdgpu_buffer_rsrc_t a_rs = buffer_rsrc(A + (size_t)m0 * K, (size_t)(M - m0) * K * 2);
    unsigned a_off[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int r = (wn * 4 + i) * 4 + (lane >> 4);
        const int ch = (lane & 15) ^ (r & 15);
        const int row = m0 + r < M ? r : M - 1 - m0;
        a_off[i] = (unsigned)(row * K + ch * 8) * 2u;
    }
    auto load_a = [&](int kt, int slot) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            __attribute__((address_space(3))) void *dst = (__attribute__((address_space(3))) void *)(
                Asm + (size_t)(slot * 2 + kg) * BM * KTILE + (wn * 4 + i) * 4 * KTILE);
            const unsigned off = a_off[i];
            __builtin_amdgcn_raw_ptr_buffer_load_lds(a_rs, dst, 16, off, kt * KTILE * 2, 0, 0);
        }
    };
    // (resources in plain variables: a target builtin given an argument whose
    // type depends on a template parameter loses the kernel's host launch stub)
    const __amdgpu_buffer_rsrc_t w_rs0 = buffer_rsrc(W + (size_t)pt0 * KT * 64, (size_t)(N / NTILE - pt0) * KT * 1024);
    const __amdgpu_buffer_rsrc_t w_rs1 = buffer_rsrc(W + (size_t)pt1 * KT * 64, (size_t)(N / NTILE - pt1) * KT * 1024);
    const __amdgpu_buffer_rsrc_t s_rs0 = buffer_rsrc(S + pt0 * NTILE, ((size_t)(K / g) * N - pt0 * NTILE) * 2);
    const __amdgpu_buffer_rsrc_t s_rs1 = buffer_rsrc(S + pt1 * NTILE, ((size_t)(K / g) * N - pt1 * NTILE) * 2);
    const __amdgpu_buffer_rsrc_t d_rs0 = buffer_rsrc(DELTA ? D + pt0 * NTILE : S, DELTA ? ((size_t)(K / g) * N - pt0 * NTILE) * 2 : 4);
    const __amdgpu_buffer_rsrc_t d_rs1 = buffer_rsrc(DELTA ? D + pt1 * NTILE : S, DELTA ? ((size_t)(K / g) * N - pt1 * NTILE) * 2 : 4);
    uint4v rw[SG][WN];
    uint32_t rs[SG][WN][NS], rd[SG][WN][NS];   // aligned scale / delta pairs (half c & 1)
    const unsigned w_off = (unsigned)lane * 16u;
    const unsigned s_off = ((unsigned)c >> 1) * 4u;
    // every load of step st (clamped: the count per step is fixed, which the
    // waits rely on)
    auto load = [&](int st, int slot) {
        const int k = kbeg + st <= klast ? kbeg + st : klast;
        load_a(k, slot);
#pragma unroll
        for (int t = 0; t < WN; ++t) {
            const __amdgpu_buffer_rsrc_t wr = odd(t) ? w_rs1 : w_rs0;
            const int wo = (rel(t) * KT + k) * 1024;
            rw[slot][t] = __builtin_bit_cast(uint4v, __builtin_amdgcn_raw_buffer_load_b128(wr, w_off, wo, 0));
        }
        const int gb = opaque_s(mid_group<GK>(k, g) * N * 2);   // (one load per step)
#pragma unroll
        for (int t = 0; t < WN; ++t) {
            const __amdgpu_buffer_rsrc_t sr = odd(t) ? s_rs1 : s_rs0;
#pragma unroll
            for (int h = 0; h < NS; ++h) {
                const int so = gb + h * N * 2 + 32 * rel(t);
                rs[slot][t][h] = __builtin_amdgcn_raw_buffer_load_b32(sr, s_off, so, 0);
            }
        }
        if (DELTA) {
#pragma unroll
            for (int t = 0; t < WN; ++t) {
                const __amdgpu_buffer_rsrc_t dr = odd(t) ? d_rs1 : d_rs0;
#pragma unroll
                for (int h = 0; h < NS; ++h) {
                    const int so = gb + h * N * 2 + 32 * rel(t);
                    rd[slot][t][h] = __builtin_amdgcn_raw_buffer_load_b32(dr, s_off, so, 0);
                }
            }
        }
    };

    // GK == 4 (g = 64): the k-tile's two groups are its low-nibble k-steps
    // 0, 1 (xl, group sums asum[0]) and its high-nibble k-steps 2, 3 (xh,
    // asum[1]), each with its own scale and delta
    float4v acc[WM][WN], xl[WM][WN], xh[WM][WN], asum[NS];
    const half8 ones = {1, 1, 1, 1, 1, 1, 1, 1};
    const float4v fzero = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int h = 0; h < NS; ++h) asum[h] = fzero;
#pragma unroll
    for (int mt = 0; mt < WM; ++mt)
#pragma unroll
        for (int t = 0; t < WN; ++t) acc[mt][t] = xl[mt][t] = xh[mt][t] = fzero;
    int st_ = 0;   // the step being computed
    // k2s: k2 of the group(s) whose delta term is pending
    float k16[WN], k1[WN], k2[WN][NS], k2s[WN][NS];

    auto compute = [&](int slot, bool first) {
#pragma unroll
        for (int t = 0; t < WN; ++t) {
            float sv[NS];
#pragma unroll
            for (int h = 0; h < NS; ++h) {
                sv[h] = h2f((uint16_t)(rs[slot][t][h] >> sh));
                const float dv = DELTA ? h2f((uint16_t)(rd[slot][t][h] >> sh)) : 0.f;
                k2[t][h] = DELTA ? (dv - 8.0f * sv[h]) : (-8.0f * sv[h]);
                pin(k2[t][h]);
            }
            k16[t] = sv[0] * 0x1p24f;
            k1[t] = sv[NS - 1] * 0x1p20f;
            pin(k16[t]); pin(k1[t]);
        }
        // (the refill below goes to the previous step's slot: this slot's
        // code registers stay valid until they are split here)
        load(st_ + SG - 1, (slot + SG - 1) % SG);
        if (st_ >= kn) return;                            // past this k-group's range
        CodeOps ops[WN];
#pragma unroll
        for (int t = 0; t < WN; ++t) ops[t] = split_codes(rw[slot][t]);
        const _Float16 *as = Asm + (size_t)(slot * 2 + kg) * BM * KTILE;
#pragma unroll
        for (int mt = 0; mt < WM; ++mt) {
            const int r = 16 * mt + c;
            half8 a[4];
#pragma unroll
            for (int o = 0; o < 4; ++o)
                a[o] = *reinterpret_cast<const half8 *>(as + r * KTILE + 8 * ((4 * o + kq) ^ c));
            if (mt == wn) {   // this wave's share of the group sums
                asum[0] = mfma_f16(a[0], ones, first ? fzero : asum[0]);
                asum[0] = mfma_f16(a[1], ones, asum[0]);
                asum[NS - 1] = mfma_f16(a[2], ones, NS == 2 ? fzero : asum[0]);
                asum[NS - 1] = mfma_f16(a[3], ones, asum[NS - 1]);
            }
#pragma unroll
            for (int t = 0; t < WN; ++t) {
                xl[mt][t] = mfma_f16(a[0], ops[t].lo[0], first ? fzero : xl[mt][t]);
                xl[mt][t] = mfma_f16(a[1], ops[t].lo[1], xl[mt][t]);
                xh[mt][t] = mfma_f16(a[2], ops[t].hi[0], first ? fzero : xh[mt][t]);
                xh[mt][t] = mfma_f16(a[3], ops[t].hi[1], xh[mt][t]);
            }
        }
    };
    // end of a weight group: scale applied to its raw sums, this wave's group
    // sums published (parity par), the delta factor kept for later
    auto close = [&](int par) {
#pragma unroll
        for (int mt = 0; mt < WM; ++mt)
#pragma unroll
            for (int t = 0; t < WN; ++t)
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    acc[mt][t][r] = __builtin_fmaf(k1[t], xh[mt][t][r], __builtin_fmaf(k16[t], xl[mt][t][r], acc[mt][t][r]));
        if (c == 0)
#pragma unroll
            for (int h = 0; h < NS; ++h)
                *reinterpret_cast<float4v *>(gx + ((kg * 2 + par) * NS + h) * BM + 16 * wn + 4 * kq) = asum[h];
#pragma unroll
        for (int t = 0; t < WN; ++t)
#pragma unroll
            for (int h = 0; h < NS; ++h) k2s[t][h] = k2[t][h];
    };
    // the pending delta term of the group published with parity par
    auto delta_term = [&](int par) {
#pragma unroll
        for (int mt = 0; mt < WM; ++mt)
#pragma unroll
            for (int h = 0; h < NS; ++h) {
                const float4v gs = *reinterpret_cast<const float4v *>(gx + ((kg * 2 + par) * NS + h) * BM + 16 * mt + 4 * kq);
#pragma unroll
                for (int t = 0; t < WN; ++t)
#pragma unroll
                    for (int r = 0; r < 4; ++r) acc[mt][t][r] = __builtin_fmaf(k2s[t][h], gs[r], acc[mt][t][r]);
            }
    };
    auto sync = [&]() {
        debug_stage_sync();
        asm volatile("" ::: "memory");
        __builtin_amdgcn_s_barrier();
        asm volatile("" ::: "memory");
    };
    // st: the step, slot = st % SG (st comes in slot order from a multiple of SG)
    // tail: a step after the main loop, which waits for every load in flight
    // (as in the 64 x 64 kernel: the compiler drops the unread loads there)
    auto step = [&](int st, int slot, bool tail) {
        constexpr unsigned WAIT = waitcnt_vm((SG - 2) * L);
        if (tail)
            __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));
        else
            __builtin_amdgcn_s_waitcnt(WAIT);
        sync();
        // nothing that reads this slot's registers moves above the wait
        __builtin_amdgcn_sched_barrier(0);
        st_ = st;
        if (GK == 1 || GK == 3 || GK == 4) {
            // groups of one k-tile (or two per k-tile): the previous step's group gets its delta
            // term, this step's group is closed
            if (st > 0 && st - 1 < kn) delta_term((slot - 1) & 1);
            compute(slot, true);
            if (st < kn) close(slot & 1);
        } else if (GK == 2) {
            if (slot & 1) {
                compute(slot, false);
                if (st < kn) close((slot >> 1) & 1);
            } else {
                if (st > 0 && st - 1 < kn) delta_term(((slot + SG - 1) % SG >> 1) & 1);
                compute(slot, true);
            }
        } else {
            compute(slot, false);   // one group over all of K, closed after the loop
        }
    };

    const int nsteps = KH;   // >= KT - KH
#pragma unroll
    for (int i = 0; i < SG - 1; ++i) {
        load(i, i);
        __builtin_amdgcn_sched_barrier(0);   // step by step, as the loop refills
    }
    int st = 0;
    for (; st + SG <= nsteps; st += SG) {
#pragma unroll
        for (int i = 0; i < SG; ++i) {
            step(st + i, i, false);
            asm volatile("" ::: "memory");
            __builtin_amdgcn_sched_barrier(0);
        }
    }
#pragma unroll
    for (int i = 0; i < SG - 1; ++i)
        if (st + i < nsteps) step(st + i, i, true);
    __builtin_amdgcn_s_waitcnt(0);   // the last (unused) loads

    // the last group's delta term (one group over all of K: closed here)
    if (GK == 0) close(0);
    const bool last_pending = GK == 0 ? true : (kn == nsteps && kn > 0);
    const int last_par = GK == 2 ? (((nsteps - 1) % SG) >> 1) & 1 : ((nsteps - 1) % SG) & 1;
    sync();
    if (last_pending) delta_term(GK == 0 ? 0 : last_par);

    // the two k-groups meet: k-group 1 hands its sums to k-group 0 (the ring
    // is dead: 4 waves x 32 floats x 64 lanes = 32 KB)
    sync();
    float *red = reinterpret_cast<float *>(Asm);
    if (kg == 1) {
#pragma unroll
        for (int mt = 0; mt < WM; ++mt)
#pragma unroll
            for (int t = 0; t < WN; ++t)
#pragma unroll
                for (int r = 0; r < 4; ++r) red[(wn * 32 + (mt * WN + t) * 4 + r) * 64 + lane] = acc[mt][t][r];
    }
    sync();
    if (kg == 1) return;
#pragma unroll
    for (int mt = 0; mt < WM; ++mt)
#pragma unroll
        for (int t = 0; t < WN; ++t)
#pragma unroll
            for (int r = 0; r < 4; ++r) acc[mt][t][r] += red[(wn * 32 + (mt * WN + t) * 4 + r) * 64 + lane];
#pragma unroll
    for (int mt = 0; mt < WM; ++mt)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int row = m0 + 16 * mt + 4 * kq + r;
            if (row >= M) continue;
            if (GATED) {
                C[(size_t)row * (N / 2) + pt0 * NTILE + c] = f2h(silu_mul(acc[mt][0][r], acc[mt][1][r]));
            } else {
#pragma unroll
                for (int t = 0; t < WN; ++t) C[(size_t)row * N + col0 + 16 * t] = f2h(acc[mt][t][r]);
            }
        }
}

template <bool DELTA, int GK, bool GATED>
static hipError_t run_mid(const uint16_t *A, const uint32_t *W, const uint16_t *S,
                          const uint16_t *D, uint16_t *C, int M, int N, int K, int g,
                          hipStream_t st)
{
    dim3 grid((unsigned)(N / 64), (unsigned)((M + 63) / 64));
    const size_t lds = (size_t)MID_STAGES * 64 * KTILE * sizeof(_Float16);
    hipLaunchKernelGGL((w4a16_mid_kernel<MID_STAGES, DELTA, GK, GATED>), grid, dim3(256), lds, st, A,
                       reinterpret_cast<const uint4v *>(W), S, D, C, M, N, K, g);
    return hipGetLastError();
}

template <bool DELTA, bool GATED>
static hipError_t run_mid_g(const uint16_t *A, const uint32_t *W, const uint16_t *S,
                            const uint16_t *D, uint16_t *C, int M, int N, int K, int g,
                            hipStream_t st)
{
    // the two-k-tile form needs groups of exactly 2 k-tiles (MID_STAGES even:
    // group parity follows the ring slot)
    static_assert(MID_STAGES % 2 == 0, "k-tile parity must follow the ring slot");
    if (g == K) return run_mid<DELTA, 0, GATED>(A, W, S, D, C, M, N, K, g, st);
    if (g == 2 * KTILE) return run_mid<DELTA, 2, GATED>(A, W, S, D, C, M, N, K, g, st);
    if (g == KTILE) return run_mid<DELTA, 1, GATED>(A, W, S, D, C, M, N, K, g, st);
    return run_mid<DELTA, 3, GATED>(A, W, S, D, C, M, N, K, g, st);
}

template <bool DELTA, int GK, bool GATED>
static hipError_t run_mid2(const uint16_t *A, const uint32_t *W, const uint16_t *S,
                           const uint16_t *D, uint16_t *C, int M, int N, int K, int g,
                           hipStream_t st)
{
    constexpr int SG = MID2_STAGES, NS = GK == 4 ? 2 : 1;
    const size_t lds = (size_t)SG * 2 * 64 * KTILE * sizeof(_Float16) + 2 * 2 * NS * 64 * sizeof(float);
    auto kern = w4a16_mid2_kernel<SG, DELTA, GK, GATED>;
    // LDS beyond 64 KB: the attribute is set once per device (and instantiation)
    static std::atomic<unsigned> attr_devs{0};
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    const unsigned bit = dev >= 0 && dev < 32 ? 1u << dev : 0u;
    if (!(attr_devs.load(std::memory_order_acquire) & bit)) {
        e = hipFuncSetAttribute((const void *)kern, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
        if (e != hipSuccess) return e;
        attr_devs.fetch_or(bit, std::memory_order_release);
    }
    dim3 grid((unsigned)(N / 128), (unsigned)((M + 63) / 64));
    hipLaunchKernelGGL(kern, grid, dim3(512), lds, st, A, reinterpret_cast<const uint4v *>(W), S, D,
                       C, M, N, K, g);
    return hipGetLastError();
}

template <bool DELTA, bool GATED>
static hipError_t run_mid2_g(const uint16_t *A, const uint32_t *W, const uint16_t *S,
                             const uint16_t *D, uint16_t *C, int M, int N, int K, int g,
                             hipStream_t st)
{
    if (g == K) return run_mid2<DELTA, 0, GATED>(A, W, S, D, C, M, N, K, g, st);
    if (g == 2 * KTILE) return run_mid2<DELTA, 2, GATED>(A, W, S, D, C, M, N, K, g, st);
    if (g == KTILE) return run_mid2<DELTA, 1, GATED>(A, W, S, D, C, M, N, K, g, st);
    if (g == KTILE / 2) return run_mid2<DELTA, 4, GATED>(A, W, S, D, C, M, N, K, g, st);
    return run_mid2<DELTA, 3, GATED>(A, W, S, D, C, M, N, K, g, st);
}

// The 8-wave 64 x 128 kernel (K split inside the workgroup) when it still
// gives every CU a workgroup and each k-group at least 2 k-tiles; else the
// 4-wave 64 x 64 kernel.
bool use_mid2(int M, int N, int K)
{
    return N % 128 == 0 && (long)(N / 128) * ((M + 63) / 64) >= 256 && K / KTILE >= 4;
}

hipError_t launch_w4a16_mid(const uint16_t *A, const uint32_t *W, const uint16_t *S,
                            const uint16_t *D, uint16_t *C, int M, int N, int K, int g,
                            bool fuse_delta, hipStream_t st, bool gated)
{
    if (use_mid2(M, N, K)) {
        const bool dl = D && fuse_delta;
        if (gated)
            return dl ? run_mid2_g<true, true>(A, W, S, D, C, M, N, K, g, st)
                      : run_mid2_g<false, true>(A, W, S, nullptr, C, M, N, K, g, st);
        return dl ? run_mid2_g<true, false>(A, W, S, D, C, M, N, K, g, st)
                  : run_mid2_g<false, false>(A, W, S, nullptr, C, M, N, K, g, st);
    }
    if (g < KTILE) return hipErrorInvalidValue;   // (the 64 x 64 kernel takes g >= 128)
    const bool dl = D && fuse_delta;
    if (gated)
        return dl ? run_mid_g<true, true>(A, W, S, D, C, M, N, K, g, st)
                  : run_mid_g<false, true>(A, W, S, nullptr, C, M, N, K, g, st);
    return dl ? run_mid_g<true, false>(A, W, S, D, C, M, N, K, g, st)
              : run_mid_g<false, false>(A, W, S, nullptr, C, M, N, K, g, st);
}

} // namespace qg
