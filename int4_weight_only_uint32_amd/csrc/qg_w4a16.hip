// W4A16 GEMM kernels and the two-stage asymmetric correction.
//
// Method ("Marlin INT4 on Ada - how it works", section "The core mismatch:
// symmetric vs asymmetric"): with delta[g,n] = zero[g,n] + 8*scale[g,n],
//     C = A . W_sym + A_group_sum @ delta,  W_sym[k,n] = (q[k,n] - 8) scale[g,n]
// which is exact because delta does not depend on k.
//
// Skinny kernel (M < 128; for most M <= 16 shapes the decode kernel below,
// which shares the activation tile between waves, is used instead).  A wave owns MT 16-row m-tiles x NT 16-column
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

#include <type_traits>

namespace qg {

template <int MT, int NT, int P, int NWMAX, bool DELTA, bool GATED>
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
    uint32_t rs[P][NT], rd[P][NT];
    const int sh = 16 * (c & 1);
    auto load = [&](int kt, uint4v (&a)[MT * 4], uint4v (&w)[NT], uint32_t (&sv)[NT],
                    uint32_t (&dv)[NT]) {
#pragma unroll
        for (int j = 0; j < MT * 4; ++j) a[j] = asrc[j][kt * (KTILE / 8)];
#pragma unroll
        for (int t = 0; t < NT; ++t) w[t] = wbase[((size_t)trel(t) * KT + kt) * 64];
        const int gi = (kt * KTILE) / g;
        const uint32_t *srow = reinterpret_cast<const uint32_t *>(S + (size_t)gi * N + (col0 & ~1));
#pragma unroll
        for (int t = 0; t < NT; ++t) sv[t] = srow[8 * trel(t)];
        if (DELTA) {
            const uint32_t *drow = reinterpret_cast<const uint32_t *>(D + (size_t)gi * N + (col0 & ~1));
#pragma unroll
            for (int t = 0; t < NT; ++t) dv[t] = drow[8 * trel(t)];
        }
    };
    // Consuming a slot happens in two halves: `stage` moves the slot's
    // activations into LDS and splits its codes into MFMA operands, after which
    // the slot's registers are free and the refill can be issued; `finish`
    // then does the MFMAs and the per-group scaling while the refill is in
    // flight.
    struct Staged {
        CodeOps ops[NT];
        float s[NT], d[NT];
    };
    auto stage = [&](const uint4v (&ar)[MT * 4], const uint4v (&w)[NT], const uint32_t (&sv)[NT],
                     const uint32_t (&dv)[NT], Staged &st) {
#pragma unroll
        for (int j = 0; j < MT * 4; ++j) *reinterpret_cast<uint4v *>(scratch + adst[j]) = ar[j];
#pragma unroll
        for (int t = 0; t < NT; ++t) {
            st.ops[t] = split_codes(w[t]);
            st.s[t] = h2f((uint16_t)(sv[t] >> sh));
            st.d[t] = DELTA ? h2f((uint16_t)(dv[t] >> sh)) : 0.f;
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
            const float s = st.s[t];
            const float c1 = s * 0x1p20f, c16 = s * 0x1p24f;
            const float c2 = DELTA ? (st.d[t] - 8.0f * s) : (-8.0f * s);
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

// ---- decode kernel (M <= 16) ----
// A workgroup of 4 waves owns 4*NT consecutive 16-column strips (wave w the
// strips 4*NT*cg + NT*w .. +NT-1) and one of `nsplit` contiguous ranges of
// 128-k tiles.  Each k-tile of A (16 rows x 128 k, 4 KB) is fetched once per
// workgroup -- one 16-byte load per thread, rows past M reading row M-1 --
// and shared through LDS (double buffered, one barrier per k-tile), so the
// activation traffic is one tile per workgroup instead of one per wave.
// Each wave streams its codes, scales and deltas through a P-deep register
// ring; the MFMA and scaling steps are those of the skinny kernel.
//
// nsplit > 1: the workgroups of a column group each hold fp32 partial sums
// for the same outputs.  Each writes them to its slot of the workspace with
// device-coherent stores, waits for them to complete, and increments the
// column group's counter (device-scope atomic).  The one that sees
// nsplit - 1 adds the slots in split order (deterministic), converts to
// fp16, stores C and puts the counter back to zero.  Only device-coherent
// accesses touch the shared slots, so no cache-wide fence is needed; the
// workspace counters must be zero before the first call and stay zero
// between calls.
// GATED: W is a gate/up pair packed as one [K, N] weight (gate columns
// 0 .. N/2-1, up columns N/2 .. N-1) and C receives silu(gate) * up [M, N/2].
// Waves 0, 1 of workgroup cg take gate n-tiles 2cg, 2cg+1, waves 2, 3 the up
// n-tiles of the same columns; after the (split-K) sums, the up waves hand
// their values to the gate waves through LDS.
template <int NT, int P, int WV, bool DELTA, bool GATED = false>
__global__ __launch_bounds__(64 * WV) void w4a16_decode_kernel(
    const uint16_t *__restrict__ A, const uint4v *__restrict__ W, const uint16_t *__restrict__ S,
    const uint16_t *__restrict__ D, uint16_t *__restrict__ C, int M, int N, int K, int g,
    int nsplit, unsigned *__restrict__ counters, float *__restrict__ partials)
{
    static_assert(NT == 1, "the scale table holds one column per lane");
    static_assert(WV == 4 || WV == 8, "4 or 8 waves per workgroup");
    static_assert(!GATED || WV == 4, "the gate/up pairing takes 4 waves");
    constexpr int COLS = 16 * WV;            // columns per workgroup
    __shared__ __attribute__((aligned(16))) _Float16 As[2][16 * KTILE];
    __shared__ unsigned arrived;
    __shared__ float xch[GATED ? 2 * 4 * 64 : 1];   // up values for the gate waves
    // (scale | delta << 16) of this workgroup's 64 columns for every group its
    // k-range touches: filled once, read once per k-tile (an LDS read instead
    // of two global loads per k-tile)
    extern __shared__ uint32_t sdt[];
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int c = lane & 15, kq = lane >> 4;
    const int KT = K / KTILE;
    const int cg = blockIdx.x / nsplit, sp = blockIdx.x - cg * nsplit;
    const int kt_beg = (sp * KT) / nsplit, kt_end = ((sp + 1) * KT) / nsplit;
    const int n = kt_end - kt_beg;
    const int last = kt_end - 1;
    const int Nh = N / 2;                    // GATED: output width
    const int nt0 = GATED ? (wave < 2 ? 2 * cg + wave : Nh / NTILE + 2 * cg + wave - 2)
                          : (cg * WV + wave) * NT;
    const int col0 = GATED ? 32 * cg + 16 * (wave & 1) + c : nt0 * NTILE + c;

    // scale table: its loads are issued first (the oldest in flight), and,
    // when it fits in TB words per thread, written to LDS only after the
    // ring's first loads are out, so its latency overlaps theirs instead of
    // preceding them
    constexpr int TB = 4;
    const int gi0 = (kt_beg * KTILE) / g;
    const int ng = n > 0 ? ((kt_end - 1) * KTILE) / g - gi0 + 1 : 0;
    const int total = ng * (COLS / 2);
    const bool tfast = total <= TB * 64 * WV;
    // scale pairs of the table's COLS columns: contiguous, or (GATED) the 32
    // gate columns 32cg.. and the 32 up columns Nh + 32cg..
    const int pbase = GATED ? 16 * cg : cg * (COLS / 2);
    const int pgap = GATED ? Nh / 2 - 16 : 0;   // added to pairs 16.. (GATED)
    const uint32_t *s32 = reinterpret_cast<const uint32_t *>(S) + (size_t)gi0 * (N / 2) + pbase;
    const uint32_t *d32 = DELTA ? reinterpret_cast<const uint32_t *>(D) + (size_t)gi0 * (N / 2) + pbase : nullptr;
    uint32_t tsv[TB], tdv[TB];
    if (n > 0) {
        if (tfast) {
            // unconditional, clamped: the waits for these count exactly
#pragma unroll
            for (int i = 0; i < TB; ++i) {
                int idx = tid + i * 64 * WV;
                idx = idx < total ? idx : total - 1;
                const int gl = idx / (COLS / 2), pr = idx % (COLS / 2);
                const int sp2 = pr + (GATED && pr >= 16 ? pgap : 0);
                tsv[i] = s32[(size_t)gl * (N / 2) + sp2];
                tdv[i] = DELTA ? d32[(size_t)gl * (N / 2) + sp2] : 0u;
            }
        } else {
            for (int idx = tid; idx < total; idx += 64 * WV) {
                const int gl = idx / (COLS / 2), pr = idx % (COLS / 2);
                const int sp2 = pr + (GATED && pr >= 16 ? pgap : 0);
                const uint32_t s2 = s32[(size_t)gl * (N / 2) + sp2];
                const uint32_t d2 = DELTA ? d32[(size_t)gl * (N / 2) + sp2] : 0u;
                sdt[gl * COLS + 2 * pr] = (s2 & 0xFFFFu) | (d2 << 16);
                sdt[gl * COLS + 2 * pr + 1] = (s2 >> 16) | (d2 & 0xFFFF0000u);
            }
        }
    }

    // activation tile (16 rows x 256 bytes): with 4 waves thread t fetches
    // row t/16, 16-byte chunk t%16; with 8 waves row t/32, 8-byte piece t%32.
    // A 16-byte chunk lands at position chunk ^ row within its 256-byte LDS
    // row so the 16 rows an MFMA operand reads fall in distinct banks.
    using AVec = typename std::conditional<WV == 4, uint4v, uint2v>::type;
    constexpr int APR = 256 / sizeof(AVec);      // pieces per row
    const int arow_i = tid / APR, apc = tid % APR;
    const int arow = arow_i < M ? arow_i : M - 1;
    const AVec *asrc = reinterpret_cast<const AVec *>(A + (size_t)arow * K) + apc;
    const int ach = apc * (int)sizeof(AVec) / 16, asub = (apc * (int)sizeof(AVec) % 16) / 2;
    const int adst = arow_i * KTILE + 8 * (ach ^ (arow_i & 15)) + asub;
    const uint4v *wbase = W + (size_t)nt0 * KT * 64 + lane;
    const int gbase = (kt_beg * KTILE) / g;

    float4v acc[NT];
#pragma unroll
    for (int t = 0; t < NT; ++t) acc[t] = float4v{0.f, 0.f, 0.f, 0.f};
    const half8 ones = {1, 1, 1, 1, 1, 1, 1, 1};
    const float4v fzero = {0.f, 0.f, 0.f, 0.f};

    AVec ra[P];
    uint4v rw[P][NT];
    auto load = [&](int kt, AVec &a, uint4v (&w)[NT]) {
        a = asrc[(size_t)kt * (KTILE * 2 / sizeof(AVec))];
#pragma unroll
        for (int t = 0; t < NT; ++t) w[t] = wbase[((size_t)t * KT + kt) * 64];
    };
    auto finish = [&](int buf, int kt, const CodeOps (&ops)[NT]) {
        half8 a[4];
#pragma unroll
        for (int o = 0; o < 4; ++o)
            a[o] = *reinterpret_cast<const half8 *>(&As[buf][c * KTILE + 8 * ((4 * o + kq) ^ c)]);
        const uint32_t sd = sdt[((kt * KTILE) / g - gbase) * COLS + 16 * wave + c];
        float4v as = mfma_f16(a[0], ones, fzero);
        as = mfma_f16(a[1], ones, as);
        as = mfma_f16(a[2], ones, as);
        as = mfma_f16(a[3], ones, as);
#pragma unroll
        for (int t = 0; t < NT; ++t) {
            const float s = h2f((uint16_t)(sd & 0xFFFFu));
            const float d = DELTA ? h2f((uint16_t)(sd >> 16)) : 0.f;
            const float c1 = s * 0x1p20f, c16 = s * 0x1p24f;
            const float c2 = DELTA ? (d - 8.0f * s) : (-8.0f * s);
            float4v xl = mfma_f16(a[0], ops[t].lo[0], fzero);
            xl = mfma_f16(a[1], ops[t].lo[1], xl);
            float4v xh = mfma_f16(a[2], ops[t].hi[0], fzero);
            xh = mfma_f16(a[3], ops[t].hi[1], xh);
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                float v = __builtin_fmaf(c16, xl[r], acc[t][r]);
                v = __builtin_fmaf(c1, xh[r], v);
                acc[t][r] = __builtin_fmaf(c2, as[r], v);
            }
        }
    };
    auto step = [&](int kt, int slot, int kt_next) {
        const int buf = (kt - kt_beg) & 1;
        *reinterpret_cast<AVec *>(&As[buf][adst]) = ra[slot];
        CodeOps ops[NT];
#pragma unroll
        for (int t = 0; t < NT; ++t) {
            ops[t] = split_codes(rw[slot][t]);
            pin(ops[t].lo[0]); pin(ops[t].lo[1]); pin(ops[t].hi[0]); pin(ops[t].hi[1]);
        }
        // unconditional (clamped) refill: a conditional load would make every
        // later wait assume it might be missing and wait for everything
        load(kt_next, ra[slot], rw[slot]);
        __syncthreads();
        finish(buf, kt, ops);
    };

    if (n > 0) {
#pragma unroll
        for (int i = 0; i < P; ++i) {
            const int kt = kt_beg + i;
            load(kt < last ? kt : last, ra[i], rw[i]);
            // slot by slot, in the order the loop refills them (the waits in
            // the loop are computed for both orders)
            __builtin_amdgcn_sched_barrier(0);
        }
        if (tfast) {
#pragma unroll
            for (int i = 0; i < TB; ++i) {
                const int idx = tid + i * 64 * WV;
                if (idx < total) {
                    const int gl = idx / (COLS / 2), pr = idx % (COLS / 2);
                    sdt[gl * COLS + 2 * pr] = (tsv[i] & 0xFFFFu) | (tdv[i] << 16);
                    sdt[gl * COLS + 2 * pr + 1] = (tsv[i] >> 16) | (tdv[i] & 0xFFFF0000u);
                }
            }
        }
        int j = 0;
        for (; j + P <= n; j += P) {
#pragma unroll
            for (int i = 0; i < P; ++i) {
                const int kt = kt_beg + j + i + P;
                step(kt_beg + j + i, i, kt < last ? kt : last);
                // keep each refill ahead of the loop's back edge (see the
                // skinny kernel) and the next slot's work out of this step
                asm volatile("" ::: "memory");
                __builtin_amdgcn_sched_barrier(0);
            }
        }
#pragma unroll
        for (int i = 0; i < P - 1; ++i)
            if (j + i < n) step(kt_beg + j + i, i, last);
    }

    // C rows 4 kq + r, columns (nt0 + t) * 16 + c; GATED: silu(gate) * up
    // into C [M, Nh] by the gate waves (reached by every thread of the
    // workgroup, or of none: the barrier is uniform)
    auto store = [&](const float4v (&v)[NT]) {
        if (GATED) {
            if (wave >= 2)
#pragma unroll
                for (int r = 0; r < 4; ++r) xch[(wave - 2) * 256 + r * 64 + lane] = v[0][r];
            __syncthreads();
            if (wave < 2)
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int row = 4 * kq + r;
                    const float gv = v[0][r], u = xch[wave * 256 + r * 64 + lane];
                    if (row < M) C[(size_t)row * Nh + col0] = f2h(gv / (1.0f + __builtin_expf(-gv)) * u);
                }
            return;
        }
#pragma unroll
        for (int t = 0; t < NT; ++t)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int row = 4 * kq + r;
                if (row < M) C[(size_t)row * N + col0 + 16 * t] = f2h(v[t][r]);
            }
    };
    if (nsplit == 1) {
        store(acc);
        return;
    }
    // slot layout: [cg][split][wave][t][r][lane] fp32
    constexpr int PER_WAVE = NT * 4 * 64;
    float *mine = partials + ((size_t)cg * nsplit + sp) * WV * PER_WAVE + wave * PER_WAVE + lane;
#pragma unroll
    for (int t = 0; t < NT; ++t)
#pragma unroll
        for (int r = 0; r < 4; ++r)
            __hip_atomic_store(mine + (t * 4 + r) * 64, acc[t][r], __ATOMIC_RELAXED,
                               __HIP_MEMORY_SCOPE_AGENT);
    __builtin_amdgcn_s_waitcnt(0);          // this thread's slot stores are complete
    __syncthreads();                        // ... and every thread's
    if (tid == 0)
        arrived = __hip_atomic_fetch_add(&counters[cg], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __syncthreads();
    if (arrived != (unsigned)(nsplit - 1)) return;
    float4v tot[NT];
#pragma unroll
    for (int t = 0; t < NT; ++t) tot[t] = fzero;
    const float *base = partials + (size_t)cg * nsplit * WV * PER_WAVE + wave * PER_WAVE + lane;
    for (int s2 = 0; s2 < nsplit; ++s2) {
#pragma unroll
        for (int t = 0; t < NT; ++t)
#pragma unroll
            for (int r = 0; r < 4; ++r)
                tot[t][r] += (s2 == sp) ? acc[t][r]
                                        : __hip_atomic_load(base + (size_t)s2 * WV * PER_WAVE + (t * 4 + r) * 64,
                                                            __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    store(tot);
    if (tid == 0) __hip_atomic_store(&counters[cg], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

namespace decode {
constexpr int NT = 1, P = 2, WV = 4;      // 8 waves measured slower
constexpr int COLS = WV * NT * NTILE;    // columns per workgroup
}

// Groups the k-range of one split touches (at most): the size of the decode
// kernel's scale table in 64-column rows.
int decode_max_groups(int K, int g, int nsplit)
{
    const int KT = K / KTILE;
    const int span = (KT + nsplit - 1) / nsplit;          // k-tiles per split, at most
    const int per_group = g / KTILE > 0 ? g / KTILE : 1;  // k-tiles per group
    return (span + per_group - 1) / per_group + 1;
}

// Split count of the decode kernel.  All workgroups are resident at once, and
// a CU holding one workgroup more than the others finishes last, so the count
// that keeps every CU at <= 2 workgroups (512 slots on 256 CUs) is taken when
// it still fills >= 7/8 of the slots (at K = 17408, N = 5120: 6 splits, 480
// workgroups, 6-12 % faster than 8 splits and 640 workgroups).  Otherwise the
// smallest power of two giving at least 512 workgroups.  Both keep >= 2
// k-tiles per split and <= 16 splits; more splits while one split's scale
// table would exceed 32 KB of LDS.
// The two-per-CU split count when it applies (see decode_splits), else 0.
static int decode_balanced_splits(int N, int K)
{
    const int KT = K / KTILE, ncg = N / decode::COLS;
    const int fit = 512 / ncg;
    return (fit >= 2 && fit <= 16 && ncg * fit >= 448 && KT / fit >= 2) ? fit : 0;
}

int decode_splits(int N, int K)
{
    const int KT = K / KTILE, ncg = N / decode::COLS;
    int ns = 1;
    if ((size_t)ncg * sizeof(unsigned) > W4A16_WS_COUNTER_BYTES) return 1;   // no counter for it
    if (const int fit = decode_balanced_splits(N, K))
        ns = fit;
    else
        while (ns < 16 && (long)ncg * ns < 512 && KT / (2 * ns) >= 2) ns *= 2;
    while (ns < 1024 && (size_t)decode_max_groups(K, KTILE, ns) * decode::COLS * 4 > 32768) ns *= 2;
    return ns;
}

// Decode workspace: the fixed counter region (W4A16_WS_COUNTER_BYTES, shared
// by every W4A16 layout and written by nothing but the counters), then the
// partial-sum slots.  0 when the shape is not split.
// Whether M <= 16 runs the decode kernel rather than the skinny one (which
// splits K between the 8 waves of a workgroup of 32 columns and needs no
// cross-workgroup step).  Measured on MI355X (M = 4-16, interleaved repeats):
// * two or fewer decode splits (wide N): the decode kernel;
// * more than 256 skinny workgroups (some CUs hold two, the rest one) on
//   weights of >= 32 M elements: the decode kernel (K = 4096: N = 10240
//   9.6 against 13.2 us, N = 12288 12.0 against 13.9);
// * otherwise the decode kernel only when the skinny kernel leaves CUs idle
//   (< 256 workgroups) and each decode split still streams >= 16 k-tiles
//   (K = 16384, N = 4096: 14.8 against 17.4 us; K = 17408, N = 5120); with
//   shorter splits its fixed costs (scale table, split-K epilogue) lose
//   (K = 4096, N = 4096-8192: 9.2-10 against 7.2-8.5 us; K = N = 8192: 12.7
//   against 11.7).
bool use_decode_kernel(int M, int N, int K)
{
    if (M > 16 || N % decode::COLS) return false;
    const int ns = decode_splits(N, K);
    if (ns <= 2) return true;
    const long skinny_wgs = N / 32;
    if (skinny_wgs > 256) return (long long)K * N >= (1ll << 25);
    return skinny_wgs < 256 && (K / KTILE) / ns >= 16;
}

size_t decode_workspace_bytes(int M, int N, int K)
{
    if (!use_decode_kernel(M, N, K)) return 0;
    const int ns = decode_splits(N, K);
    if (ns == 1) return 0;
    const size_t ncg = (size_t)(N / decode::COLS);
    return W4A16_WS_COUNTER_BYTES + ncg * ns * 16 * decode::COLS * sizeof(float);
}

template <bool DELTA, bool GATED = false>
static hipError_t run_decode(const uint16_t *A, const uint32_t *W, const uint16_t *S,
                             const uint16_t *D, uint16_t *C, int M, int N, int K, int g,
                             int nsplit, void *ws, hipStream_t st)
{
    const int ncg = N / decode::COLS;
    unsigned *counters = nullptr;
    float *partials = nullptr;
    if (nsplit > 1) {
        counters = static_cast<unsigned *>(ws);
        partials = reinterpret_cast<float *>(static_cast<char *>(ws) + W4A16_WS_COUNTER_BYTES);
    }
    const size_t table = (size_t)decode_max_groups(K, g, nsplit) * decode::COLS * sizeof(uint32_t);
    hipLaunchKernelGGL((w4a16_decode_kernel<decode::NT, decode::P, decode::WV, DELTA, GATED>),
                       dim3(ncg * nsplit), dim3(64 * decode::WV), table, st, A, reinterpret_cast<const uint4v *>(W), S, D, C, M,
                       N, K, g, nsplit, counters, partials);
    return hipGetLastError();
}

hipError_t launch_w4a16_decode(const uint16_t *A, const uint32_t *W, const uint16_t *S,
                               const uint16_t *D, uint16_t *C, int M, int N, int K, int g,
                               bool fuse_delta, int nsplit, void *ws, hipStream_t st)
{
    if (M > 16 || N % decode::COLS || nsplit < 1 || (nsplit > 1 && !ws))
        return hipErrorInvalidValue;
    if (D && fuse_delta) return run_decode<true>(A, W, S, D, C, M, N, K, g, nsplit, ws, st);
    return run_decode<false>(A, W, S, nullptr, C, M, N, K, g, nsplit, ws, st);
}

template <int MT, int NT, int P, int NWMAX, bool DELTA, bool GATED>
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
    hipLaunchKernelGGL((w4a16_skinny_kernel<MT, NT, P, NWMAX, DELTA, GATED>), grid, dim3(64 * cf.nw), lds,
                       st, A, reinterpret_cast<const uint4v *>(W), S, D, C, M, N, K, g, cf.nw);
    return hipGetLastError();
}

// ---- tiled kernel (M >= 128) ----
// Workgroup tile BM = 16*WM rows x BN = 64*WN columns, 4 waves; wave w owns
// columns [16*WN*w, 16*WN*(w+1)) (WN n-tiles) and all BM rows (WM m-tiles).
// Two configurations: 128 x 256 (WM = 8, WN = 4) for large M x N, and
// 64 x 128 (WM = 4, WN = 2) when the large tile would leave the GPU short of
// workgroups (mid-size M).  A is staged through LDS (two buffers of BM x 128
// fp16) with gfx950's direct global->LDS 16-byte loads, no registers in
// between.  Within a 256-byte row the 16-byte chunk ch is stored at position
// ch ^ (row % 16), so the 16 rows an MFMA operand reads fall in distinct LDS
// banks; packed codes go straight from global memory to registers, each wave
// reading only its own columns.  Codes are dequantized per element to fp16
// ((v - 8) * scale, exact up to the one fp16 rounding of the product) and fed
// to 16x16x32 fp16 MFMAs.  Asymmetric weights: the per-group sums of A are
// accumulated by MFMAs against an all-ones operand (wave w sums m-tiles
// w*WM/4 .. (w+1)*WM/4 - 1), parked in LDS, and every 16 groups applied as
// one extra MFMA k-step whose A side is the group sums (split into a high and
// a low fp16 part) and whose B side is delta -- the "A_group_sum @ delta"
// term of the method, fused.
// Rows from which the tiled/mid kernels take over from the skinny one (the mid
// kernel measured faster from about M = 80 on).
constexpr int TILED_MIN_M = 81;

namespace tiled {
constexpr int WIN = 16;                         // groups per correction k-step
}

typedef _Float16 half2v __attribute__((ext_vector_type(2)));

// fp16 operand of k-step STEP (0..3) of a 128-k tile, scaled per element.
template <int STEP>
__device__ inline half8 dequant_scaled(uint4v w, half2v s2)
{
    const unsigned xa = (STEP & 1) ? w.z : w.x;
    const unsigned xb = (STEP & 1) ? w.w : w.y;
    const unsigned m = (STEP >= 2) ? 0x00F000F0u : 0x000F000Fu;
    const unsigned magic = 0x64006400u;       // fp16 1024.0 in both halves
    unsigned p[4] = {(xa & m) | magic, ((xa >> 8) & m) | magic, (xb & m) | magic,
                     ((xb >> 8) & m) | magic};
    unsigned out[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        half2v h = __builtin_bit_cast(half2v, p[i]);
        half2v v;
        if (STEP >= 2) {
            // 1024 + 16 v  ->  (1024 + 16 v) / 16 - 72 = v - 8   (exact)
            v = h * half2v{(_Float16)0.0625f, (_Float16)0.0625f} - half2v{(_Float16)72.f, (_Float16)72.f};
        } else {
            // 1024 + v  ->  v - 8   (exact)
            v = h - half2v{(_Float16)1032.f, (_Float16)1032.f};
        }
        v = v * s2;
        out[i] = __builtin_bit_cast(unsigned, v);
    }
    return __builtin_bit_cast(half8, uint4v{out[0], out[1], out[2], out[3]});
}

template <int WM, int WN, bool DELTA, bool GATED>
__global__ __launch_bounds__(256, (WM * WN >= 32) ? 2 : 3) void w4a16_tiled_kernel(
    const uint16_t *__restrict__ A, const uint4v *__restrict__ W, const uint16_t *__restrict__ S,
    const uint16_t *__restrict__ D, uint16_t *__restrict__ C, int M, int N, int K, int g)
{
    using namespace tiled;
    static_assert(WM % 4 == 0, "each wave sums WM/4 m-tiles of the group sums");
    constexpr int BM = 16 * WM, BN = 64 * WN;
    constexpr int ABLK = BM / 16;                     // 1 KB A blocks per wave and k-tile
    constexpr int GM = WM / 4;                        // group-sum m-tiles per wave
    __shared__ __attribute__((aligned(16))) _Float16 As[2][BM * 128];
    __shared__ __attribute__((aligned(16))) float asum_win[DELTA ? BM * WIN : 1];

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int c = lane & 15, kq = lane >> 4;
    const int KT = K / KTILE, G = K / g;
    const int m0 = blockIdx.y * BM;
    const int n0 = blockIdx.x * BN + wave * 16 * WN;   // this wave's first column
    const bool active = n0 < N;
    const int ntile0 = n0 / NTILE;
    // GATED: the wave's WN (virtual) n-tiles are WN/2 gate/up pairs: n-tile t
    // is tile t/2 of the gate run starting at ntile0/2 (t even) or of the up
    // run starting at N/32 + ntile0/2 (t odd); each run has its resources
    static_assert(!GATED || WN % 2 == 0, "gate/up pairs need an even WN");
    const int Nh16 = N / (2 * NTILE);
    auto odd = [](int t) { return GATED && (t & 1); };
    auto rel = [](int t) { return GATED ? (t >> 1) : t; };

    // ---- A: global -> LDS directly.  One wave instruction fills 1 KB = 4
    // rows; lane i lands at position i of that block, i.e. row 4b + i/16,
    // physical chunk i%16, which holds logical chunk (i%16) ^ (row%16).
    // Rows past M read row M-1 (their results are never stored).
    // Buffer loads (uniform resource, fixed per-lane byte offset, k offset in
    // a scalar register): no per-lane address arithmetic in the k-loop, and
    // the compiler then does not drain the next tile's direct-to-LDS loads
    // before this tile's LDS reads.
    const __amdgpu_buffer_rsrc_t a_rs = buffer_rsrc(A + (size_t)m0 * K, (size_t)(M - m0) * K * 2);
    unsigned a_off[ABLK];
#pragma unroll
    for (int i = 0; i < ABLK; ++i) {
        const int r = (wave * ABLK + i) * 4 + (lane >> 4);   // BM/4 blocks of 4 rows
        const int ch = (lane & 15) ^ (r & 15);
        const int row = m0 + r < M ? r : M - 1 - m0;
        a_off[i] = (unsigned)(row * K + ch * 8) * 2u;
    }
    auto load_a = [&](int kt, int st) {
#pragma unroll
        for (int i = 0; i < ABLK; ++i) {
            const int blk = wave * ABLK + i;
            // (arguments in variables of non-dependent type: a target
            // builtin called with template-dependent arguments is
            // instantiated in the host pass too, where it does not exist,
            // and the kernel would silently lose its host launch stub)
            __attribute__((address_space(3))) void *dst =
                (__attribute__((address_space(3))) void *)(&As[st][blk * 4 * 128]);
            const unsigned off = a_off[i];
            __builtin_amdgcn_raw_ptr_buffer_load_lds(a_rs, dst, 16, off, kt * KTILE * 2, 0, 0);
        }
    };
    auto a_frag = [&](const _Float16 *as, int mt, int o) {
        const int r = 16 * mt + c;
        const int pch = (4 * o + kq) ^ c;
        return *reinterpret_cast<const half8 *>(as + r * 128 + pch * 8);
    };
    // ---- codes and scales of this wave's WN n-tiles
    uint4v wreg[WN];
    uint16_t sreg[WN];
    const int ntw = active ? ntile0 : 0;   // (inactive waves load nothing)
    // first physical tile of the (gate, up) runs; resources in plain
    // variables (a target builtin given an argument whose type depends on a
    // template parameter loses the kernel's host launch stub)
    const int pb0 = GATED ? gated_tile(ntw, 0, Nh16) : ntw, pb1 = GATED ? gated_tile(ntw, 1, Nh16) : ntw;
    auto ptile = [&](int t) { return (odd(t) ? pb1 : pb0) + rel(t); };
    const __amdgpu_buffer_rsrc_t w_rs0 = buffer_rsrc(W + (size_t)pb0 * KT * 64, (size_t)(N / NTILE - pb0) * KT * 1024);
    const __amdgpu_buffer_rsrc_t w_rs1 = buffer_rsrc(W + (size_t)pb1 * KT * 64, (size_t)(N / NTILE - pb1) * KT * 1024);
    const __amdgpu_buffer_rsrc_t s_rs0 = buffer_rsrc(S + pb0 * NTILE, ((size_t)G * N - pb0 * NTILE) * 2);
    const __amdgpu_buffer_rsrc_t s_rs1 = buffer_rsrc(S + pb1 * NTILE, ((size_t)G * N - pb1 * NTILE) * 2);
    const unsigned w_off = (unsigned)lane * 16u, s_off = (unsigned)c * 2u;
    auto load_w = [&](int kt) {
        if (!active) return;
        const int gb = ((kt * KTILE) / g) * N * 2;
#pragma unroll
        for (int t = 0; t < WN; ++t) {
            const __amdgpu_buffer_rsrc_t wr = odd(t) ? w_rs1 : w_rs0;
            const __amdgpu_buffer_rsrc_t sr = odd(t) ? s_rs1 : s_rs0;
            const int wo = (rel(t) * KT + kt) * 1024, so = gb + 32 * rel(t);
            wreg[t] = __builtin_bit_cast(uint4v, __builtin_amdgcn_raw_buffer_load_b128(wr, w_off, wo, 0));
            sreg[t] = __builtin_amdgcn_raw_buffer_load_b16(sr, s_off, so, 0);
        }
    };

    float4v acc[WM][WN];
#pragma unroll
    for (int mt = 0; mt < WM; ++mt)
#pragma unroll
        for (int t = 0; t < WN; ++t) acc[mt][t] = float4v{0.f, 0.f, 0.f, 0.f};
    float4v gsum[GM];
#pragma unroll
    for (int j = 0; j < GM; ++j) gsum[j] = float4v{0.f, 0.f, 0.f, 0.f};
    const half8 ones = {1, 1, 1, 1, 1, 1, 1, 1};
    if (DELTA)
        for (int i = tid; i < BM * WIN; i += 256) asum_win[i] = 0.f;

    // the delta k-step for the window of groups [gw0, gw0 + WIN)
    auto delta_step = [&](int gw0) {
        if (!active) return;
        half8 be[WN];
#pragma unroll
        for (int t = 0; t < WN; ++t) {
            const int colx = ptile(t) * NTILE + c;
#pragma unroll
            for (int s8 = 0; s8 < 8; ++s8) {
                const int gg = gw0 + 8 * (kq & 1) + s8;
                be[t][s8] = gg < G ? __builtin_bit_cast(_Float16, D[(size_t)gg * N + colx])
                                   : (_Float16)0.f;
            }
        }
#pragma unroll
        for (int mt = 0; mt < WM; ++mt) {
            const float *src = &asum_win[(16 * mt + c) * WIN + 8 * (kq & 1)];
            half8 ae;
#pragma unroll
            for (int s8 = 0; s8 < 8; ++s8) {
                const float a = src[s8];
                const _Float16 hi = (_Float16)a;
                ae[s8] = (kq < 2) ? hi : (_Float16)(a - (float)hi);
            }
#pragma unroll
            for (int t = 0; t < WN; ++t) acc[mt][t] = mfma_f16(ae, be[t], acc[mt][t]);
        }
    };

    load_a(0, 0);
    load_w(0);
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    for (int kt = 0; kt < KT; ++kt) {
        const int st = kt & 1;
        uint4v wc[WN];
        half2v s2[WN];
#pragma unroll
        for (int t = 0; t < WN; ++t) {
            wc[t] = wreg[t];
            const _Float16 sh = __builtin_bit_cast(_Float16, sreg[t]);
            s2[t] = half2v{sh, sh};
        }
        // unconditional, clamped: the last k-tile reloads its own tile into
        // the idle buffer (a conditional load would leave the compiler unsure
        // which loads are in flight, and it would drain them all)
        load_a(kt + 1 < KT ? kt + 1 : kt, st ^ 1);
        load_w(kt + 1 < KT ? kt + 1 : kt);
        const _Float16 *as = As[st];
        if (active) {
#define QG_TILED_STEP(O)                                                                      \
    {                                                                                         \
        half8 b[WN];                                                                          \
        _Pragma("unroll") for (int t = 0; t < WN; ++t) b[t] = dequant_scaled<O>(wc[t], s2[t]); \
        _Pragma("unroll") for (int mt = 0; mt < WM; ++mt)                                     \
        {                                                                                     \
            const half8 a = a_frag(as, mt, O);                                                \
            _Pragma("unroll") for (int t = 0; t < WN; ++t) acc[mt][t] = mfma_f16(a, b[t], acc[mt][t]); \
        }                                                                                     \
    }
            QG_TILED_STEP(0)
            QG_TILED_STEP(1)
            QG_TILED_STEP(2)
            QG_TILED_STEP(3)
#undef QG_TILED_STEP
        }
        if (DELTA) {
            // group sums of this wave's GM m-tiles
#pragma unroll
            for (int j = 0; j < GM; ++j) {
                const int mt = GM * wave + j;
#pragma unroll
                for (int o = 0; o < 4; ++o) {
                    const half8 a = a_frag(as, mt, o);
                    gsum[j] = mfma_f16(a, ones, gsum[j]);
                }
            }
            const int gi = (kt * KTILE) / g;
            const bool gend = ((kt + 1) * KTILE) % g == 0;
            if (gend) {
#pragma unroll
                for (int j = 0; j < GM; ++j) {
#pragma unroll
                    for (int r = 0; r < 4; ++r)
                        asum_win[(16 * (GM * wave + j) + 4 * kq + r) * WIN + (gi % WIN)] = gsum[j][r];
                    gsum[j] = float4v{0.f, 0.f, 0.f, 0.f};
                }
            }
        }
        // the direct loads of the next A tile (and the next codes) must have
        // landed before any wave reads them
        __builtin_amdgcn_s_waitcnt(0);
        __syncthreads();
        if (DELTA) {
            const int gi = (kt * KTILE) / g;
            const bool gend = ((kt + 1) * KTILE) % g == 0;
            if (gend && (gi % WIN == WIN - 1 || gi == G - 1)) {
                delta_step(gi - gi % WIN);
                // later groups of the next window overwrite these slots only
                // after the next barrier, when every wave has read them
            }
        }
    }

    if (!active) return;
#pragma unroll
    for (int mt = 0; mt < WM; ++mt)
#pragma unroll
        for (int t = 0; t < WN; t += (GATED ? 2 : 1))
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int row = m0 + 16 * mt + 4 * kq + r;
                if (row >= M) continue;
                if (GATED)
                    C[(size_t)row * (N / 2) + ptile(t) * NTILE + c] =
                        f2h(silu_mul(acc[mt][t][r], acc[mt][t + 1][r]));
                else
                    C[(size_t)row * N + n0 + 16 * t + c] = f2h(acc[mt][t][r]);
            }
}

// ---- tiled kernel, symmetric weights, 128 x 256 tile, ordered schedule ----
// The same tile, operands and arithmetic as w4a16_tiled_kernel<8, 4, false>
// (its output is bit-identical), with the k-tile body laid out by hand: each
// 32-k step reads its eight activation fragments in pairs, one pair ahead of
// the MFMAs that use them, and dequantizes the next step's codes between
// those MFMAs, so that LDS latency and dequantization VALU both hide under
// matrix work.  sched_barrier fences keep the compiler from regrouping the
// pairs.  (x & mask) | 0x6400 is one v_and_or_b32 (the compiler emits an AND
// and an OR when both constants are literals).  Codes and scales of the next
// tile are issued after its activations, so the end-of-tile wait leaves them
// in flight.
__device__ inline unsigned and_or_b32(unsigned x, unsigned m, unsigned c)
{
    unsigned r;
    asm("v_and_or_b32 %0, %1, %2, %3" : "=v"(r) : "v"(x), "s"(m), "v"(c));
    return r;
}

template <int STEP>
__device__ inline half8 dequant_scaled_ao(uint4v w, half2v s2, unsigned magic)
{
    const unsigned xa = (STEP & 1) ? w.z : w.x;
    const unsigned xb = (STEP & 1) ? w.w : w.y;
    const unsigned m = (STEP >= 2) ? 0x00F000F0u : 0x000F000Fu;
    const unsigned p[4] = {and_or_b32(xa, m, magic), and_or_b32(xa >> 8, m, magic),
                           and_or_b32(xb, m, magic), and_or_b32(xb >> 8, m, magic)};
    unsigned out[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const half2v h = __builtin_bit_cast(half2v, p[i]);
        half2v v;
        if (STEP >= 2)
            v = h * half2v{(_Float16)0.0625f, (_Float16)0.0625f} - half2v{(_Float16)72.f, (_Float16)72.f};
        else
            v = h - half2v{(_Float16)1032.f, (_Float16)1032.f};
        out[i] = __builtin_bit_cast(unsigned, v * s2);
    }
    return __builtin_bit_cast(half8, uint4v{out[0], out[1], out[2], out[3]});
}

template <bool GATED>
__global__ __launch_bounds__(256, 2) void w4a16_tiled_sym_kernel(
    const uint16_t *__restrict__ A, const uint4v *__restrict__ W, const uint16_t *__restrict__ S,
    uint16_t *__restrict__ C, int M, int N, int K, int g)
{
    constexpr int WM = 8, WN = 4, BM = 16 * WM, BN = 64 * WN, ABLK = BM / 16;
    __shared__ __attribute__((aligned(16))) _Float16 As[2][BM * 128];

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int c = lane & 15, kq = lane >> 4;
    const int KT = K / KTILE;
    const int m0 = blockIdx.y * BM;
    const int n0 = blockIdx.x * BN + wave * 16 * WN;
    const bool active = n0 < N;
    // waves past the last column load valid columns (their results are not
    // stored) so that every wave issues the same loads
    const int n0c = active ? n0 : N - 16 * WN;
    const int ntile0 = n0c / NTILE;
    const int sh = 16 * (c & 1);
    // GATED: n-tile t is tile t/2 of the gate run at ntile0/2 (t even) or of
    // the up run at N/32 + ntile0/2 (t odd), each with its own resources
    const int Nh16 = N / (2 * NTILE);
    auto odd = [](int t) { return GATED && (t & 1); };
    auto rel = [](int t) { return GATED ? (t >> 1) : t; };
    const int pb0 = GATED ? gated_tile(ntile0, 0, Nh16) : ntile0, pb1 = GATED ? gated_tile(ntile0, 1, Nh16) : ntile0;

    // Buffer loads: a workgroup-uniform resource, a fixed per-lane byte
    // offset and the k-dependent byte offset in a scalar register (no
    // per-lane address arithmetic in the k-loop).  A rows past M read row
    // M-1 (their results are never stored).
    const __amdgpu_buffer_rsrc_t a_rs = buffer_rsrc(A + (size_t)m0 * K, (size_t)(M - m0) * K * 2);
    unsigned a_off[ABLK];
#pragma unroll
    for (int i = 0; i < ABLK; ++i) {
        const int r = (wave * ABLK + i) * 4 + (lane >> 4);
        const int ch = (lane & 15) ^ (r & 15);
        const int row = m0 + r < M ? r : M - 1 - m0;
        a_off[i] = (unsigned)(row * K + ch * 8) * 2u;
    }
    auto load_a = [&](int kt, int st) {
#pragma unroll
        for (int i = 0; i < ABLK; ++i) {
            const int blk = wave * ABLK + i;
            __builtin_amdgcn_raw_ptr_buffer_load_lds(
                a_rs, (__attribute__((address_space(3))) void *)(&As[st][blk * 4 * 128]), 16, a_off[i],
                kt * KTILE * 2, 0, 0);
        }
    };
    auto a_frag = [&](const _Float16 *as, int mt, int o) {
        const int r = 16 * mt + c;
        const int pch = (4 * o + kq) ^ c;
        return *reinterpret_cast<const half8 *>(as + r * 128 + pch * 8);
    };
    uint4v wreg[WN];
    uint32_t sreg[WN];   // aligned scale pair holding this lane's column (half c & 1)
    // (resources in plain variables: a target builtin given an argument whose
    // type depends on a template parameter loses the kernel's host launch stub)
    const __amdgpu_buffer_rsrc_t w_rs0 = buffer_rsrc(W + (size_t)pb0 * KT * 64, (size_t)(N / NTILE - pb0) * KT * 1024);
    const __amdgpu_buffer_rsrc_t w_rs1 = buffer_rsrc(W + (size_t)pb1 * KT * 64, (size_t)(N / NTILE - pb1) * KT * 1024);
    const __amdgpu_buffer_rsrc_t s_rs0 = buffer_rsrc(S + pb0 * NTILE, ((size_t)(K / g) * N - pb0 * NTILE) * 2);
    const __amdgpu_buffer_rsrc_t s_rs1 = buffer_rsrc(S + pb1 * NTILE, ((size_t)(K / g) * N - pb1 * NTILE) * 2);
    const unsigned w_off = (unsigned)lane * 16u;      // this lane's 16 bytes of a code tile
    const unsigned s_off = ((unsigned)c >> 1) * 4u;   // this lane's scale pair within 16 columns
    auto load_w = [&](int kt) {
        const int k = kt < KT ? kt : KT - 1;
        const int gb = ((k * KTILE) / g) * N * 2;      // byte offset of this k-tile's group row
#pragma unroll
        for (int t = 0; t < WN; ++t) {
            const __amdgpu_buffer_rsrc_t wr = odd(t) ? w_rs1 : w_rs0;
            const int wo = (rel(t) * KT + k) * 1024;
            wreg[t] = __builtin_bit_cast(uint4v, __builtin_amdgcn_raw_buffer_load_b128(wr, w_off, wo, 0));
        }
#pragma unroll
        for (int t = 0; t < WN; ++t) {
            const __amdgpu_buffer_rsrc_t sr = odd(t) ? s_rs1 : s_rs0;
            const int so = gb + 32 * rel(t);
            sreg[t] = __builtin_amdgcn_raw_buffer_load_b32(sr, s_off, so, 0);
        }
    };

    float4v acc[WM][WN];
#pragma unroll
    for (int mt = 0; mt < WM; ++mt)
#pragma unroll
        for (int t = 0; t < WN; ++t) acc[mt][t] = float4v{0.f, 0.f, 0.f, 0.f};
    unsigned magic;   // 0x6400 (fp16 1024) in both halves, in a register
    asm volatile("v_mov_b32 %0, 0x64006400" : "=v"(magic));

    load_a(0, 0);
    load_w(0);
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();

    for (int kt = 0; kt < KT; ++kt) {
        const int st = kt & 1;
        uint4v wc[WN];
        half2v s2[WN];
#pragma unroll
        for (int t = 0; t < WN; ++t) {
            wc[t] = wreg[t];
            const _Float16 sv = __builtin_bit_cast(_Float16, (uint16_t)(sreg[t] >> sh));
            s2[t] = half2v{sv, sv};
            pin(wc[t]);
        }
        // take this tile's codes before any new load is issued (the wait for
        // them must not cover the loads below)
        __builtin_amdgcn_sched_barrier(0);
        // next tile: activations first, then codes (the last tile reloads its
        // own activations into the idle buffer, keeping the load count fixed)
        load_a(kt + 1 < KT ? kt + 1 : kt, st ^ 1);
        load_w(kt + 1);
        const _Float16 *as = As[st];
        if (active) {
            half8 bc[WN];
#pragma unroll
            for (int t = 0; t < WN; ++t) bc[t] = dequant_scaled_ao<0>(wc[t], s2[t], magic);
#define QG_SYM_STEP(O)                                                                        \
            {                                                                                 \
                half8 bn[WN];                                                                 \
                half8 af[2][2];                                                               \
                af[0][0] = a_frag(as, 0, O);                                                  \
                af[0][1] = a_frag(as, 1, O);                                                  \
                _Pragma("unroll") for (int p = 0; p < WM / 2; ++p) {                          \
                    if (p + 1 < WM / 2) {                                                     \
                        af[(p + 1) & 1][0] = a_frag(as, 2 * p + 2, O);                        \
                        af[(p + 1) & 1][1] = a_frag(as, 2 * p + 3, O);                        \
                    }                                                                         \
                    _Pragma("unroll") for (int t = 0; t < WN; ++t) {                          \
                        acc[2 * p][t] = mfma_f16(af[p & 1][0], bc[t], acc[2 * p][t]);         \
                        acc[2 * p + 1][t] = mfma_f16(af[p & 1][1], bc[t], acc[2 * p + 1][t]); \
                    }                                                                         \
                    if (O < 3) bn[p] = dequant_scaled_ao<(O + 1) & 3>(wc[p], s2[p], magic);   \
                    __builtin_amdgcn_sched_barrier(0);                                        \
                }                                                                             \
                if (O < 3) {                                                                  \
                    _Pragma("unroll") for (int t = 0; t < WN; ++t) bc[t] = bn[t];             \
                }                                                                             \
            }
            QG_SYM_STEP(0)
            QG_SYM_STEP(1)
            QG_SYM_STEP(2)
            QG_SYM_STEP(3)
#undef QG_SYM_STEP
        }
        // this wave's activation loads of the next tile have landed (only its
        // 2 WN code and scale loads may still be in flight); the barrier then
        // makes every wave's part visible and frees this tile's buffer
        __builtin_amdgcn_s_waitcnt((2 * WN) | (0x7 << 4) | (0xF << 8));
        asm volatile("" ::: "memory");
        __builtin_amdgcn_s_barrier();
        asm volatile("" ::: "memory");
    }
    __builtin_amdgcn_s_waitcnt(0);   // the last (unused) code loads

    if (!active) return;
#pragma unroll
    for (int mt = 0; mt < WM; ++mt)
#pragma unroll
        for (int t = 0; t < WN; t += (GATED ? 2 : 1))
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int row = m0 + 16 * mt + 4 * kq + r;
                if (row >= M) continue;
                if (GATED)
                    C[(size_t)row * (N / 2) + (pb0 + rel(t)) * NTILE + c] =
                        f2h(silu_mul(acc[mt][t][r], acc[mt][t + 1][r]));
                else
                    C[(size_t)row * N + n0 + 16 * t + c] = f2h(acc[mt][t][r]);
            }
}

template <int WM, int WN, bool DELTA, bool GATED>
static hipError_t run_tiled(const uint16_t *A, const uint32_t *W, const uint16_t *S,
                            const uint16_t *D, uint16_t *C, int M, int N, int K, int g,
                            hipStream_t st)
{
    constexpr int BM = 16 * WM, BN = 64 * WN;
    dim3 grid((unsigned)((N + BN - 1) / BN), (unsigned)((M + BM - 1) / BM));
    hipLaunchKernelGGL((w4a16_tiled_kernel<WM, WN, DELTA, GATED>), grid, dim3(256), 0, st, A,
                       reinterpret_cast<const uint4v *>(W), S, D, C, M, N, K, g);
    return hipGetLastError();
}

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
// scaled on its own (any g), 2 = groups of two k-tiles (g = 256), 0 = one
// group (g = K).  Pipeline: MID_STAGES k-tiles in flight.
// A k-tile of A (64 rows, 16 KB) goes straight from global memory to one of
// MID_STAGES LDS buffers (wave w fills rows 16w .. 16w + 15; 16-byte chunk ch
// of row r lands at position ch ^ (r % 16)); codes, scales and deltas of the
// same k-tile go to the matching slot of a register ring.  Each k-tile starts
// with a wait that leaves the later k-tiles' loads in flight and one barrier,
// after which the slot used by the previous k-tile is refilled.
constexpr int MID_STAGES = 4;

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
        const int gb = ((k * KTILE) / g) * N * 2;      // byte offset of this k-tile's group row
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
    auto step = [&](int kt, int slot) {
        constexpr unsigned WAIT = waitcnt_vm((SG - 2) * L);
        __builtin_amdgcn_s_waitcnt(WAIT);
        asm volatile("" ::: "memory");
        __builtin_amdgcn_s_barrier();
        asm volatile("" ::: "memory");
        // nothing that reads this slot's registers moves above the wait
        __builtin_amdgcn_sched_barrier(0);
        kt_ = kt;
        if (GK == 1) {
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
            step(kt + i, i);
            asm volatile("" ::: "memory");
            __builtin_amdgcn_sched_barrier(0);
        }
    }
#pragma unroll
    for (int i = 0; i < SG - 1; ++i)
        if (kt + i < KT) step(kt + i, i);
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
    constexpr int L = 4 + WN + WN + (DELTA ? WN : 0);     // loads per thread and step
    static_assert((SG - 2) * L < 64, "vmcnt holds 6 bits");
    static_assert(SG % 4 == 0, "group parities follow the ring slot");
    // LDS: the ring [SG][2 k-groups][BM * KTILE] fp16, then the group sums
    // shared within a k-group [2 k-groups][2 parities][BM] fp32
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
    uint32_t rs[SG][WN], rd[SG][WN];   // aligned scale / delta pairs (half c & 1)
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
        const int gb = ((k * KTILE) / g) * N * 2;
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

    float4v acc[WM][WN], xl[WM][WN], xh[WM][WN], asum;
    const half8 ones = {1, 1, 1, 1, 1, 1, 1, 1};
    const float4v fzero = {0.f, 0.f, 0.f, 0.f};
    asum = fzero;
#pragma unroll
    for (int mt = 0; mt < WM; ++mt)
#pragma unroll
        for (int t = 0; t < WN; ++t) acc[mt][t] = xl[mt][t] = xh[mt][t] = fzero;
    int st_ = 0;   // the step being computed
    float k16[WN], k1[WN], k2[WN], k2s[WN];   // k2s: k2 of the group whose delta term is pending

    auto compute = [&](int slot, bool first) {
#pragma unroll
        for (int t = 0; t < WN; ++t) {
            const float sv = h2f((uint16_t)(rs[slot][t] >> sh));
            const float dv = DELTA ? h2f((uint16_t)(rd[slot][t] >> sh)) : 0.f;
            k16[t] = sv * 0x1p24f;
            k1[t] = sv * 0x1p20f;
            k2[t] = DELTA ? (dv - 8.0f * sv) : (-8.0f * sv);
            pin(k16[t]); pin(k1[t]); pin(k2[t]);
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
                asum = mfma_f16(a[0], ones, first ? fzero : asum);
                asum = mfma_f16(a[1], ones, asum);
                asum = mfma_f16(a[2], ones, asum);
                asum = mfma_f16(a[3], ones, asum);
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
            *reinterpret_cast<float4v *>(gx + (kg * 2 + par) * BM + 16 * wn + 4 * kq) = asum;
#pragma unroll
        for (int t = 0; t < WN; ++t) k2s[t] = k2[t];
    };
    // the pending delta term of the group published with parity par
    auto delta_term = [&](int par) {
#pragma unroll
        for (int mt = 0; mt < WM; ++mt) {
            const float4v gs = *reinterpret_cast<const float4v *>(gx + (kg * 2 + par) * BM + 16 * mt + 4 * kq);
#pragma unroll
            for (int t = 0; t < WN; ++t)
#pragma unroll
                for (int r = 0; r < 4; ++r) acc[mt][t][r] = __builtin_fmaf(k2s[t], gs[r], acc[mt][t][r]);
        }
    };
    auto sync = [&]() {
        asm volatile("" ::: "memory");
        __builtin_amdgcn_s_barrier();
        asm volatile("" ::: "memory");
    };
    // st: the step, slot = st % SG (st comes in slot order from a multiple of SG)
    auto step = [&](int st, int slot) {
        constexpr unsigned WAIT = waitcnt_vm((SG - 2) * L);
        __builtin_amdgcn_s_waitcnt(WAIT);
        sync();
        // nothing that reads this slot's registers moves above the wait
        __builtin_amdgcn_sched_barrier(0);
        st_ = st;
        if (GK == 1) {
            // groups of one k-tile: the previous step's group gets its delta
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
            step(st + i, i);
            asm volatile("" ::: "memory");
            __builtin_amdgcn_sched_barrier(0);
        }
    }
#pragma unroll
    for (int i = 0; i < SG - 1; ++i)
        if (st + i < nsteps) step(st + i, i);
    __builtin_amdgcn_s_waitcnt(0);   // the last (unused) loads

    // the last group's delta term (one group over all of K: closed here)
    if (GK == 0) close(0);
    const bool last_pending = GK == 0 ? true : (kn == nsteps && kn > 0);
    const int last_par = GK == 1 ? ((nsteps - 1) % SG) & 1 : (((nsteps - 1) % SG) >> 1) & 1;
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
    return run_mid<DELTA, 1, GATED>(A, W, S, D, C, M, N, K, g, st);
}

template <bool DELTA, int GK, bool GATED>
static hipError_t run_mid2(const uint16_t *A, const uint32_t *W, const uint16_t *S,
                           const uint16_t *D, uint16_t *C, int M, int N, int K, int g,
                           hipStream_t st)
{
    constexpr int SG = MID2_STAGES;
    const size_t lds = (size_t)SG * 2 * 64 * KTILE * sizeof(_Float16) + 2 * 2 * 64 * sizeof(float);
    auto kern = w4a16_mid2_kernel<SG, DELTA, GK, GATED>;
    static bool attr_set = false;   // (per instantiation) LDS beyond 64 KB
    if (!attr_set) {
        hipError_t e = hipFuncSetAttribute((const void *)kern,
                                           hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
        if (e != hipSuccess) return e;
        attr_set = true;
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
    return run_mid2<DELTA, 1, GATED>(A, W, S, D, C, M, N, K, g, st);
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
    const bool dl = D && fuse_delta;
    if (gated)
        return dl ? run_mid_g<true, true>(A, W, S, D, C, M, N, K, g, st)
                  : run_mid_g<false, true>(A, W, S, nullptr, C, M, N, K, g, st);
    return dl ? run_mid_g<true, false>(A, W, S, D, C, M, N, K, g, st)
              : run_mid_g<false, false>(A, W, S, nullptr, C, M, N, K, g, st);
}

// Configuration for M >= MID_MIN_M: 0 = mid kernel (64 x 64 tiles),
// 1 = tiled 64 x 128, 2 = tiled 128 x 256.  Measured on MI355X (K 4096-5120,
// N 8192-17408): the big tile is the most efficient per tile and wins once it
// fills whole rounds of two or more workgroups per CU; below that the
// 64 x 128 tile wins while it has >= 512 workgroups; smaller problems need the
// mid kernel's 64 x 64 tiles to keep two waves per SIMD busy.
int tiled_config(int M, int N)
{
    const long big = (long)((M + 127) / 128) * ((N + 255) / 256);
    const long small = (long)((M + 63) / 64) * ((N + 127) / 128);
    if (big >= 512 && (big % 256 == 0 || big >= 1024)) return 2;
    if (small >= 512) return 1;
    return 0;
}

template <bool GATED>
static hipError_t run_tiled_cfg(int cfg, const uint16_t *A, const uint32_t *W, const uint16_t *S,
                                const uint16_t *D, uint16_t *C, int M, int N, int K, int g,
                                bool fuse_delta, hipStream_t st)
{
    const bool dl = D && fuse_delta;
    if (cfg == 0) return launch_w4a16_mid(A, W, S, D, C, M, N, K, g, fuse_delta, st, GATED);
    if (cfg == 1) {
        if (dl) return run_tiled<4, 2, true, GATED>(A, W, S, D, C, M, N, K, g, st);
        return run_tiled<4, 2, false, GATED>(A, W, S, nullptr, C, M, N, K, g, st);
    }
    if (dl) return run_tiled<8, 4, true, GATED>(A, W, S, D, C, M, N, K, g, st);
    dim3 grid((unsigned)((N + 255) / 256), (unsigned)((M + 127) / 128));
    hipLaunchKernelGGL(w4a16_tiled_sym_kernel<GATED>, grid, dim3(256), 0, st, A,
                       reinterpret_cast<const uint4v *>(W), S, C, M, N, K, g);
    return hipGetLastError();
}

hipError_t launch_w4a16_tiled_cfg(int cfg, const uint16_t *A, const uint32_t *W,
                                  const uint16_t *S, const uint16_t *D, uint16_t *C, int M, int N,
                                  int K, int g, bool fuse_delta, hipStream_t st, bool gated)
{
    return gated ? run_tiled_cfg<true>(cfg, A, W, S, D, C, M, N, K, g, fuse_delta, st)
                 : run_tiled_cfg<false>(cfg, A, W, S, D, C, M, N, K, g, fuse_delta, st);
}

// Rows of the first launch when the 128 x 256 tiles would end in a partly
// filled round (two workgroups per CU, 512 per round): that launch covers the
// largest multiple of 128 rows whose tiles fill whole rounds and the rows left
// over go to a second launch with its own configuration (smaller tiles), so
// the last round is not run a quarter full.  M when no split pays.
int tiled_row_split(int M, int N)
{
    constexpr long ROUND = 512;
    const long nbn = (N + 255) / 256, nbm = (M + 127) / 128;
    const long tiles = nbn * nbm;
    const long rem = tiles % ROUND;
    if (tiles < ROUND || rem == 0 || rem > ROUND / 2) return M;
    const long m1 = ((tiles - rem) / nbn) * 128;
    return m1 > 0 && m1 < M ? (int)m1 : M;
}

hipError_t launch_w4a16_tiled(const uint16_t *A, const uint32_t *W, const uint16_t *S,
                              const uint16_t *D, uint16_t *C, int M, int N, int K, int g,
                              bool fuse_delta, hipStream_t st, bool gated)
{
    const int cfg = tiled_config(M, N);
    if (cfg == 2) {
        const int m1 = tiled_row_split(M, N);
        if (m1 < M) {
            hipError_t e = launch_w4a16_tiled_cfg(2, A, W, S, D, C, m1, N, K, g, fuse_delta, st, gated);
            if (e != hipSuccess) return e;
            const int m2 = M - m1;
            const int ldc = gated ? N / 2 : N;   // row stride of the output
            return launch_w4a16_tiled_cfg(tiled_config(m2, N), A + (size_t)m1 * K, W, S, D,
                                          C + (size_t)m1 * ldc, m2, N, K, g, fuse_delta, st, gated);
        }
    }
    return launch_w4a16_tiled_cfg(cfg, A, W, S, D, C, M, N, K, g, fuse_delta, st, gated);
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

size_t w4a16_workspace_bytes(int M, int N, int K)
{
    // the decode kernel's split-K counters and partial sums (M <= 16); the
    // skinny and tiled kernels need none
    return decode_workspace_bytes(M, N, K);
}

template <bool DELTA, bool GATED>
static hipError_t dispatch_skinny(const SkinnyCfg &c, const uint16_t *A, const uint32_t *W,
                                  const uint16_t *S, const uint16_t *D, uint16_t *C, int M, int N,
                                  int K, int g, hipStream_t st)
{
    if (c.S != 1) return hipErrorInvalidConfiguration;
#define QG_SK(MT_, NT_, P_, NWMAX_)                                                             \
    if (c.MT == MT_ && c.NT == NT_ && c.P == P_ && c.nw <= NWMAX_)                              \
        return run_skinny<MT_, NT_, P_, NWMAX_, DELTA, GATED>(c, A, W, S, D, C, M, N, K, g, st);
    QG_SK(1, 2, 2, 8) QG_SK(2, 4, 2, 4) QG_SK(4, 2, 2, 4)
#undef QG_SK
    return hipErrorInvalidConfiguration;
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
    if (use_decode_kernel(M, N, K))
        return launch_w4a16_decode(A, W, S, D, C, M, N, K, g, fuse_delta,
                                   decode_workspace_bytes(M, N, K) ? decode_splits(N, K) : 1, ws,
                                   st);
    return launch_w4a16_skinny_cfg(skinny_config(M, N, K), A, W, S, D, C, M, N, K, g,
                                   fuse_delta, ws, st);
}

// ---- shapes with tails: K or N not a multiple of 128 (the pages' dispatcher
//      requires both; "Gaps and follow-ups" lists the head projection's N
//      as the gap) ----
// The pack pads the weight to [Kp, Np] (codes 8, scales 0); a call copies A
// into the workspace with zero columns up to Kp, runs the GEMM on the padded
// shape, and crops the padded product to C.  All in the workspace after the
// counter region: [counters | GEMM workspace][A padded][C padded].
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
    const size_t gemm = w4a16_workspace_bytes(M, Np, Kp);
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
    const size_t gemm = w4a16_workspace_bytes(M, Np, Kp);
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
// kernel (M <= 16 where it is chosen), otherwise the skinny, mid or tiled
// kernel with the gated epilogue (gated_tile pairs their n-tiles).

bool swiglu_uses_decode(int M, int N, int K) { return M <= 16 && use_decode_kernel(M, 2 * N, K); }

size_t swiglu_workspace_bytes(int M, int N, int K)
{
    // only the decode kernel's split-K needs a workspace
    return swiglu_uses_decode(M, N, K) ? decode_workspace_bytes(M, 2 * N, K) : 0;
}

hipError_t launch_w4a16_swiglu(const uint16_t *A, const uint32_t *W, const uint16_t *S,
                               const uint16_t *D, uint16_t *H, int M, int N, int K, int g,
                               void *ws, hipStream_t st)
{
    const int N2 = 2 * N;
    if (swiglu_uses_decode(M, N, K)) {
        const int ns = decode_workspace_bytes(M, N2, K) ? decode_splits(N2, K) : 1;
        if (ns > 1 && !ws) return hipErrorInvalidValue;
        return D ? run_decode<true, true>(A, W, S, D, H, M, N2, K, g, ns, ws, st)
                 : run_decode<false, true>(A, W, S, nullptr, H, M, N2, K, g, ns, ws, st);
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

// Stage 2: one thread per output cell: C += sum_g a_sum[m,g] * delta[g,n].
__global__ __launch_bounds__(256) void correction_accum_kernel(const float *__restrict__ a_sum,
                                                               const uint16_t *__restrict__ D,
                                                               uint16_t *__restrict__ C, int N,
                                                               int G, size_t total)
{
    size_t idx = (size_t)blockIdx.x * 256 + threadIdx.x;
    if (idx >= total) return;
    const size_t m = idx / N, n = idx % N;
    float corr = 0.f;
    for (int gi = 0; gi < G; ++gi) corr += a_sum[m * G + gi] * h2f(D[(size_t)gi * N + n]);
    C[idx] = f2h(h2f(C[idx]) + corr);
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
    size_t total = (size_t)M * N;
    hipLaunchKernelGGL(correction_accum_kernel, dim3((unsigned)((total + 255) / 256)), dim3(256),
                       0, st, a_sum, D, C, N, G, total);
    return hipGetLastError();
}

} // namespace qg
