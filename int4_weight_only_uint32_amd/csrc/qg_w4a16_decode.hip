// W4A16 decode kernel (M <= 16, and up to 80 with several m-tiles):
// activation tile shared through LDS, split-K
// with a last-arriver reduction.  Arithmetic ("Marlin INT4 on Ada - how it
// works", "The core mismatch: symmetric vs asymmetric"): with one m-tile as in
// the skinny kernel, codes as exact fp16 subnormals in the MFMAs, group scale
// and delta applied on the fp32 accumulators; with several, the weights
// (v - 8) s + delta dequantized to fp16 in registers (DQ below).
#include "qg_device.h"
#include "qg_launch.h"

#include <type_traits>

namespace qg {

// ---- decode kernel (decode-size batches) ----
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
// GPT: weight groups per 128-k tile (1 for g >= 128; 2 for g = 64, 4 for
// g = 32).  Each 32-k MFMA step lies inside one group (the packed layout puts
// k-steps 0, 1 in the low nibbles and 2, 3 in the high ones), so with g = 64
// the low- and high-nibble products are the two groups' and with g = 32 each
// step's product is its own group's; the group sums of A split the same way.
// MT: 16-row m-tiles (M <= 16 MT).  Each k-tile of A is 16 MT rows (MT
// 16-byte loads per thread), every wave multiplies each of its code tiles
// into all MT m-tiles, and the split-K slots hold 16 MT rows.
// DQ: the codes are instead dequantized in registers to binary16 weights
// (v - 8) s + delta (one rounding, v_pk_fma_f16; the group's scale and delta
// from the table) and the MFMAs accumulate the product itself: no group sums
// of A and no scaling of the accumulators, for about 16 more VALU
// instructions per code tile, which the MT m-tiles share.
template <int NT, int P, int WV, bool DELTA, bool GATED = false, int GPT = 1, int MT = 1, bool DQ = false>
__global__ __launch_bounds__(64 * WV) void w4a16_decode_kernel(
    const uint16_t *__restrict__ A, const uint4v *__restrict__ W, const uint16_t *__restrict__ S,
    const uint16_t *__restrict__ D, uint16_t *__restrict__ C, int M, int N, int K, int g,
    int nsplit, int cg_main, int nsplit2, unsigned *__restrict__ counters, float *__restrict__ partials,
    int ldc, int ncols)
{
    static_assert(NT == 1, "the scale table holds one column per lane");
    static_assert(WV == 4 || WV == 8, "4 or 8 waves per workgroup");
    static_assert(!GATED || WV == 4, "the gate/up pairing takes 4 waves");
    static_assert(MT == 1 || WV == 4, "several m-tiles take 4 waves");
    constexpr int COLS = 16 * WV;            // columns per workgroup
    __shared__ __attribute__((aligned(16))) _Float16 As[2][MT * 16 * KTILE];
    __shared__ unsigned arrived;
    __shared__ float xch[GATED ? MT * 2 * 4 * 64 : 1];   // up values for the gate waves
    // (scale | delta << 16) of this workgroup's 64 columns for every group its
    // k-range touches: filled once, read once per k-tile (an LDS read instead
    // of two global loads per k-tile)
    extern __shared__ uint32_t sdt[];
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int c = lane & 15, kq = lane >> 4;
    const int KT = K / KTILE;
    // column groups below cg_main take nsplit splits, the others nsplit2
    // (shorter) ones; workgroup b1 + j is split j % nsplit2 of tail column
    // group j / nsplit2.  slot0: the column group's first partial-sum slot
    // (the main column groups need none when nsplit == 1).
    const int b1 = cg_main * nsplit;
    const bool tail_cg = (int)blockIdx.x >= b1;
    const int ns = tail_cg ? nsplit2 : nsplit;
    const int cg = tail_cg ? cg_main + ((int)blockIdx.x - b1) / nsplit2 : (int)blockIdx.x / nsplit;
    const int sp = tail_cg ? (int)blockIdx.x - b1 - (cg - cg_main) * nsplit2 : (int)blockIdx.x - cg * nsplit;
    const int slot0 = tail_cg ? (nsplit > 1 ? b1 : 0) + (cg - cg_main) * nsplit2 : cg * nsplit;
    const int kt_beg = (sp * KT) / ns, kt_end = ((sp + 1) * KT) / ns;
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
    const int ng = n > 0 ? (kt_end * KTILE - 1) / g - gi0 + 1 : 0;
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

    // activation tile (16 MT rows x 256 bytes): with 4 waves thread t fetches
    // rows t/16 + 16 i (i < MT), 16-byte chunk t%16; with 8 waves row t/32,
    // 8-byte piece t%32.
    // A 16-byte chunk lands at position chunk ^ row within its 256-byte LDS
    // row so the 16 rows an MFMA operand reads fall in distinct banks.
    using AVec = typename std::conditional<WV == 4, uint4v, uint2v>::type;
    constexpr int APR = 256 / sizeof(AVec);      // pieces per row
    const int arow_i = tid / APR, apc = tid % APR;
    // loads through buffer resources: a uniform base, a fixed per-lane byte
    // offset and the k-tile's offset in a scalar register.  Rows past M get
    // an offset beyond the resource's range, so their loads return zeros
    // without a memory access (those rows' results are never stored).
    const __amdgpu_buffer_rsrc_t a_rs = buffer_rsrc(A, (size_t)M * K * 2);
    const int ach = apc * (int)sizeof(AVec) / 16, asub = (apc * (int)sizeof(AVec) % 16) / 2;
    unsigned a_off[MT];
    int adst[MT];
#pragma unroll
    for (int i = 0; i < MT; ++i) {
        const int row = arow_i + 16 * i;
        a_off[i] = row < M ? (unsigned)(row * K) * 2u + (unsigned)(apc * (int)sizeof(AVec)) : 0x80000000u;
        adst[i] = row * KTILE + 8 * (ach ^ (row & 15)) + asub;
    }
    const __amdgpu_buffer_rsrc_t w_rs = buffer_rsrc(W + (size_t)nt0 * KT * 64, (size_t)NT * KT * 1024);
    const unsigned w_off = (unsigned)lane * 16u;
    const int gbase = (kt_beg * KTILE) / g;

    // DQ: k-steps 0, 1 accumulate into acc, 2, 3 into acc2 (two short MFMA
    // chains per k-tile instead of one of four), added after the loop
    float4v acc[MT][NT], acc2[DQ ? MT : 1][NT];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int t = 0; t < NT; ++t) {
            acc[mt][t] = float4v{0.f, 0.f, 0.f, 0.f};
            if (DQ) acc2[mt][t] = float4v{0.f, 0.f, 0.f, 0.f};
        }
    unsigned mag_lo = 0, mag_hi = 0;   // DQ: center_codes' constants in vector registers
    if (DQ) {
        asm volatile("v_mov_b32 %0, 0x64006400" : "=v"(mag_lo));
        asm volatile("v_mov_b32 %0, 0x54005400" : "=v"(mag_hi));
    }
    const half8 ones = {1, 1, 1, 1, 1, 1, 1, 1};
    const float4v fzero = {0.f, 0.f, 0.f, 0.f};

    AVec ra[P][MT];
    uint4v rw[P][NT];
    auto load = [&](int kt, AVec (&a)[MT], uint4v (&w)[NT]) {
#pragma unroll
        for (int i = 0; i < MT; ++i) {
            if constexpr (WV == 4)
                a[i] = __builtin_bit_cast(uint4v, __builtin_amdgcn_raw_buffer_load_b128(a_rs, a_off[i], kt * KTILE * 2, 0));
            else
                a[i] = __builtin_bit_cast(uint2v, __builtin_amdgcn_raw_buffer_load_b64(a_rs, a_off[i], kt * KTILE * 2, 0));
        }
#pragma unroll
        for (int t = 0; t < NT; ++t)
            w[t] = __builtin_bit_cast(uint4v, __builtin_amdgcn_raw_buffer_load_b128(w_rs, w_off, (t * KT + kt) * 1024, QG_NT));
    };
    auto finish = [&](int buf, int kt, const CodeOps (&ops)[NT]) {
    if constexpr (DQ) {
        // the binary16 weights of the tile's four k-steps, each step with its
        // group's scale and delta (both halves of a register alike)
        const uint32_t *sdp = &sdt[((kt * KTILE) / g - gbase) * COLS + 16 * wave + c];
        half8 bq[NT][4];
#pragma unroll
        for (int q = 0; q < GPT; ++q) {
            const uint32_t sd = sdp[q * COLS];
            const half2v s2 = __builtin_bit_cast(half2v, __builtin_amdgcn_perm(sd, sd, 0x01000100u));
            const half2v d2 = __builtin_bit_cast(half2v, __builtin_amdgcn_perm(sd, sd, 0x03020302u));
#pragma unroll
            for (int t = 0; t < NT; ++t) {
                const half8 cs[4] = {ops[t].lo[0], ops[t].lo[1], ops[t].hi[0], ops[t].hi[1]};
#pragma unroll
                for (int k = q * (4 / GPT); k < (q + 1) * (4 / GPT); ++k) {
                    const uint4v cw = __builtin_bit_cast(uint4v, cs[k]);
                    unsigned out[4];
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        // the element through a scalar: a bit_cast of a vector
                        // element reads element 0 with this compiler
                        const unsigned e = cw[i];
                        const half2v v = __builtin_bit_cast(half2v, e);
                        out[i] = __builtin_bit_cast(unsigned, DELTA ? __builtin_elementwise_fma(v, s2, d2) : v * s2);
                    }
                    bq[t][k] = __builtin_bit_cast(half8, uint4v{out[0], out[1], out[2], out[3]});
                }
            }
        }
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
            half8 a[4];
#pragma unroll
            for (int o = 0; o < 4; ++o)
                a[o] = *reinterpret_cast<const half8 *>(&As[buf][(16 * mt + c) * KTILE + 8 * ((4 * o + kq) ^ c)]);
#pragma unroll
            for (int t = 0; t < NT; ++t) {
                acc[mt][t] = mfma_f16(a[0], bq[t][0], acc[mt][t]);
                acc[mt][t] = mfma_f16(a[1], bq[t][1], acc[mt][t]);
                acc2[mt][t] = mfma_f16(a[2], bq[t][2], acc2[mt][t]);
                acc2[mt][t] = mfma_f16(a[3], bq[t][3], acc2[mt][t]);
            }
        }
        return;
    }
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
        half8 a[4];
#pragma unroll
        for (int o = 0; o < 4; ++o)
            a[o] = *reinterpret_cast<const half8 *>(&As[buf][(16 * mt + c) * KTILE + 8 * ((4 * o + kq) ^ c)]);
        if (GPT > 1) {
            // groups of 64 or 32 k: one scale and delta per group of the tile
            constexpr int SPG = 4 / GPT;                // MFMA steps per group
            const uint32_t *sdp = &sdt[((kt * KTILE) / g - gbase) * COLS + 16 * wave + c];
            float4v as[GPT];
#pragma unroll
            for (int q = 0; q < GPT; ++q) {
                as[q] = mfma_f16(a[SPG * q], ones, fzero);
                if (SPG == 2) as[q] = mfma_f16(a[SPG * q + 1], ones, as[q]);
            }
#pragma unroll
            for (int t = 0; t < NT; ++t) {
                const half8 op[4] = {ops[t].lo[0], ops[t].lo[1], ops[t].hi[0], ops[t].hi[1]};
                float4v x[GPT];
#pragma unroll
                for (int q = 0; q < GPT; ++q) {
                    x[q] = mfma_f16(a[SPG * q], op[SPG * q], fzero);
                    if (SPG == 2) x[q] = mfma_f16(a[SPG * q + 1], op[SPG * q + 1], x[q]);
                }
#pragma unroll
                for (int q = 0; q < GPT; ++q) {
                    const uint32_t sd = sdp[q * COLS];
                    const float s = h2f((uint16_t)(sd & 0xFFFFu));
                    const float d = DELTA ? h2f((uint16_t)(sd >> 16)) : 0.f;
                    // steps 0, 1 hold low nibbles (2^-24 v), steps 2, 3 high ones (2^-20 v)
                    const float cx = s * (SPG * q < 2 ? 0x1p24f : 0x1p20f);
                    const float c2 = DELTA ? (d - 8.0f * s) : (-8.0f * s);
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        const float v = __builtin_fmaf(cx, x[q][r], acc[mt][t][r]);
                        acc[mt][t][r] = __builtin_fmaf(c2, as[q][r], v);
                    }
                }
            }
            continue;
        }
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
                float v = __builtin_fmaf(c16, xl[r], acc[mt][t][r]);
                v = __builtin_fmaf(c1, xh[r], v);
                acc[mt][t][r] = __builtin_fmaf(c2, as[r], v);
            }
        }
    }
    };
    auto step = [&](int kt, int slot, int kt_next) {
        const int buf = (kt - kt_beg) & 1;
#pragma unroll
        for (int i = 0; i < MT; ++i) *reinterpret_cast<AVec *>(&As[buf][adst[i]]) = ra[slot][i];
        CodeOps ops[NT];
#pragma unroll
        for (int t = 0; t < NT; ++t) {
            ops[t] = DQ ? center_codes(rw[slot][t], mag_lo, mag_hi) : split_codes(rw[slot][t]);
            pin(ops[t].lo[0]); pin(ops[t].lo[1]); pin(ops[t].hi[0]); pin(ops[t].hi[1]);
        }
        // unconditional (clamped) refill: a conditional load would make every
        // later wait assume it might be missing and wait for everything
        load(kt_next, ra[slot], rw[slot]);
        debug_stage_sync();
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
    if (DQ)
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
#pragma unroll
            for (int t = 0; t < NT; ++t) acc[mt][t] += acc2[mt][t];

    // C rows 16 mt + 4 kq + r, columns (nt0 + t) * 16 + c below ncols, row
    // stride ldc (a padded weight writes its logical columns straight into
    // the caller's C); GATED: silu(gate) * up into C [M, Nh] by the gate
    // waves (reached by every thread of the workgroup, or of none: the
    // barrier is uniform)
    auto store = [&](const float4v (&v)[MT][NT]) {
        if (GATED) {
            if (wave >= 2)
#pragma unroll
                for (int mt = 0; mt < MT; ++mt)
#pragma unroll
                    for (int r = 0; r < 4; ++r) xch[((mt * 2 + wave - 2) * 4 + r) * 64 + lane] = v[mt][0][r];
            __syncthreads();
            if (wave < 2)
#pragma unroll
                for (int mt = 0; mt < MT; ++mt)
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        const int row = 16 * mt + 4 * kq + r;
                        const float gv = v[mt][0][r], u = xch[((mt * 2 + wave) * 4 + r) * 64 + lane];
                        if (row < M) C[(size_t)row * Nh + col0] = f2h(silu_mul(gv, u));
                    }
            return;
        }
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
#pragma unroll
            for (int t = 0; t < NT; ++t)
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int row = 16 * mt + 4 * kq + r;
                    const int col = col0 + 16 * t;
                    if (row < M && col < ncols) C[(size_t)row * ldc + col] = f2h(v[mt][t][r]);
                }
    };
    if (ns == 1) {
        store(acc);
        return;
    }
    // slot layout: [cg][split][wave][mt][t][r][lane] fp32
    constexpr int PER_WAVE = MT * NT * 4 * 64;
    float *mine = partials + ((size_t)slot0 + sp) * WV * PER_WAVE + wave * PER_WAVE + lane;
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int t = 0; t < NT; ++t)
#pragma unroll
            for (int r = 0; r < 4; ++r)
                __hip_atomic_store(mine + ((mt * NT + t) * 4 + r) * 64, acc[mt][t][r], __ATOMIC_RELAXED,
                                   __HIP_MEMORY_SCOPE_AGENT);
    __builtin_amdgcn_s_waitcnt(0);          // this thread's slot stores are complete
    __syncthreads();                        // ... and every thread's
    if (tid == 0)
        arrived = __hip_atomic_fetch_add(&counters[cg], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __syncthreads();
    if (arrived != (unsigned)(ns - 1)) return;
    float4v tot[MT][NT];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int t = 0; t < NT; ++t) tot[mt][t] = fzero;
    const float *base = partials + (size_t)slot0 * WV * PER_WAVE + wave * PER_WAVE + lane;
    for (int s2 = 0; s2 < ns; ++s2) {
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
#pragma unroll
            for (int t = 0; t < NT; ++t)
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    tot[mt][t][r] += (s2 == sp) ? acc[mt][t][r]
                                                : __hip_atomic_load(base + (size_t)s2 * WV * PER_WAVE + ((mt * NT + t) * 4 + r) * 64,
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
    if (g < KTILE) return span * (KTILE / g);             // whole groups per k-tile
    const int per_group = g / KTILE;                      // k-tiles per group
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

int decode_splits(int N, int K, int g)
{
    const int KT = K / KTILE, ncg = N / decode::COLS;
    int ns = 1;
    if ((size_t)ncg * sizeof(unsigned) > W4A16_WS_COUNTER_BYTES) return 1;   // no counter for it
    if (const int fit = decode_balanced_splits(N, K))
        ns = fit;
    else
        while (ns < 16 && (long)ncg * ns < 512 && KT / (2 * ns) >= 2) ns *= 2;
    // the table's largest size over group sizes >= 128 is that of g = 128
    const int gt = g < KTILE ? g : KTILE;
    while (ns < 1024 && (size_t)decode_max_groups(K, gt, ns) * decode::COLS * 4 > 32768) ns *= 2;
    return ns;
}

// Grid balance.  All decode workgroups are resident at once, and a CU that
// holds one workgroup more than most finishes last.  When the plain grid
// (ncg column groups x ns splits) leaves a small remainder over whole rounds
// of 256 CUs (at most 64 workgroups), the column groups that fill those rounds
// keep ns splits and the remaining ones take F x ns shorter splits, so the CUs
// that get an extra workgroup get a fraction of one.  F is the largest of 8,
// 4, 2 whose splits still stream >= 10 k-tiles (M <= 8, where a workgroup's
// fixed costs weigh more) or >= 5 k-tiles (larger M), with <= 256 such
// workgroups.  Same arithmetic and reduction order per column group.
// Measured (M = 16 / 1 / 64 on K5120 x N17408: 544 workgroups, 32 CUs holding
// three): F = 1 15.15 / 13.37 / 30.50 us, F = 2 14.11 / 12.56 / 26.45, F = 4
// 13.97 / 13.06 / 25.63, F = 8 16.63 / 16.04 / 28.79.
DecodeGrid decode_grid(int M, int N, int K, int ns)
{
    const int ncg = N / decode::COLS, KT = K / KTILE;
    DecodeGrid d{ncg, ns, ncg * ns, ns > 1 ? ncg * ns : 0};
    const int full = (d.wgs / 256) * 256;
    const int rem = d.wgs - full;
    if (full == 0 || rem == 0 || rem > 64) return d;
    const int main = full / ns;
    if (main < 1 || main >= ncg) return d;
    const int kmin = M <= 8 ? 10 : 5;
    for (int F = 8; F >= 2; F /= 2) {
        const int ns2 = ns * F;
        if (KT / ns2 < kmin || (ncg - main) * ns2 > 256) continue;
        d.cg_main = main;
        d.ns2 = ns2;
        d.wgs = main * ns + (ncg - main) * ns2;
        d.slots = (ns > 1 ? main * ns : 0) + (ncg - main) * ns2;
        return d;
    }
    return d;
}

// Decode workspace: the fixed counter region (W4A16_WS_COUNTER_BYTES, shared
// by every W4A16 layout and written by nothing but the counters), then the
// partial-sum slots.  0 when the shape is not split.
// Whether a shape runs the decode kernel rather than the skinny one.  M <= 16
// (against the skinny kernel, which
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
// 17 <= M <= 80 (several m-tiles): whether the decode kernel beats
// the skinny kernel, whose waves each stage their own activation rows (16 MT
// rows per k-tile) where the decode kernel's four waves share one tile.
// Measured on MI355X (A/B in one process, µs skinny -> decode): two m-tiles
// always (K4096 N4096 M32 13.0 -> 11.7, K2048 N2048 M32 9.4 -> 9.3, K5120
// N17408 M32 30.4 -> 23.0); three to five when the weight has more than 2^24
// elements (K5120 N17408 M80 77.1 -> 40.8, K4096 N8192 M48 16.6 -> 14.1,
// K5120 N5120 M64 18.1 -> 16.3), not at or below it (K4096 N4096 M64 15.1
// against 16.6, K2048 N2048 M64 10.7 against 12.9).  Groups of 64 and 32
// alike (g = 64: K5120 N17408 M48 54.3 -> 29.3, K4096 N8192 M64 19.7 ->
// 16.8; g = 32: K4096 N8192 M80 36.8 -> 20.9; K4096 N4096 M33 g = 64 17.6
// either way).  Re-measured with the m-tiles' in-register dequantization:
// the small weights still favour the skinny kernel (K4096 N4096 M64/M80 15.3 /
// 15.6 against 15.8 / 18.3, K2048 N2048 M64 10.7 against 13.0).
static bool decode_multi_tile_pays(int M, int N, int K)
{
    const int mt = (M + 15) / 16;
    return mt <= 2 || (long long)K * N > (1ll << 24);
}

bool use_decode_kernel(int M, int N, int K, int g)
{
    if (M > DECODE_MAX_M || N % decode::COLS) return false;
    if (M > 16) return decode_multi_tile_pays(M, N, K);
    const int ns = decode_splits(N, K, g);
    if (ns <= 2) return true;
    const long skinny_wgs = N / 32;
    if (skinny_wgs > 256) return (long long)K * N >= (1ll << 25);
    return skinny_wgs < 256 && (K / KTILE) / ns >= 16;
}

size_t decode_workspace_bytes(int M, int N, int K, int g)
{
    if (!use_decode_kernel(M, N, K, g)) return 0;
    const size_t slots = (size_t)decode_grid(M, N, K, decode_splits(N, K, g)).slots;
    if (slots == 0) return 0;                                  // nothing split
    const size_t rows = 16 * (size_t)((M + 15) / 16);          // the m-tiles' rows
    return W4A16_WS_COUNTER_BYTES + slots * rows * decode::COLS * sizeof(float);
}

// Whether MT m-tiles dequantize the codes (DQ above): the dequantization is
// shared by the m-tiles, the group sums and scaling it saves are per m-tile.
constexpr bool decode_dq(int MT) { return MT >= 2; }

template <bool DELTA, bool GATED = false, int GPT = 1, int MT = 1>
static hipError_t run_decode(const uint16_t *A, const uint32_t *W, const uint16_t *S,
                             const uint16_t *D, uint16_t *C, int M, int N, int K, int g,
                             int nsplit, void *ws, hipStream_t st, int ldc, int ncols)
{
    const DecodeGrid grid = decode_grid(M, N, K, nsplit);
    unsigned *counters = nullptr;
    float *partials = nullptr;
    if (grid.slots > 0) {
        if (!ws) return hipErrorInvalidValue;
        counters = static_cast<unsigned *>(ws);
        partials = reinterpret_cast<float *>(static_cast<char *>(ws) + W4A16_WS_COUNTER_BYTES);
    }
    const size_t table = (size_t)decode_max_groups(K, g, nsplit) * decode::COLS * sizeof(uint32_t);
    // the kernel's static LDS: two activation tiles, the counter word, the
    // gated hand-over
    constexpr size_t stat = 2 * MT * 16 * KTILE * 2 + 4 + (GATED ? MT * 2 * 4 * 64 * 4 : 4);
    if (table + stat > 64 * 1024) {
        const hipError_t e = hipFuncSetAttribute(
            reinterpret_cast<const void *>(&w4a16_decode_kernel<decode::NT, decode::P, decode::WV, DELTA, GATED, GPT, MT, decode_dq(MT)>),
            hipFuncAttributeMaxDynamicSharedMemorySize, (int)table);
        if (e != hipSuccess) return e;
    }
    hipLaunchKernelGGL((w4a16_decode_kernel<decode::NT, decode::P, decode::WV, DELTA, GATED, GPT, MT, decode_dq(MT)>),
                       dim3(grid.wgs), dim3(64 * decode::WV), table, st, A, reinterpret_cast<const uint4v *>(W), S, D, C, M,
                       N, K, g, nsplit, grid.cg_main, grid.ns2, counters, partials, ldc, ncols);
    return hipGetLastError();
}

hipError_t launch_w4a16_decode(const uint16_t *A, const uint32_t *W, const uint16_t *S,
                               const uint16_t *D, uint16_t *C, int M, int N, int K, int g,
                               bool fuse_delta, int nsplit, void *ws, hipStream_t st,
                               bool gated, int ldc, int ncols)
{
    if (ldc < 0) ldc = gated ? N / 2 : N;
    if (ncols < 0) ncols = gated ? N / 2 : N;
    if (M > DECODE_MAX_M || N % decode::COLS || nsplit < 1 || (nsplit > 1 && !ws) ||
        ncols > (gated ? N / 2 : N) || ldc < ncols || (gated && (ldc != N / 2 || ncols != N / 2)))
        return hipErrorInvalidValue;
    const bool dl = D && fuse_delta;
    const int gpt = g < KTILE ? KTILE / g : 1;
    const int mt = (M + 15) / 16;
#define QG_DEC(GPT_, MT_)                                                                     \
    if (gpt == GPT_ && mt == MT_) {                                                           \
        if (gated)                                                                            \
            return dl ? run_decode<true, true, GPT_, MT_>(A, W, S, D, C, M, N, K, g, nsplit, ws, st, ldc, ncols) \
                      : run_decode<false, true, GPT_, MT_>(A, W, S, nullptr, C, M, N, K, g, nsplit, ws, st, ldc, ncols); \
        return dl ? run_decode<true, false, GPT_, MT_>(A, W, S, D, C, M, N, K, g, nsplit, ws, st, ldc, ncols)   \
                  : run_decode<false, false, GPT_, MT_>(A, W, S, nullptr, C, M, N, K, g, nsplit, ws, st, ldc, ncols); \
    }
    QG_DEC(1, 1) QG_DEC(2, 1) QG_DEC(4, 1)
    QG_DEC(1, 2) QG_DEC(1, 3) QG_DEC(1, 4) QG_DEC(1, 5)
    QG_DEC(2, 2) QG_DEC(2, 3) QG_DEC(2, 4) QG_DEC(2, 5)
    QG_DEC(4, 2) QG_DEC(4, 3) QG_DEC(4, 4) QG_DEC(4, 5)
#undef QG_DEC
    return hipErrorInvalidValue;
}

} // namespace qg
