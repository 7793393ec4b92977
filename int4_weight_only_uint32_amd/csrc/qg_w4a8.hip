// Grouped W4A8 GEMM: 4-bit weights x per-token int8 activations on int8 MFMA
// with exact int32 accumulation per weight group, then per-group and
// per-token scaling in fp32.  Symmetric weights, (v - 8) s, or asymmetric
// zero-point ones, v s + z = (v - 8) s + delta with delta = z + 8 s: the
// delta term needs only the integer group sums of A, taken exactly on the
// same int8 MFMAs against an all-ones operand (the HyperQwen article's
// verification section, point 2: zero-point uint4 weights with int8
// activations).
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
// Kernel.  Per 128-k tile and n-tile, one 128-bit word of codes per lane
// becomes two 16x16x64 int8 operands of 16*(v-8) by masking and an XOR; A's
// bytes are staged in the same k order.  At the end of each group the int32
// accumulator (exactly 16x the group's integer product) is shifted right by 4,
// optionally stored to acc_debug, and folded into the fp32 accumulator with
// the group scale; the per-token scale is applied last.
#include "qg_device.h"
#include "qg_launch.h"

namespace qg {

// Workgroup: 4 waves over the same 64 rows of one expert; wave w owns NT
// n-tiles.  Each 128-k tile of A (64 rows x 128 int8) is fetched
// row-contiguously by the whole workgroup and stored to LDS in MFMA operand
// order (for lane (row, kq): the 16 bytes k = 8kq..8kq+7 and 32+8kq..39+8kq,
// bytes reordered to match the codes' nibble order; then the same for the
// upper 64 k), double-buffered, one barrier per tile.  The activation
// fragments, codes and group scales of the next P tiles wait in a register
// ring whose loads are unconditional (indices clamped to the last tile), so
// every wait covers only the slot being consumed -- a scale loaded just before
// its use would wait for every load issued before it.  DELTA: the group
// deltas ride in the ring beside the scales, and two more MFMAs per 16-row
// tile and k-tile sum the tile's activations per row.
// GQ: weight groups per k-tile (G1 is then true as well).  GQ = 2 (groups of
// 64): the two 64-k MFMA steps of a k-tile are the tile's two groups (the low
// nibbles hold k 0..63 of the tile, the high ones k 64..127).  GQ = 4 (groups
// of 32): each step's operands split into their two 8-byte halves -- bytes
// 0..7 of lane kq hold k 8kq .. 8kq + 7 of the step, bytes 8..15 k 32 + 8kq ..
// 39 + 8kq, on the activation side as on the code side -- so each group of 32
// is one 16x16x32 int8 MFMA on one half.  Each group's product is scaled on
// its own.
template <int NT, int P, bool DEBUG, bool G1, bool DELTA, int GQ = 1>
__global__ __launch_bounds__(256, 2) void w4a8_kernel(
    const int8_t *__restrict__ Aq, const float *__restrict__ a_scale,
    const uint4v *__restrict__ Wall, const uint16_t *__restrict__ Sall,
    const uint16_t *__restrict__ Dall, const int32_t *__restrict__ offsets, int M_total,
    int N, int K, int g,
    uint16_t *__restrict__ C, int32_t *__restrict__ acc_debug)
{
    constexpr int MT = 4;                                  // 64 rows
    // [stage][row][op][kq] x 16 bytes; kq position swizzled with row bits
    __shared__ __attribute__((aligned(16))) uint4v As[2][64 * 8];

    const int e = blockIdx.z;
    int r0 = 0, r1 = M_total;
    if (offsets) {
        r0 = offsets[e];
        r1 = offsets[e + 1];
        r0 = r0 < 0 ? 0 : (r0 > M_total ? M_total : r0);
        r1 = r1 < r0 ? r0 : (r1 > M_total ? M_total : r1);
    }
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int c = lane & 15, kq = lane >> 4;
    const int KT = K / KTILE, G = K / g;
    const int nt0 = (blockIdx.x * 4 + wave) * NT;
    const uint4v *W = Wall + (size_t)e * KT * (N / NTILE) * 64;
    const uint16_t *S = Sall + (size_t)e * G * N;
    const uint16_t *D = DELTA ? Dall + (size_t)e * G * N : nullptr;
    const int sh = 16 * (c & 1);

    // The grid's y extent comes from the caller's bound on rows per expert,
    // which the host cannot check against the device offsets: a workgroup
    // takes row blocks y, y + gridDim.y, ... until the expert's rows run out,
    // so an understated bound costs time, never rows.  The exit test is
    // uniform over the workgroup and comes before any barrier of the block.
    for (int mb = blockIdx.y;; mb += gridDim.y) {
        const int m0 = r0 + mb * 16 * MT;
        if (m0 >= r1) break;

        // ---- A staging: thread t copies 2 x 16 bytes: row t/4 (of 64), bytes
        // 32 (t%4) .. 32 (t%4) + 31 of the 128-k tile.  Rows past the expert's
        // last row read that last row (never stored).
        int arow = m0 + (tid >> 2);
        arow = arow < r1 ? arow : r1 - 1;
        // buffer resources with wave-uniform bases: per-lane offsets are 32-bit
        // and the k-tile advance is a scalar offset, so no 64-bit address
        // arithmetic runs per load (reads past a resource's range return 0)
        const __amdgpu_buffer_rsrc_t a_rs = buffer_rsrc(Aq + (size_t)m0 * K, (size_t)(r1 - m0) * K);
        const int a_off = (arow - m0) * K + 32 * (tid & 3);
        // the 32 bytes k0 .. k0+31 (k0 = 32 (t%4)) split into four 8-byte pieces:
        // piece j holds k = k0 + 8j .. k0 + 8j + 7 -> operand op = k0 / 64, slot
        // kq = j, half = (k0 / 32) % 2
        auto slot = [&](int row, int op, int q) { return row * 8 + op * 4 + (q ^ ((row >> 1) & 3)); };
        auto store_a = [&](int st, const uint4v (&areg)[2]) {
            const int row = tid >> 2, k0 = 32 * (tid & 3);
            const int op = k0 / 64, half = (k0 / 32) & 1;
            unsigned d[8] = {areg[0].x, areg[0].y, areg[0].z, areg[0].w,
                             areg[1].x, areg[1].y, areg[1].z, areg[1].w};
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                uint2v piece = {swap_mid_bytes(d[2 * j]), swap_mid_bytes(d[2 * j + 1])};
                *reinterpret_cast<uint2v *>(reinterpret_cast<char *>(&As[st][slot(row, op, j)]) + 8 * half) = piece;
            }
        };

        const int col0 = nt0 * NTILE + c;
        const __amdgpu_buffer_rsrc_t w_rs =
            buffer_rsrc(W + (size_t)nt0 * KT * 64, (size_t)(N / NTILE - nt0) * KT * 1024);
        const __amdgpu_buffer_rsrc_t s_rs = buffer_rsrc(S + nt0 * NTILE, ((size_t)G * N - nt0 * NTILE) * 2);
        const __amdgpu_buffer_rsrc_t d_rs =
            buffer_rsrc(DELTA ? D + nt0 * NTILE : S, DELTA ? ((size_t)G * N - nt0 * NTILE) * 2 : 4);
        const int s_off = (c & ~1) * 2;     // this lane's column pair, bytes

        float4v accf[MT][NT];
        int4v acci[MT][NT];
        int4v qsum[MT];   // DELTA: the group's activation sums, rows 4 kq + r
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
            qsum[mt] = int4v{0, 0, 0, 0};
#pragma unroll
            for (int t = 0; t < NT; ++t) {
                accf[mt][t] = float4v{0.f, 0.f, 0.f, 0.f};
                acci[mt][t] = int4v{0, 0, 0, 0};
            }
        }

        // register ring: activations, codes, group scales (32-bit pair holding
        // this lane's column, half c & 1)
        uint4v ra[P][2], rw[P][NT];
        uint32_t rs[P][NT][GQ], rd[P][NT][GQ];
        auto load = [&](int kt, int sl) {
            const int k = kt < KT ? kt : KT - 1;
            ra[sl][0] = __builtin_bit_cast(uint4v, __builtin_amdgcn_raw_buffer_load_b128(a_rs, a_off, k * KTILE, 0));
            ra[sl][1] = __builtin_bit_cast(uint4v, __builtin_amdgcn_raw_buffer_load_b128(a_rs, a_off + 16, k * KTILE, 0));
#pragma unroll
            for (int t = 0; t < NT; ++t)
                rw[sl][t] = __builtin_bit_cast(uint4v, __builtin_amdgcn_raw_buffer_load_b128(
                                                           w_rs, (t * KT * 64 + lane) * 16, k * 1024, QG_NT));
            const int so = ((k * KTILE) / g) * N * 2;   // the group's scale row, bytes
#pragma unroll
            for (int t = 0; t < NT; ++t)
#pragma unroll
                for (int q = 0; q < GQ; ++q)
                    rs[sl][t][q] = __builtin_amdgcn_raw_buffer_load_b32(s_rs, s_off + 32 * t, so + q * N * 2, 0);
            if (DELTA) {
#pragma unroll
                for (int t = 0; t < NT; ++t)
#pragma unroll
                    for (int q = 0; q < GQ; ++q)
                        rd[sl][t][q] = __builtin_amdgcn_raw_buffer_load_b32(d_rs, s_off + 32 * t, so + q * N * 2, 0);
            }
        };

        auto step = [&](int kt, int sl) {
            const int st = kt & 1;
            store_a(st, ra[sl]);
            CodeOpsI8 b[NT];
            float sv[NT][GQ], dv[NT][GQ];
#pragma unroll
            for (int t = 0; t < NT; ++t) {
                b[t] = split_codes_i8(rw[sl][t]);
                pin(b[t].op[0]);
                pin(b[t].op[1]);
#pragma unroll
                for (int q = 0; q < GQ; ++q) {
                    sv[t][q] = h2f((uint16_t)(rs[sl][t][q] >> sh));
                    dv[t][q] = DELTA ? h2f((uint16_t)(rd[sl][t][q] >> sh)) : 0.0f;
                    pin(sv[t][q]);
                    if (DELTA) pin(dv[t][q]);
                }
            }
            load(kt + P, sl);
            debug_stage_sync();
            __syncthreads();
            int4v alo[MT], ahi[MT];
#pragma unroll
            for (int mt = 0; mt < MT; ++mt) {
                const int row = 16 * mt + c;
                alo[mt] = __builtin_bit_cast(int4v, As[st][slot(row, 0, kq)]);
                ahi[mt] = __builtin_bit_cast(int4v, As[st][slot(row, 1, kq)]);
            }
            if (GQ > 1) {
                // several groups per k-tile: group q's product (and activation
                // sums) from its own MFMA: the 64-k step q (GQ = 2) or half q % 2
                // of step q / 2 (GQ = 4)
                const int4v z4 = {0, 0, 0, 0};
                const int4v ones = {0x01010101, 0x01010101, 0x01010101, 0x01010101};
                auto group_mfma = [&](int q, int4v a_lo, int4v a_hi, int4v b_lo, int4v b_hi) {
                    const int4v av = q * 2 / GQ == 0 ? a_lo : a_hi;
                    const int4v bv = q * 2 / GQ == 0 ? b_lo : b_hi;
                    if (GQ == 2) return mfma_i8(av, bv, z4);
                    return (q & 1) ? mfma_i8_k32(av.z, av.w, bv.z, bv.w, z4)
                                   : mfma_i8_k32(av.x, av.y, bv.x, bv.y, z4);
                };
                const int gi = GQ * kt;
                // group q's scaled product (its delta term follows separately)
                auto group_term = [&](int mt, int t, int q) {
                    const int4v p = group_mfma(q, alo[mt], ahi[mt], b[t].op[0], b[t].op[1]);
                    if (DEBUG) {
                        const int4v pq = p >> 4;   // exact: multiples of 16
                        accf[mt][t] += sv[t][q] * __builtin_convertvector(pq, float4v);
#pragma unroll
                        for (int r = 0; r < 4; ++r) {
                            const int row = m0 + 16 * mt + 4 * kq + r;
                            if (row < r1)
                                acc_debug[((size_t)row * G + gi + q) * N + col0 + 16 * t] = pq[r];
                        }
                    } else {
                        accf[mt][t] += (sv[t][q] * 0.0625f) * __builtin_convertvector(p, float4v);
                    }
                };
                if (GQ == 2) {
                    // every m-tile's two activation sums first, then n-tile by n-tile
                    int4v qs[MT][GQ];
#pragma unroll
                    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
                        for (int q = 0; q < GQ; ++q) qs[mt][q] = DELTA ? group_mfma(q, alo[mt], ahi[mt], ones, ones) : z4;
#pragma unroll
                    for (int t = 0; t < NT; ++t)
#pragma unroll
                        for (int mt = 0; mt < MT; ++mt) {
#pragma unroll
                            for (int q = 0; q < GQ; ++q) group_term(mt, t, q);
#pragma unroll
                            for (int q = 0; q < GQ; ++q)
                                if (DELTA) accf[mt][t] += dv[t][q] * __builtin_convertvector(qs[mt][q], float4v);
                        }
                } else {
                    // m-tile by m-tile: its four sums live across its n-tiles only
                    // (all sixteen at once would spill)
#pragma unroll
                    for (int mt = 0; mt < MT; ++mt) {
                        int4v qs[GQ];
#pragma unroll
                        for (int q = 0; q < GQ; ++q) qs[q] = DELTA ? group_mfma(q, alo[mt], ahi[mt], ones, ones) : z4;
#pragma unroll
                        for (int t = 0; t < NT; ++t) {
#pragma unroll
                            for (int q = 0; q < GQ; ++q) group_term(mt, t, q);
#pragma unroll
                            for (int q = 0; q < GQ; ++q)
                                if (DELTA) accf[mt][t] += dv[t][q] * __builtin_convertvector(qs[q], float4v);
                        }
                    }
                }
                return;
            }
            // G1 (one k-tile per group): each tile's group sum starts from a zero
            // MFMA operand, so nothing is reset and nothing stays live across tiles
            const int4v zero4 = {0, 0, 0, 0};
            if (DELTA) {
                // sum over k of A[row, k] * 1: every column of the product holds
                // the row's sum, so each lane gets its own rows' sums
                const int4v ones = {0x01010101, 0x01010101, 0x01010101, 0x01010101};
#pragma unroll
                for (int mt = 0; mt < MT; ++mt) {
                    qsum[mt] = mfma_i8(alo[mt], ones, G1 ? zero4 : qsum[mt]);
                    qsum[mt] = mfma_i8(ahi[mt], ones, qsum[mt]);
                }
            }
#pragma unroll
            for (int t = 0; t < NT; ++t)
#pragma unroll
                for (int mt = 0; mt < MT; ++mt) {
                    acci[mt][t] = mfma_i8(alo[mt], b[t].op[0], G1 ? zero4 : acci[mt][t]);
                    acci[mt][t] = mfma_i8(ahi[mt], b[t].op[1], acci[mt][t]);
                }
            if (G1 || ((kt + 1) * KTILE) % g == 0) {   // end of a weight group
                const int gi = (kt * KTILE) / g;
#pragma unroll
                for (int t = 0; t < NT; ++t) {
                    // acci is exactly 16x the group's integer product; for groups of
                    // up to 1024 k, |acci| <= 16 * 127 * 8 * g < 2^24 and its fp32
                    // conversion is exact, so scaling it by s/16 (exact) gives the
                    // same fma result as scaling acci >> 4 by s (longer groups, e.g.
                    // one per column, round that conversion once: 2^-24 relative)
                    const float sv16 = sv[t][0] * 0.0625f;
#pragma unroll
                    for (int mt = 0; mt < MT; ++mt) {
                        if (DEBUG) {
                            const int4v qv = acci[mt][t] >> 4;   // exact: terms are multiples of 16
                            accf[mt][t] += sv[t][0] * __builtin_convertvector(qv, float4v);
#pragma unroll
                            for (int r = 0; r < 4; ++r) {
                                const int row = m0 + 16 * mt + 4 * kq + r;
                                if (row < r1)
                                    acc_debug[((size_t)row * G + gi) * N + col0 + 16 * t] = qv[r];
                            }
                        } else {
                            accf[mt][t] += sv16 * __builtin_convertvector(acci[mt][t], float4v);
                        }
                        // the delta term: |qsum| <= 127 g < 2^24, exact in fp32
                        if (DELTA) accf[mt][t] += dv[t][0] * __builtin_convertvector(qsum[mt], float4v);
                        if (!G1) acci[mt][t] = int4v{0, 0, 0, 0};
                    }
                }
                if (DELTA && !G1)
#pragma unroll
                    for (int mt = 0; mt < MT; ++mt) qsum[mt] = int4v{0, 0, 0, 0};
            }
        };

#pragma unroll
        for (int i = 0; i < P; ++i) load(i, i);
        int kt = 0;
        for (; kt + P <= KT; kt += P) {
#pragma unroll
            for (int i = 0; i < P; ++i) {
                step(kt + i, i);
                // keep each refill ahead of the loop's back edge and the next
                // slot's work out of this step (the compiler would otherwise fold
                // the last slot's loads into the top of the loop)
                asm volatile("" ::: "memory");
                __builtin_amdgcn_sched_barrier(0);
            }
        }
#pragma unroll
        for (int i = 0; i < P - 1; ++i)
            if (kt + i < KT) step(kt + i, i);

        // C: the 64 x (64 NT) fp16 tile is assembled in LDS (the activation
        // stages are dead once every wave is past its last step) and written
        // as whole 16-byte row pieces; a lane's own 16 x 16 results are two
        // bytes apart in four rows, which as direct stores cost the kernel
        // ~13 % at the expert batch (all workgroups end together)
        constexpr int TW = 4 * NT * NTILE;                    // tile width, columns
        static_assert(64 * TW * 2 <= (int)sizeof(As), "the C tile fits in the A stages");
        uint16_t *ct = reinterpret_cast<uint16_t *>(&As[0][0]);
        __syncthreads();
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int rl = 16 * mt + 4 * kq + r, row = m0 + rl;
                const float as = row < r1 ? a_scale[row] : 0.0f;
#pragma unroll
                for (int t = 0; t < NT; ++t)
                    ct[rl * TW + wave * NT * NTILE + 16 * t + c] = f2h(as * accf[mt][t][r]);
            }
        __syncthreads();
        if ((reinterpret_cast<uintptr_t>(C) & 15) == 0) {
            constexpr int PPR = TW * 2 / 16;                  // 16-byte pieces per row
            const int c0 = blockIdx.x * TW;
#pragma unroll
            for (int j = 0; j < 64 * PPR / 256; ++j) {
                const int idx = tid + 256 * j, rl = idx / PPR, pc = idx % PPR;
                const int row = m0 + rl;
                if (row < r1)
                    *reinterpret_cast<uint4v *>(C + (size_t)row * N + c0 + 8 * pc) =
                        *reinterpret_cast<const uint4v *>(ct + rl * TW + 8 * pc);
            }
        } else {
            // C only 2-byte aligned: the same values, two bytes at a time
            const int c0 = blockIdx.x * TW;
            for (int idx = tid; idx < 64 * TW; idx += 256) {
                const int rl = idx / TW, cc = idx % TW, row = m0 + rl;
                if (row < r1) C[(size_t)row * N + c0 + cc] = ct[idx];
            }
        }
        // the next row block restarts the LDS buffers at stage 0: every wave must
        // be done reading the C tile first
        __syncthreads();
    }
}

template <int NT, int P, bool DEBUG, bool G1, bool DELTA, int GQ = 1>
static hipError_t run_w4a8(const int8_t *Aq, const float *a_scale, const uint32_t *W,
                           const uint16_t *S, const uint16_t *D, const int32_t *offsets, int E,
                           int M_total, int max_rows, int N, int K, int g, uint16_t *C,
                           int32_t *acc_debug, hipStream_t st)
{
    const int NT16 = N / NTILE;
    dim3 grid((unsigned)((NT16 + 4 * NT - 1) / (4 * NT)), (unsigned)((max_rows + 63) / 64), (unsigned)E);
    hipLaunchKernelGGL((w4a8_kernel<NT, P, DEBUG, G1, DELTA, GQ>), grid, dim3(256), 0, st, Aq, a_scale,
                       reinterpret_cast<const uint4v *>(W), S, D, offsets, M_total, N, K, g, C,
                       acc_debug);
    return hipGetLastError();
}

template <bool DEBUG, bool G1, int GQ = 1>
static hipError_t run_w4a8_d(const int8_t *Aq, const float *a_scale, const uint32_t *W,
                             const uint16_t *S, const uint16_t *D, const int32_t *offsets, int E,
                             int M_total, int max_rows, int N, int K, int g, uint16_t *C,
                             int32_t *acc_debug, hipStream_t st)
{
    // N % 128 == 0 -> the n-tile count is a multiple of 8: NT = 2 tiles the
    // columns exactly (4 waves x 2 n-tiles = 128 columns per workgroup).
    // With deltas and groups of several k-tiles the group's activation sums
    // stay live across tiles too: a ring of 2 (204 VGPRs) instead of 3, which
    // would spill at two workgroups per CU.
    return D ? run_w4a8<2, G1 && GQ == 1 ? 3 : 2, DEBUG, G1, true, GQ>(Aq, a_scale, W, S, D, offsets, E, M_total, max_rows, N, K, g, C, acc_debug, st)
             : run_w4a8<2, GQ == 4 ? 2 : 3, DEBUG, G1, false, GQ>(Aq, a_scale, W, S, nullptr, offsets, E, M_total, max_rows, N, K, g, C, acc_debug, st);
}

// ---- shapes with tails (K or N not a multiple of 128): the packs are padded
//      to [Kp, Np] (pack_int4_weights); A_q is copied with zero columns up to
//      Kp into the workspace, the kernel runs on the padded shape into a
//      padded product there, which is cropped to C.  Workspace:
//      [counter region, untouched][A_q padded, 256-aligned][C padded].  The
//      leading region is the W4A16 split-K counters' place in every
//      workspace: W4A8 never writes it, so one workspace can serve W4A16 and
//      W4A8 calls in turn on one stream without a W4A8 call leaving nonzero
//      counters behind for the next split-K W4A16 call. ----
__global__ __launch_bounds__(256) void pad_cols_i8_kernel(const int8_t *__restrict__ A,
                                                          int8_t *__restrict__ Ap, int M, int K,
                                                          int Kp)
{
    const size_t i = (size_t)blockIdx.x * 256 + threadIdx.x;
    if (i >= (size_t)M * Kp) return;
    const size_t m = i / Kp;
    const int k = (int)(i % Kp);
    Ap[i] = k < K ? A[m * K + k] : (int8_t)0;
}

size_t w4a8_tail_workspace_bytes(int M_total, int N, int K, int g)
{
    int Kp, Np, gp;
    padded_shape(K, N, g, &Kp, &Np, &gp);
    return W4A16_WS_COUNTER_BYTES + ((size_t)M_total * Kp + 255) / 256 * 256 +
           (size_t)M_total * Np * sizeof(uint16_t);
}

hipError_t launch_w4a8(const int8_t *Aq, const float *a_scale, const uint32_t *W,
                       const uint16_t *S, const uint16_t *D, const int32_t *offsets, int E,
                       int M_total, int max_rows, int N, int K, int g, uint16_t *C,
                       int32_t *acc_debug, hipStream_t st)
{
    if (g == KTILE / 2) {   // groups of 64
        if (acc_debug)
            return run_w4a8_d<true, true, 2>(Aq, a_scale, W, S, D, offsets, E, M_total, max_rows, N, K, g, C, acc_debug, st);
        return run_w4a8_d<false, true, 2>(Aq, a_scale, W, S, D, offsets, E, M_total, max_rows, N, K, g, C, nullptr, st);
    }
    if (g == KTILE / 4) {   // groups of 32
        if (acc_debug)
            return run_w4a8_d<true, true, 4>(Aq, a_scale, W, S, D, offsets, E, M_total, max_rows, N, K, g, C, acc_debug, st);
        return run_w4a8_d<false, true, 4>(Aq, a_scale, W, S, D, offsets, E, M_total, max_rows, N, K, g, C, nullptr, st);
    }
    if (g < KTILE) return hipErrorInvalidValue;   // no other group below a k-tile
    const bool g1 = g == KTILE;
    if (acc_debug)
        return g1 ? run_w4a8_d<true, true>(Aq, a_scale, W, S, D, offsets, E, M_total, max_rows, N, K, g, C, acc_debug, st)
                  : run_w4a8_d<true, false>(Aq, a_scale, W, S, D, offsets, E, M_total, max_rows, N, K, g, C, acc_debug, st);
    return g1 ? run_w4a8_d<false, true>(Aq, a_scale, W, S, D, offsets, E, M_total, max_rows, N, K, g, C, nullptr, st)
              : run_w4a8_d<false, false>(Aq, a_scale, W, S, D, offsets, E, M_total, max_rows, N, K, g, C, nullptr, st);
}

} // namespace qg

namespace qg {

hipError_t launch_w4a8_tail(const int8_t *Aq, const float *a_scale, const uint32_t *W,
                            const uint16_t *S, const uint16_t *D, const int32_t *offsets, int E,
                            int M_total, int max_rows, int N, int K, int g, uint16_t *C, void *ws,
                            hipStream_t st)
{
    if (!ws) return hipErrorInvalidValue;
    int Kp, Np, gp;
    padded_shape(K, N, g, &Kp, &Np, &gp);
    char *base = static_cast<char *>(ws) + W4A16_WS_COUNTER_BYTES;   // past the counters
    int8_t *Ap = reinterpret_cast<int8_t *>(base);
    uint16_t *Cp = reinterpret_cast<uint16_t *>(base + ((size_t)M_total * Kp + 255) / 256 * 256);
    const size_t n = (size_t)M_total * Kp;
    hipLaunchKernelGGL(pad_cols_i8_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st, Aq,
                       Ap, M_total, K, Kp);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    e = launch_w4a8(Ap, a_scale, W, S, D, offsets, E, M_total, max_rows, Np, Kp, gp, Cp, nullptr, st);
    if (e != hipSuccess) return e;
    return launch_crop_cols(Cp, C, M_total, N, Np, st);
}

} // namespace qg
