// W4A16 tiled kernels for large M (64 x 128 and 128 x 256 tiles, the
// hand-ordered symmetric 128 x 256 kernel) and the rule that picks the tile.
// Per-element dequantization (q - 8) * scale to fp16, fp16 MFMAs; the
// asymmetric term A_group_sum @ delta ("Marlin INT4 on Ada - how it works",
// "The core mismatch: symmetric vs asymmetric") as extra MFMA k-steps.
#include "qg_device.h"
#include "qg_launch.h"

#include <type_traits>

namespace qg {

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
namespace tiled {
constexpr int WIN = 16;                         // groups per correction k-step
}

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

// GPT: weight groups per 128-k tile (1 for g >= 128, 2 for g = 64, 4 for
// g = 32): each 32-k MFMA step lies in one group, so step O dequantizes with
// the scale of group O / (4 / GPT) of the tile, and the group sums of A are
// taken per group.
template <int WM, int WN, bool DELTA, bool GATED, int GPT = 1>
__global__ __launch_bounds__(256, (WM * WN >= 32) ? 2 : 3) void w4a16_tiled_kernel(
    const uint16_t *__restrict__ A, const uint4v *__restrict__ W, const uint16_t *__restrict__ S,
    const uint16_t *__restrict__ D, uint16_t *__restrict__ C, int M, int N, int K, int g, int ldn)
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
    uint16_t sreg[WN][GPT];
    const int ntw = active ? ntile0 : 0;   // (inactive waves load nothing)
    // first physical tile of the (gate, up) runs; resources in plain
    // variables (a target builtin given an argument whose type depends on a
    // template parameter loses the kernel's host launch stub)
    const int pb0 = GATED ? gated_tile(ntw, 0, Nh16) : ntw, pb1 = GATED ? gated_tile(ntw, 1, Nh16) : ntw;
    auto ptile = [&](int t) { return (odd(t) ? pb1 : pb0) + rel(t); };
    const __amdgpu_buffer_rsrc_t w_rs0 = buffer_rsrc(W + (size_t)pb0 * KT * 64, (size_t)(N / NTILE - pb0) * KT * 1024);
    const __amdgpu_buffer_rsrc_t w_rs1 = buffer_rsrc(W + (size_t)pb1 * KT * 64, (size_t)(N / NTILE - pb1) * KT * 1024);
    const __amdgpu_buffer_rsrc_t s_rs0 = buffer_rsrc(S + pb0 * NTILE, ((size_t)(G - 1) * ldn + N - pb0 * NTILE) * 2);
    const __amdgpu_buffer_rsrc_t s_rs1 = buffer_rsrc(S + pb1 * NTILE, ((size_t)(G - 1) * ldn + N - pb1 * NTILE) * 2);
    const unsigned w_off = (unsigned)lane * 16u, s_off = (unsigned)c * 2u;
    auto load_w = [&](int kt) {
        if (!active) return;
        const int gb = ((kt * KTILE) / g) * ldn * 2;
#pragma unroll
        for (int t = 0; t < WN; ++t) {
            const __amdgpu_buffer_rsrc_t wr = odd(t) ? w_rs1 : w_rs0;
            const __amdgpu_buffer_rsrc_t sr = odd(t) ? s_rs1 : s_rs0;
            const int wo = (rel(t) * KT + kt) * 1024, so = gb + 32 * rel(t);
            wreg[t] = __builtin_bit_cast(uint4v, __builtin_amdgcn_raw_buffer_load_b128(wr, w_off, wo, 0));
#pragma unroll
            for (int q = 0; q < GPT; ++q)
                sreg[t][q] = __builtin_amdgcn_raw_buffer_load_b16(sr, s_off, so + q * ldn * 2, 0);
        }
    };

    float4v acc[WM][WN];
#pragma unroll
    for (int mt = 0; mt < WM; ++mt)
#pragma unroll
        for (int t = 0; t < WN; ++t) acc[mt][t] = float4v{0.f, 0.f, 0.f, 0.f};
    float4v gsum[GM][GPT];
#pragma unroll
    for (int j = 0; j < GM; ++j)
#pragma unroll
        for (int q = 0; q < GPT; ++q) gsum[j][q] = float4v{0.f, 0.f, 0.f, 0.f};
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
                be[t][s8] = gg < G ? __builtin_bit_cast(_Float16, D[(size_t)gg * ldn + colx])
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
        half2v s2[WN][GPT];
#pragma unroll
        for (int t = 0; t < WN; ++t) {
            wc[t] = wreg[t];
#pragma unroll
            for (int q = 0; q < GPT; ++q) {
                const _Float16 sh = __builtin_bit_cast(_Float16, sreg[t][q]);
                s2[t][q] = half2v{sh, sh};
            }
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
        _Pragma("unroll") for (int t = 0; t < WN; ++t) b[t] = dequant_scaled<O>(wc[t], s2[t][(O) / (4 / GPT)]); \
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
            // group sums of this wave's GM m-tiles (per group of the tile)
#pragma unroll
            for (int j = 0; j < GM; ++j) {
                const int mt = GM * wave + j;
#pragma unroll
                for (int o = 0; o < 4; ++o) {
                    const half8 a = a_frag(as, mt, o);
                    gsum[j][o / (4 / GPT)] = mfma_f16(a, ones, gsum[j][o / (4 / GPT)]);
                }
            }
            const int gi = (kt * KTILE) / g;
            const bool gend = GPT > 1 || ((kt + 1) * KTILE) % g == 0;
            if (gend) {
#pragma unroll
                for (int j = 0; j < GM; ++j)
#pragma unroll
                    for (int q = 0; q < GPT; ++q) {
#pragma unroll
                        for (int r = 0; r < 4; ++r)
                            asum_win[(16 * (GM * wave + j) + 4 * kq + r) * WIN + ((gi + q) % WIN)] =
                                gsum[j][q][r];
                        gsum[j][q] = float4v{0.f, 0.f, 0.f, 0.f};
                    }
            }
        }
        // the direct loads of the next A tile (and the next codes) must have
        // landed before any wave reads them
        __builtin_amdgcn_s_waitcnt(0);
        __syncthreads();
        if (DELTA) {
            // the tile's last group (a window of WIN groups never splits a tile)
            const int gi = (kt * KTILE) / g + GPT - 1;
            const bool gend = GPT > 1 || ((kt + 1) * KTILE) % g == 0;
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
                    C[(size_t)row * ldn + n0 + 16 * t + c] = f2h(acc[mt][t][r]);
            }
}

// ---- tiled kernel, symmetric weights, 128 x 256 tile, ordered schedule ----
// The same tile, operands and arithmetic as w4a16_tiled_kernel<8, 4, false>
// (its output is bit-identical), with the k-tile body laid out by hand: each
// 32-k step reads its eight activation fragments in pairs, one pair ahead of
// the MFMAs that use them, and dequantizes the next step's codes between
// those MFMAs, so that LDS latency and dequantization VALU both hide under
// matrix work.  sched_barrier fences keep the compiler from regrouping the
// pairs.  (x & mask) | 0x6400 is one v_and_or_b32 (and_or_b32).  Codes and
// scales of the next tile are issued after its activations, so the
// end-of-tile wait leaves them in flight.

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
    uint16_t *__restrict__ C, int M, int N, int K, int g, int ldn)
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
    const __amdgpu_buffer_rsrc_t s_rs0 = buffer_rsrc(S + pb0 * NTILE, ((size_t)(K / g - 1) * ldn + N - pb0 * NTILE) * 2);
    const __amdgpu_buffer_rsrc_t s_rs1 = buffer_rsrc(S + pb1 * NTILE, ((size_t)(K / g - 1) * ldn + N - pb1 * NTILE) * 2);
    const unsigned w_off = (unsigned)lane * 16u;      // this lane's 16 bytes of a code tile
    const unsigned s_off = ((unsigned)c >> 1) * 4u;   // this lane's scale pair within 16 columns
    auto load_w = [&](int kt) {
        const int k = kt < KT ? kt : KT - 1;
        const int gb = ((k * KTILE) / g) * ldn * 2;    // byte offset of this k-tile's group row
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
        debug_stage_sync();
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
                    C[(size_t)row * ldn + n0 + 16 * t + c] = f2h(acc[mt][t][r]);
            }
}

template <int WM, int WN, bool DELTA, bool GATED, int GPT = 1>
static hipError_t run_tiled(const uint16_t *A, const uint32_t *W, const uint16_t *S,
                            const uint16_t *D, uint16_t *C, int M, int N, int K, int g,
                            hipStream_t st, int ldn = -1)
{
    constexpr int BM = 16 * WM, BN = 64 * WN;
    dim3 grid((unsigned)((N + BN - 1) / BN), (unsigned)((M + BM - 1) / BM));
    hipLaunchKernelGGL((w4a16_tiled_kernel<WM, WN, DELTA, GATED, GPT>), grid, dim3(256), 0, st, A,
                       reinterpret_cast<const uint4v *>(W), S, D, C, M, N, K, g, ldn < 0 ? N : ldn);
    return hipGetLastError();
}

// Groups of 64 or 32 (GPT = 2 or 4 groups per k-tile): the generic tiled
// kernels (64 x 128 in place of the mid kernels, except the 8-wave one with
// groups of 64; the generic 128 x 256 in place of the symmetric one).
template <bool GATED, int GPT>
static hipError_t run_tiled_small_groups(int cfg, const uint16_t *A, const uint32_t *W,
                                         const uint16_t *S, const uint16_t *D, uint16_t *C, int M,
                                         int N, int K, int g, bool fuse_delta, hipStream_t st)
{
    const bool dl = D && fuse_delta;
    if (cfg != 2)
        return dl ? run_tiled<4, 2, true, GATED, GPT>(A, W, S, D, C, M, N, K, g, st)
                  : run_tiled<4, 2, false, GATED, GPT>(A, W, S, nullptr, C, M, N, K, g, st);
    return dl ? run_tiled<8, 4, true, GATED, GPT>(A, W, S, D, C, M, N, K, g, st)
              : run_tiled<8, 4, false, GATED, GPT>(A, W, S, nullptr, C, M, N, K, g, st);
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

// ldn: row stride of S, D and C when the launch covers a column range of a
// wider weight (W, S, D and C then point at the range's first column); only
// the tiled kernels with groups of >= 128 take one.
template <bool GATED>
static hipError_t run_tiled_cfg(int cfg, const uint16_t *A, const uint32_t *W, const uint16_t *S,
                                const uint16_t *D, uint16_t *C, int M, int N, int K, int g,
                                bool fuse_delta, hipStream_t st, int ldn = -1)
{
    if (ldn < 0) ldn = N;
    if (ldn != N && (GATED || g < KTILE || cfg == 0)) return hipErrorInvalidValue;
    if (g < KTILE) {
        // groups of 64 on the 8-wave mid kernel (its low- and high-nibble
        // sums are the two groups of a k-tile)
        if (g == KTILE / 2 && cfg == 0 && use_mid2(M, N, K))
            return launch_w4a16_mid(A, W, S, D, C, M, N, K, g, fuse_delta, st, GATED);
        return KTILE / g == 2
                   ? run_tiled_small_groups<GATED, 2>(cfg, A, W, S, D, C, M, N, K, g, fuse_delta, st)
                   : run_tiled_small_groups<GATED, 4>(cfg, A, W, S, D, C, M, N, K, g, fuse_delta, st);
    }
    const bool dl = D && fuse_delta;
    if (cfg == 0) return launch_w4a16_mid(A, W, S, D, C, M, N, K, g, fuse_delta, st, GATED);
    if (cfg == 1) {
        if (dl) return run_tiled<4, 2, true, GATED>(A, W, S, D, C, M, N, K, g, st, ldn);
        return run_tiled<4, 2, false, GATED>(A, W, S, nullptr, C, M, N, K, g, st, ldn);
    }
    if (dl) return run_tiled<8, 4, true, GATED>(A, W, S, D, C, M, N, K, g, st, ldn);
    dim3 grid((unsigned)((N + 255) / 256), (unsigned)((M + 127) / 128));
    hipLaunchKernelGGL(w4a16_tiled_sym_kernel<GATED>, grid, dim3(256), 0, st, A,
                       reinterpret_cast<const uint4v *>(W), S, C, M, N, K, g, ldn);
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

// Columns of the first launch when a column split balances the grid better
// than the row split: the 128 x 256 tiles over the leading columns fill whole
// rounds of 512 workgroups, and the remaining columns (all rows) are exactly
// one round of 512 64 x 128 workgroups, two per CU.  (The row split's second
// launch has 4 x 136 = 544 such workgroups at M = 4096, N = 17408, so 32 CUs
// take a third; that launch is issue-bound, so those CUs set its length.)
// N when no such split exists.  Not for gated pairs or groups below 128.
int tiled_col_split(int M, int N, int g, bool gated)
{
    if (gated || g < KTILE || N % 256) return N;
    const long nbm = (M + 127) / 128, nbn = N / 256;
    for (long nb1 = nbn - 1; nb1 >= 1; --nb1) {
        if ((nb1 * nbm) % 512) continue;
        const int n2 = N - (int)(nb1 * 256);
        const long tail = (long)((M + 63) / 64) * (n2 / 128);
        if (tail == 512 && tiled_config(M, n2) == 1) return (int)(nb1 * 256);
        if (tail > 512) break;
    }
    return N;
}

hipError_t launch_w4a16_tiled(const uint16_t *A, const uint32_t *W, const uint16_t *S,
                              const uint16_t *D, uint16_t *C, int M, int N, int K, int g,
                              bool fuse_delta, hipStream_t st, bool gated)
{
    const int cfg = tiled_config(M, N);
    if (cfg == 2 && tiled_row_split(M, N) < M) {
        const int n1 = tiled_col_split(M, N, g, gated);
        if (n1 < N) {
            hipError_t e = run_tiled_cfg<false>(2, A, W, S, D, C, M, n1, K, g, fuse_delta, st, N);
            if (e != hipSuccess) return e;
            // the remaining strips of 16 columns: KT KB each
            const size_t strip_words = (size_t)(K / KTILE) * 256;
            return run_tiled_cfg<false>(1, A, W + (size_t)(n1 / NTILE) * strip_words, S + n1,
                                        D ? D + n1 : nullptr, C + n1, M, N - n1, K, g, fuse_delta, st, N);
        }
    }
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

} // namespace qg
