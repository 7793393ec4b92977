// Internal device helpers of the packed-int4 GEMM library (gfx950 only).
//
// Packed weight layout (this library's own; produced by pack_int4_weights):
//   The K x N code matrix is cut into tiles of 128 k x 16 n.  Tile (nt, kt)
//   occupies 256 consecutive uint32 starting at (nt * (K/128) + kt) * 256, so
//   the tiles of one 16-column strip are contiguous along K.  Inside a tile,
//   "lane" l = 0..63 owns the 16 bytes (4 uint32) at l*4 .. l*4+3: column
//   c = l % 16 of the strip and the k-quarter kq = l / 16.  uint32 j of lane
//   l holds 8 codes; nibble p (bits 4p .. 4p+3) holds k = tile_k(kq, j, p):
//       half = p >> 2, hi = p & 1, sh = (p >> 1) & 1
//       slot = 4 * (j & 1) + 2 * sh + half          (0..7)
//       step = (j >> 1) + 2 * hi                    (0..3)
//       k    = 32 * step + 8 * kq + slot
//   so that one 128-bit load per lane gives a wave the B operands of the four
//   16x16x32 fp16 MFMA k-steps of a 128-k tile, and the nibbles of each
//   operand are reachable with one AND (see split_codes below).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace qg {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef _Float16 half2v __attribute__((ext_vector_type(2)));
typedef float float4v __attribute__((ext_vector_type(4)));
typedef int int4v __attribute__((ext_vector_type(4)));
typedef unsigned int uint4v __attribute__((ext_vector_type(4)));
typedef unsigned int uint2v __attribute__((ext_vector_type(2)));

constexpr int KTILE = 128;    // k extent of one packed tile
constexpr int NTILE = 16;     // n extent of one packed tile
constexpr int TILE_U32 = 256; // uint32 per tile

__host__ __device__ inline int tile_k(int kq, int j, int p)
{
    int half = p >> 2, hi = p & 1, sh = (p >> 1) & 1;
    int slot = 4 * (j & 1) + 2 * sh + half;
    int step = (j >> 1) + 2 * hi;
    return 32 * step + 8 * kq + slot;
}

__device__ inline float h2f(uint16_t b) { return (float)__builtin_bit_cast(_Float16, b); }
__device__ inline uint16_t f2h(float f) { return __builtin_bit_cast(uint16_t, (_Float16)f); }

// Strictly negative binary16 (not -0.0, not NaN).
__host__ __device__ inline bool f16_is_negative(uint16_t b)
{
    bool nan = (b & 0x7c00) == 0x7c00 && (b & 0x03ff) != 0;
    return (b & 0x8000) && (b & 0x7fff) && !nan;
}

// ---- fp16 B operands from one 128-bit group of codes (subnormal form) ----
// A binary16 bit pattern 0x000v (v < 16) is the subnormal v * 2^-24 and a
// pattern 0x00v0 is 16 v * 2^-24; both are exact MFMA inputs.  The four words
// x0..x3 of a lane give four operands:
//   lo[0] (k-step 0), lo[1] (k-step 1): values v * 2^-24
//   hi[0] (k-step 2), hi[1] (k-step 3): values 16 v * 2^-24
struct CodeOps {
    half8 lo[2];
    half8 hi[2];
};

__device__ inline CodeOps split_codes(uint4v w)
{
    CodeOps r;
    uint4v l0, l1, h0, h1;
    unsigned x0 = w.x, x1 = w.y, x2 = w.z, x3 = w.w;
    unsigned y0 = x0 >> 8, y1 = x1 >> 8, y2 = x2 >> 8, y3 = x3 >> 8;
    l0 = uint4v{x0 & 0x000F000Fu, y0 & 0x000F000Fu, x1 & 0x000F000Fu, y1 & 0x000F000Fu};
    l1 = uint4v{x2 & 0x000F000Fu, y2 & 0x000F000Fu, x3 & 0x000F000Fu, y3 & 0x000F000Fu};
    h0 = uint4v{x0 & 0x00F000F0u, y0 & 0x00F000F0u, x1 & 0x00F000F0u, y1 & 0x00F000F0u};
    h1 = uint4v{x2 & 0x00F000F0u, y2 & 0x00F000F0u, x3 & 0x00F000F0u, y3 & 0x00F000F0u};
    r.lo[0] = __builtin_bit_cast(half8, l0);
    r.lo[1] = __builtin_bit_cast(half8, l1);
    r.hi[0] = __builtin_bit_cast(half8, h0);
    r.hi[1] = __builtin_bit_cast(half8, h1);
    return r;
}

// ---- int8 B operands from one 128-bit group of codes ----
// Byte b of ((x << 4) & 0xF0F0F0F0) is 16 * (nibble 2b); XOR 0x80 turns the
// unsigned byte 16 v into the signed byte 16 (v - 8).  Likewise for the odd
// nibbles with (x & 0xF0F0F0F0).  Returns the two 16x16x64 int8 operands of
// the tile: [0] covers k-steps 0,1 of the fp16 numbering, [1] k-steps 2,3.
// (x & m) | c as one v_and_or_b32, the mask in a scalar register and c in a
// vector register (with two literal constants the compiler emits an AND and
// an OR)
__device__ inline unsigned and_or_b32(unsigned x, unsigned m, unsigned c)
{
    unsigned r;
    asm("v_and_or_b32 %0, %1, %2, %3" : "=v"(r) : "v"(x), "s"(m), "v"(c));
    return r;
}

// The codes of one lane's 128-bit word as exact binary16 values v - 8, in
// split_codes' operand order (k-steps 0, 1 from the low nibbles, 2, 3 from the
// high ones).  A low nibble ORed into 0x6400 (1024, spacing 1) reads 1024 + v,
// a high nibble (bits 4..7 of a half) ORed into 0x5400 (64, spacing 1/16)
// reads 64 + v, and subtracting 1032 or 72 is exact.  mag_lo, mag_hi: 0x64006400
// and 0x54005400, held in vector registers by the caller.
__device__ inline CodeOps center_codes(uint4v w, unsigned mag_lo, unsigned mag_hi)
{
    const half2v off_lo = {(_Float16)1032.f, (_Float16)1032.f};
    const half2v off_hi = {(_Float16)72.f, (_Float16)72.f};
    auto lo = [&](unsigned x) {
        return __builtin_bit_cast(unsigned, __builtin_bit_cast(half2v, and_or_b32(x, 0x000F000Fu, mag_lo)) - off_lo);
    };
    auto hi = [&](unsigned x) {
        return __builtin_bit_cast(unsigned, __builtin_bit_cast(half2v, and_or_b32(x, 0x00F000F0u, mag_hi)) - off_hi);
    };
    const unsigned x0 = w.x, x1 = w.y, x2 = w.z, x3 = w.w;
    const unsigned y0 = x0 >> 8, y1 = x1 >> 8, y2 = x2 >> 8, y3 = x3 >> 8;
    CodeOps r;
    r.lo[0] = __builtin_bit_cast(half8, uint4v{lo(x0), lo(y0), lo(x1), lo(y1)});
    r.lo[1] = __builtin_bit_cast(half8, uint4v{lo(x2), lo(y2), lo(x3), lo(y3)});
    r.hi[0] = __builtin_bit_cast(half8, uint4v{hi(x0), hi(y0), hi(x1), hi(y1)});
    r.hi[1] = __builtin_bit_cast(half8, uint4v{hi(x2), hi(y2), hi(x3), hi(y3)});
    return r;
}

struct CodeOpsI8 {
    int4v op[2];
};

__device__ inline CodeOpsI8 split_codes_i8(uint4v w)
{
    CodeOpsI8 r;
    const unsigned m = 0xF0F0F0F0u, f = 0x80808080u;
    r.op[0] = int4v{(int)(((w.x << 4) & m) ^ f), (int)(((w.y << 4) & m) ^ f),
                    (int)(((w.z << 4) & m) ^ f), (int)(((w.w << 4) & m) ^ f)};
    r.op[1] = int4v{(int)((w.x & m) ^ f), (int)((w.y & m) ^ f),
                    (int)((w.z & m) ^ f), (int)((w.w & m) ^ f)};
    return r;
}

// Bytes [b0 b1 b2 b3] -> [b0 b2 b1 b3]: the int8 operand byte order of a
// lane's four consecutive k (the even nibbles of a code word come first).
__device__ inline unsigned swap_mid_bytes(unsigned x)
{
    return (x & 0xFF0000FFu) | ((x >> 8) & 0x0000FF00u) | ((x << 8) & 0x00FF0000u);
}

// The gated activation of a gate/up pair, silu(g) * u with silu(x) = x / (1 +
// e^-x), in fp32: the hardware exponential (__expf) and reciprocal, each a few
// ulps of fp32 -- far inside the one fp16 rounding of the result, and 3-6 %
// of a prefill-size gated GEMM faster than expf and an IEEE division.  For
// g -> -inf, e^-g overflows to inf and the reciprocal gives 0 (silu -> 0).
__device__ inline float silu_mul(float g, float u)
{
    return g * __builtin_amdgcn_rcpf(1.0f + __expf(-g)) * u;
}

// Gate/up pairs in the GEMM kernels (GATED): the pair is one packed [K, 2Nh]
// weight, gate columns first.  A kernel runs over the pair's 2Nh columns in a
// virtual order that interleaves the two halves by 16-column tile -- virtual
// tile 2j is gate tile j, 2j + 1 is up tile j (physical tile Nh/16 + j) -- so
// every wave that owns an even run of virtual tiles holds both products of
// the same output columns, and its epilogue stores silu(gate) * up.  Given
// the run's first virtual tile v0 (even), tile t of the run is physical tile
// gated_tile(v0, t, Nh16) = v0 / 2 + t / 2 + (t odd ? Nh16 : 0).
__host__ __device__ inline int gated_tile(int v0, int t, int Nh16)
{
    return v0 / 2 + (t >> 1) + ((t & 1) ? Nh16 : 0);
}

// Materialize a staged value here.  In a register ring the compiler may sink
// pure arithmetic on a slot (code splitting, scale conversion) below the
// refill load of that slot; the old registers then stay live across the
// refill, the allocator rotates the ring's registers, and the copies at the
// loop's back edge wait for the loads just issued.  An empty asm that reads
// and writes the value keeps the arithmetic before the refill.
template <class T>
__device__ inline void pin(T &x)
{
    asm volatile("" : "+v"(x));
}

// A scalar the compiler cannot see through.  Loads whose offset passes
// through it stay one instruction per pipeline stage even when two stages read
// the same address (the scale row of a group that spans several k-tiles),
// which the counted vmcnt waits of the pipelined kernels rely on: merged
// loads would leave fewer operations per stage than the wait allows in flight.
__device__ inline int opaque_s(int x)
{
    asm volatile("" : "+s"(x));
    return x;
}

// Cache-policy operand of a buffer load that streams data read once (the
// weight codes of a kernel whose grid reads each code once): the non-temporal
// bit, so the stream does not evict the reused activations from the caches
// (decode kernel: 2-4 % faster at every decode shape, same results).
constexpr int QG_NT = 2;

// Buffer resource over [p, p + bytes) for raw (unstructured) buffer loads:
// base address, stride 0, range in bytes (clamped to 32 bits), and the fixed
// third-word value of this GPU family for raw dword access.
__device__ inline __amdgpu_buffer_rsrc_t buffer_rsrc(const void *p, size_t bytes)
{
    const int range = bytes > 0xFFFFFFFFull ? (int)0xFFFFFFFF : (int)(unsigned)bytes;
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(p), (short)0, range, 0x00020000);
}

// s_waitcnt immediate: vmcnt n (6 bits, split), expcnt and lgkmcnt not waited
// QG_DEBUG_SYNC (compile time, 0 unless defined): every pipeline stage of the
// GEMM kernels starts by waiting for all of the wave's outstanding memory
// operations, so nothing loaded ahead stays in flight across a stage and the
// only overlap left is between waves.  Such a build computes the same bits as
// the normal one, only slower; a difference between the two points to a
// missing wait in the normal build.
#ifndef QG_DEBUG_SYNC
#define QG_DEBUG_SYNC 0
#endif
__device__ inline void debug_stage_sync()
{
    if (QG_DEBUG_SYNC) __builtin_amdgcn_s_waitcnt(0);
}

constexpr unsigned waitcnt_vm(int n)
{
    return (unsigned)((n & 0xF) | ((n >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}

__device__ inline float4v mfma_f16(half8 a, half8 b, float4v c)
{
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}

__device__ inline int4v mfma_i8(int4v a, int4v b, int4v c)
{
    return __builtin_amdgcn_mfma_i32_16x16x64_i8(a, b, c, 0, 0, 0);
}

// 16x16x32 int8 MFMA: 8 bytes of A and of B per lane, each passed as its
// (bytes 0..3, bytes 4..7) words
__device__ inline int4v mfma_i8_k32(int a0, int a1, int b0, int b1, int4v c)
{
    const long a = (long)(((unsigned long)(unsigned)a1 << 32) | (unsigned)a0);
    const long b = (long)(((unsigned long)(unsigned)b1 << 32) | (unsigned)b0);
    return __builtin_amdgcn_mfma_i32_16x16x32_i8(a, b, c, 0, 0, 0);
}

} // namespace qg
