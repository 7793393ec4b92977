// Internal launchers between the validated C ABI (qg_api.cpp) and the kernels.
// Every launcher assumes its arguments were validated by the caller.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace qg {

// Padded shape of a pack: Kp (K up to a whole group, or to 128 for one group
// per column, g == K), Np (N up to 128), gp (the group size in the padded
// layout: g, or Kp when g == K).  Kp == K and Np == N for aligned shapes.
void padded_shape(int K, int N, int g, int *Kp, int *Np, int *gp);

// W4A16 on a shape with tails (is_tail_shape): A padded and C cropped through
// `ws` (tail_workspace_bytes), the GEMM on the padded shape.
bool is_tail_shape(int N, int K, int g);

// The kernel(s) a W4A16 (or, gated, SwiGLU) call of this padded shape runs, in
// words (for the first-dispatch log line).
void describe_w4a16(int M, int N, int K, int g, bool delta, bool gated, char *buf, size_t n);
bool use_mid2(int M, int N, int K);
size_t tail_workspace_bytes(int M, int N, int K, int g);
hipError_t launch_w4a16_tail(const uint16_t *A, const uint32_t *W, const uint16_t *S,
                             const uint16_t *D, uint16_t *C, int M, int N, int K, int g,
                             bool fuse_delta, void *ws, hipStream_t st);

// C [M, N] from the first N columns of Cp [M, Np].
hipError_t launch_crop_cols(const uint16_t *Cp, uint16_t *C, int M, int N, int Np, hipStream_t st);

// Grouped W4A8 on a shape with tails (A_q padded and C cropped through `ws`
// of w4a8_tail_workspace_bytes bytes, the kernel on the padded shape).
size_t w4a8_tail_workspace_bytes(int M_total, int N, int K, int g);
hipError_t launch_w4a8_tail(const int8_t *Aq, const float *a_scale, const uint32_t *W,
                            const uint16_t *S, const uint16_t *D, const int32_t *offsets, int E,
                            int M_total, int max_rows, int N, int K, int g, uint16_t *C, void *ws,
                            hipStream_t st);

hipError_t launch_pack(const uint8_t *q, const uint16_t *s, const uint16_t *z, int K, int N,
                       int g, bool fold, uint32_t *w, uint16_t *s_out, uint16_t *d_out,
                       hipStream_t st);

// Configuration of one skinny (small-M) W4A16 launch:
//   MT  16-row m-tiles per wave        NT  16-column n-tiles per wave
//   P   k-tiles kept in flight per wave (register ring)
//   nw  waves per workgroup, splitting the workgroup's k-range
//   S   k-splits across workgroups (only 1 is built)
struct SkinnyCfg {
    int MT, NT, P, nw, S;
};
SkinnyCfg skinny_config(int M, int N, int K);
// gated: W is a gate/up pair [K, N] (gate columns first) and C the [M, N/2]
// output silu(A W_gate) * (A W_up), both products kept in fp32 (N / 2 a
// multiple of 128).
hipError_t launch_w4a16_skinny_cfg(const SkinnyCfg &c, const uint16_t *A, const uint32_t *W,
                                   const uint16_t *S, const uint16_t *D, uint16_t *C, int M,
                                   int N, int K, int g, bool fuse_delta, void *ws,
                                   hipStream_t st, bool gated = false);
hipError_t launch_w4a16_mid(const uint16_t *A, const uint32_t *W, const uint16_t *S,
                            const uint16_t *D, uint16_t *C, int M, int N, int K, int g,
                            bool fuse_delta, hipStream_t st, bool gated = false);
int tiled_config(int M, int N);
int tiled_row_split(int M, int N);
int tiled_col_split(int M, int N, int g, bool gated);
hipError_t launch_w4a16_tiled_cfg(int cfg, const uint16_t *A, const uint32_t *W,
                                  const uint16_t *S, const uint16_t *D, uint16_t *C, int M, int N,
                                  int K, int g, bool fuse_delta, hipStream_t st, bool gated = false);
hipError_t launch_w4a16_tiled(const uint16_t *A, const uint32_t *W, const uint16_t *S,
                              const uint16_t *D, uint16_t *C, int M, int N, int K, int g,
                              bool fuse_delta, hipStream_t st, bool gated = false);

// Every non-empty W4A16 workspace starts with this many bytes of split-K
// counters.  Only the decode kernel writes them and it leaves them at zero, so
// a workspace shared by calls of different shapes and flags keeps them zero
// (the partial sums and the correction's group sums come after).
constexpr size_t W4A16_WS_COUNTER_BYTES = 65536;

// Decode kernel (M <= 80, ceil(M/16) m-tiles): split count the heuristic
// picks, whether a shape takes it, its workspace, and a launch with an
// explicit split count (nsplit > 1 needs `ws` of decode_workspace_bytes).
// g: the weight group size (groups of 64 and 32 can raise the split count,
// whose scale table grows; the default stands for any g >= 128)
int decode_splits(int N, int K, int g = 128);
// The decode grid for split count ns: column groups 0 .. cg_main-1 take ns
// splits, the others ns2; wgs workgroups, slots partial-sum slots (0: no
// split-K at all).
struct DecodeGrid {
    int cg_main, ns2, wgs, slots;
};
DecodeGrid decode_grid(int M, int N, int K, int ns);
bool use_decode_kernel(int M, int N, int K, int g = 128);
size_t decode_workspace_bytes(int M, int N, int K, int g = 128);
// ldc, ncols: C's row stride and the columns stored (default N, or N/2 for
// the gated pair); a padded weight's call stores its logical columns only
hipError_t launch_w4a16_decode(const uint16_t *A, const uint32_t *W, const uint16_t *S,
                               const uint16_t *D, uint16_t *C, int M, int N, int K, int g,
                               bool fuse_delta, int nsplit, void *ws, hipStream_t st,
                               bool gated = false, int ldc = -1, int ncols = -1);

// Rows from which the tiled/mid kernels take over from the skinny one (the mid
// kernel measured faster from about M = 80 on).
constexpr int TILED_MIN_M = 81;
constexpr int DECODE_MAX_M = TILED_MIN_M - 1;   // the decode kernel's m-tiles cover M <= 80

// Bytes of workspace the W4A16 GEMM kernels need for this shape (0 = none).
size_t w4a16_workspace_bytes(int M, int N, int K, int g);

// C = A . W; when D != nullptr and fuse_delta, the delta term is added in the
// epilogue; when D == nullptr or !fuse_delta, C is the symmetric product.
// `ws` must hold w4a16_workspace_bytes(M, N, K, g) bytes (may be null when 0).
hipError_t launch_w4a16(const uint16_t *A, const uint32_t *W, const uint16_t *S,
                        const uint16_t *D, uint16_t *C, int M, int N, int K, int g,
                        bool fuse_delta, void *ws, hipStream_t st);

// H = silu(A . W[:, :N]) * (A . W[:, N:]) for a gate/up pair packed as one
// [K, 2N] weight; `ws` of swiglu_workspace_bytes(M, N, K, g) bytes (counters
// first, zero-filled once, as for the W4A16 workspace).
bool swiglu_uses_decode(int M, int N, int K, int g);
size_t swiglu_workspace_bytes(int M, int N, int K, int g);
hipError_t launch_w4a16_swiglu(const uint16_t *A, const uint32_t *W, const uint16_t *S,
                               const uint16_t *D, uint16_t *H, int M, int N, int K, int g,
                               void *ws, hipStream_t st);

// a_sum[M, K/g] (fp32) into `a_sum`, then C += a_sum @ delta.
hipError_t launch_group_sum_correction(const uint16_t *A, const uint16_t *D, uint16_t *C,
                                       int M, int N, int K, int g, float *a_sum,
                                       hipStream_t st);

// D: stacked [E,G,N] fp16 deltas of asymmetric weights, or nullptr.
hipError_t launch_w4a8(const int8_t *Aq, const float *a_scale, const uint32_t *W,
                       const uint16_t *S, const uint16_t *D, const int32_t *offsets, int E,
                       int M_total, int max_rows, int N, int K, int g, uint16_t *C,
                       int32_t *acc_debug, hipStream_t st);

// Device address of the static scratch of qgemm_w4a16_noalloc on the current
// device (looked up once per device; the first call also clears its counter
// region on `st`).
hipError_t noalloc_scratch(hipStream_t st, void **out);

// Per-row int8 codes and fp32 scales of fp16 activations (K % 8 == 0, A
// 16-byte and Aq 8-byte aligned).
hipError_t launch_quantize_rows_int8(const uint16_t *A, int M, int K, int8_t *Aq,
                                     float *a_scale, hipStream_t st);

} // namespace qg
