/*
 * qgemm.h -- C ABI of the packed-int4 weight GEMM library for AMD Instinct
 * MI355X (gfx950).
 *
 * It computes C[M,N] = A[M,K] . W[K,N] where W is held as 4-bit codes q in
 * [0,15], eight to a uint32, with one fp16 scale (and, asymmetric, one fp16
 * zero) per group of `group_size` consecutive k and per column n:
 *
 *   symmetric offset-binary  W[k,n] = (q[k,n] - 8) * scale[k/g, n]
 *   asymmetric               W[k,n] =  q[k,n] * scale[k/g, n] + zero[k/g, n]
 *
 * Sources (web pages, cited by title and section):
 *   [Marlin-Ada]  "Marlin INT4 on Ada - how it works" (TinyLoop docs):
 *                 "The core mismatch: symmetric vs asymmetric" (both formats,
 *                 delta = zero + 8*scale, C = C_sym + A_group_sum @ delta),
 *                 "The pipeline, end to end" (pack, group-sum and correction
 *                 stages), "How the dispatcher chooses" (K, N multiples of
 *                 128; group_size == K written as -1 for per-column scales).
 *   [HyperQwen]   "HyperQwen int8 tensor-core fix of the Marlin W4A8 negative
 *                 scale bug and per-layer activation quantization": the W4A8
 *                 path (int4 weights, per-token int8 activations, integer
 *                 accumulation) and the load-time sign fold of negative group
 *                 scales (scale -> -scale, code v -> 16 - v, clamped at 15).
 *
 * Conventions for every entry point:
 *   - All tensor pointers are DEVICE pointers, row-major and contiguous, owned
 *     by the caller.  The library allocates no device memory and keeps no
 *     device state; scratch memory is a caller-provided workspace whose size
 *     qg_workspace_bytes() reports (0 for every path that needs none).
 *   - A W4A16 workspace starts with QG_W4A16_WS_COUNTER_BYTES bytes of
 *     split-K counters, then the fp32 partial sums (decode-size batches,
 *     M <= 80, where the split-K decode kernel runs) and the
 *     correction's group sums (QG_CORR_SEPARATE).  It must be zero-filled
 *     before its first use; every qgemm_w4a16 call leaves the counters at zero
 *     again, so one zero-filled workspace serves any sequence of qgemm_w4a16
 *     calls on one stream, whatever their shapes and flags.  Do not use it for
 *     anything else in between (group_sum_correction included).  Calls that
 *     may overlap in time (different streams or devices) must not share one.
 *   - fp16 tensors are passed as uint16_t (IEEE binary16 bit patterns).
 *   - `stream` is a hipStream_t passed as void* (NULL = the null stream).  All
 *     work is enqueued asynchronously; nothing is synchronised or read back.
 *   - Every argument is validated on the host BEFORE anything is launched; on
 *     error nothing is written and nothing is launched.  The return value is a
 *     QG_* status; qg_last_error() gives a per-thread description.  There is no
 *     internal fallback to another path: the caller decides what to do.
 *   - Shapes: K % 128 == 0 and N % 128 == 0 (the tile multiples the pages'
 *     dispatcher requires), M >= 1.  group_size must divide K and be 32, 64,
 *     a multiple of 128, or K; -1 is accepted as an alias of K (per-column
 *     scales), for every operation.
 *     pack_int4_weights, qgemm_w4a16 and qgemm_w4a8 also take any K, N >= 1
 *     ("tails"):
 *     group_size is then 32, 64, a multiple of 128 (the last group of g
 *     consecutive k may be partial: G = ceil(K / g)), K, or -1; see
 *     qg_padded_shape.
 *     Limits: K < 2^22 and ceil(K / g) * N * 2 < 2^31 (the kernels' 32-bit
 *     offsets; qgemm_w4a16_swiglu counts the pair's 2N), else
 *     QG_ERR_UNSUPPORTED.
 *   - A, C, scale, zero and delta must be 2-byte aligned; w_packed 16-byte
 *     aligned; A 16-byte aligned for the W4A16 GEMM, A_q 8-byte aligned for
 *     W4A8.
 *   - Calls on the same stream are ordered; concurrent calls on different
 *     streams that write the same output race (as any two kernels would).
 */
#ifndef QGEMM_H
#define QGEMM_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* ---- status codes ---- */
#define QG_OK               0
#define QG_ERR_INVALID_ARG  1  /* NULL pointer, bad alignment, M < 1, ...        */
#define QG_ERR_UNSUPPORTED  2  /* shape or group size this library has no kernel for */
#define QG_ERR_WORKSPACE    3  /* workspace missing or smaller than required      */
#define QG_ERR_DEVICE       4  /* current device is not gfx950 / no device        */
#define QG_ERR_LAUNCH       5  /* the HIP runtime rejected a launch               */

/* ---- flags ---- */
/* pack_int4_weights: fold negative group scales into the codes (symmetric
 * packs only; ignored when zero != NULL).                                   */
#define QG_PACK_FOLD_NEG_SCALES 0x1u
/* qgemm_w4a16: add the asymmetric term with the two-stage
 * group_sum_correction (after an fp16 store of the symmetric product)
 * instead of fusing it into the GEMM epilogue.                              */
#define QG_CORR_SEPARATE        0x1u

/* Size of the counter region at the start of every non-empty W4A16
 * workspace (see the conventions above).                                    */
#define QG_W4A16_WS_COUNTER_BYTES 65536u

/* ---- operations, for qg_workspace_bytes ---- */
#define QG_OP_W4A16                 1
#define QG_OP_W4A8                  2
#define QG_OP_GROUP_SUM_CORRECTION  3
#define QG_OP_PACK                  4
#define QG_OP_W4A16_SWIGLU          5

/* 1 if HIP device `device` is a gfx950 GPU this library has kernels for,
 * else 0 (also 0 when the device does not exist).  The analogue of the pages'
 * runtime architecture gate ([Marlin-Ada], "How the dispatcher chooses").   */
int qg_device_supported(int device);

/* Static text for a QG_* status. Never NULL.                                */
const char *qg_status_string(int status);

/* Description of the last error on the calling thread ("" if none). The
 * pointer stays valid until the next library call on that thread.          */
const char *qg_last_error(void);

/* Padded shape of a pack of [K,N] codes with this group size (any K, N >= 1):
 * the packed weight holds K_padded * N_padded / 8 uint32, scale_out and
 * delta_out are [groups, N_padded] fp16.  K_padded = K rounded up to a whole
 * group (to 128 when group_size is K, -1, 32 or 64), N_padded = N rounded up to 128,
 * groups = K_padded / group_size (1 per column): ceil(K / group_size), except
 * that groups of 32 or 64 may add whole groups past K (zero scale and delta in
 * the pack; the input scale and zero keep ceil(K / group_size) rows).  Equal
 * to K, N, K/g for shapes
 * without tails.  Any output pointer may be NULL.  Returns a QG_* status.  */
int qg_padded_shape(int K, int N, int group_size, int *K_padded, int *N_padded, int *groups);

/* Bytes of workspace `op` needs for this shape (0 when none). Returns
 * (size_t)-1 when the arguments are invalid.                                */
size_t qg_workspace_bytes(int op, int M, int N, int K, int group_size,
                          int num_experts, unsigned flags);

/* ---- load-time repack ([Marlin-Ada] "The pipeline, end to end";
 *      [HyperQwen] negative group-scale section) ----
 * q         [K,N] uint8, one code (0..15) per byte; larger values are an
 *           error the kernel cannot report and give unspecified codes.
 * scale     [ceil(K / group_size), N] fp16.
 * zero      [ceil(K / group_size), N] fp16, or NULL for a symmetric weight.
 * flags     QG_PACK_FOLD_NEG_SCALES: for a symmetric weight, every (g,n) with
 *           scale < 0 (strictly; -0.0 is left alone) gets scale -> -scale and
 *           codes v -> min(16 - v, 15) over that group.
 * w_packed  [K_padded*N_padded/8] uint32 out, in this library's MFMA-operand
 *           tile order (private layout; the only consumers are the GEMMs);
 *           padding codes are 8.
 * scale_out [groups,N_padded] fp16 out (groups from qg_padded_shape): the
 *           (folded) scale, 0 in padded columns and padded groups.  May
 *           alias `scale` when N % 128 == 0 and groups == ceil(K / g).
 * delta_out [groups,N_padded] fp16 out, required iff zero != NULL (0 in
 *           padded columns and groups):
 *           delta = round_to_nearest_even_fp16(zero + 8*scale), with the
 *           pre-fold scale and the sum formed exactly.
 * Runs one or two kernels on `stream`. No workspace.                        */
int pack_int4_weights(const uint8_t *q, const uint16_t *scale, const uint16_t *zero,
                      int K, int N, int group_size, unsigned flags,
                      uint32_t *w_packed, uint16_t *scale_out, uint16_t *delta_out,
                      void *stream);

/* ---- W4A16 GEMM ([Marlin-Ada] "The core mismatch") ----
 * A        [M,K] fp16 activations.
 * w_packed, scale: from pack_int4_weights.
 * delta    [G,N] fp16 from pack_int4_weights for an asymmetric weight, or NULL
 *          for a symmetric one.
 * C        [M,N] fp16 out, OVERWRITTEN with A . W (fp32 accumulation, one
 *          rounding to fp16 at the end).  The weights enter the products
 *          exactly in the decode kernel for up to 16 rows and in the skinny
 *          and mid-batch kernels (codes as exact fp16 values, scales applied
 *          in fp32), and rounded once per element to fp16 in the decode
 *          kernel for 17 to 80 rows ((v-8)*scale + delta) and in the tiled
 *          kernels ((v-8)*scale), so |W| must stay within the fp16 range;
 *          QGEMM_LOG=1 names the kernel a call runs.
 * flags    0: the delta term sum_g a_sum[m,g]*delta[g,n] is added in fp32 in
 *          the GEMM epilogue (one launch).
 *          QG_CORR_SEPARATE: C is first stored as the symmetric product and
 *          then corrected in place by group_sum_correction (needs workspace).
 * Tails (K or N not a multiple of 128, from a tail pack): A is copied into
 *          the workspace with zero columns up to K_padded, the GEMM runs on
 *          the padded shape and its product is cropped into C; the delta term
 *          is fused; QG_CORR_SEPARATE is QG_ERR_UNSUPPORTED.
 * workspace/workspace_bytes: qg_workspace_bytes(QG_OP_W4A16, ...) bytes,
 *          256-byte aligned (NULL when that is 0).  For decode-size batches
 *          (M <= 16, and up to M = 80 on all but small weights) the K range
 *          is split over several workgroups whose fp32 partial sums meet in
 *          the workspace; the last to finish adds them in a fixed order, so
 *          results do not depend on timing.  A grid that would leave a few
 *          CUs one workgroup more than the rest splits its last column groups
 *          finer (or, when nothing else is split, only those), which also
 *          takes workspace.                                                 */
int qgemm_w4a16(const uint16_t *A, const uint32_t *w_packed, const uint16_t *scale,
                const uint16_t *delta, uint16_t *C, int M, int N, int K,
                int group_size, unsigned flags, void *workspace,
                size_t workspace_bytes, void *stream);

/* ---- W4A16 GEMM without a workspace argument, for callers that cannot
 *      allocate device memory (code under HIP graph capture, tight serving
 *      loops, harnesses that forbid allocation) ----
 * Same arguments, checks, kernels and results as qgemm_w4a16 minus the
 * workspace: the scratch a call needs (split-K partial sums and counters,
 * the separate correction's group sums, a tail shape's padded A and C) is a
 * static device array of QG_NOALLOC_SCRATCH_BYTES bytes inside the library,
 * one per GPU, held until the process ends.  No device memory is allocated
 * or freed by the call.  A call whose scratch need
 * (qg_workspace_bytes(QG_OP_W4A16, ...)) exceeds QG_NOALLOC_SCRATCH_BYTES
 * returns QG_ERR_WORKSPACE before anything is launched.  The first call on a
 * device clears the scratch's counter region with a small kernel on
 * `stream`; every call leaves it at zero again.  Every call on a GPU uses
 * that GPU's one array, which keeps the last call's contents: calls that may
 * overlap in time on one GPU (different streams, threads or graphs) race and
 * must be ordered by the caller.                                            */
#define QG_NOALLOC_SCRATCH_BYTES 33554432u
int qgemm_w4a16_noalloc(const uint16_t *A, const uint32_t *w_packed, const uint16_t *scale,
                        const uint16_t *delta, uint16_t *C, int M, int N, int K,
                        int group_size, unsigned flags, void *stream);

/* ---- SwiGLU of an MLP's gate and up projections in one call ([Marlin-Ada]
 *      "Gaps and follow-ups": the fused mlp_gate + mlp_up dispatch) ----
 * The pair is ONE packed weight of shape [K, 2N]: pack_int4_weights on the
 * codes [W_gate | W_up] (gate columns 0..N-1, up columns N..2N-1) and their
 * [G, 2N] scales (and zeros) concatenated the same way.
 * A        [M,K] fp16, 16-byte aligned.
 * w_packed, scale, delta: the pair's pack (delta NULL for symmetric weights).
 * H        [M,N] fp16 out, 16-byte aligned, OVERWRITTEN with
 *            H[m,n] = silu(G[m,n]) * U[m,n],  silu(x) = x / (1 + exp(-x)),
 *          G = A . W_gate and U = A . W_up with their delta terms fused.
 *          One launch for every M: the kernel holds G and U of the same
 *          output columns in fp32 and rounds H once.
 * N % 128 == 0 (the output width), K and group_size as for qgemm_w4a16.
 * flags    must be 0.
 * workspace/workspace_bytes: qg_workspace_bytes(QG_OP_W4A16_SWIGLU, M, N, K,
 *          group_size, 1, 0) bytes, 256-byte aligned (NULL when 0: every
 *          shape but the decode batches whose grid splits K, for all column
 *          groups or for the last ones only); it starts with the same
 *          counter region as a W4A16 workspace (zero-filled once, left at
 *          zero by every call), so one workspace of the larger size serves
 *          both kinds of call on one stream.                                */
int qgemm_w4a16_swiglu(const uint16_t *A, const uint32_t *w_packed, const uint16_t *scale,
                       const uint16_t *delta, uint16_t *H, int M, int N, int K, int group_size,
                       unsigned flags, void *workspace, size_t workspace_bytes, void *stream);

/* ---- asymmetric correction as its own two stages ([Marlin-Ada] "The
 *      pipeline, end to end", a_group_sum and correction_accum) ----
 * C[m,n] += sum_g a_sum[m,g] * delta[g,n],  a_sum[m,g] = sum_{k in g} A[m,k]
 * a_sum is formed in fp32 in the workspace; C is read, updated in fp32 and
 * rounded back to fp16 (ACCUMULATES into C, unlike the GEMMs).
 * workspace: qg_workspace_bytes(QG_OP_GROUP_SUM_CORRECTION, ...) bytes.     */
int group_sum_correction(const uint16_t *A, const uint16_t *delta, uint16_t *C,
                         int M, int N, int K, int group_size, void *workspace,
                         size_t workspace_bytes, void *stream);

/* ---- grouped W4A8 GEMM ([HyperQwen] "why int8 activation quantization
 *      (W4A8) is worth doing"; zero-point weights: its verification section,
 *      point 2) ----
 * A_q          [M_total,K] int8 per-token codes; a_scale [M_total] fp32
 *              (quantize_rows_int8 makes both from fp16 activations).
 * w_packed     E stacked packs (each K*N/8 uint32).
 * w_scale      E stacked [G,N] fp16 scales (the packs' scale_out).
 * w_delta      NULL for symmetric weights; for asymmetric (zero-point) ones
 *              the E stacked [G,N] fp16 deltas (the packs' delta_out,
 *              delta = zero + 8*scale).
 * expert_offsets  DEVICE int32[E+1], non-decreasing, offsets[0] = 0,
 *              offsets[E] = M_total: expert e owns rows offsets[e] ..
 *              offsets[e+1]-1.  NULL means one expert owning all rows (E must
 *              be 1).  Rows are clipped to [0, M_total) in the kernel.
 * max_rows_per_expert  the expected largest offsets[e+1]-offsets[e]; it only
 *              sizes the launch (ceil(max_rows_per_expert / 64) row blocks per
 *              expert, each taking every further 64-row block of its expert in
 *              turn), so a bound below the true count is slower, never wrong.
 * C            [M_total,N] fp16 out, overwritten:
 *              C[m,n] = a_scale[m] * sum_g (scale_e[g,n] * acc[m,g,n]
 *                                           + delta_e[g,n] * qsum[m,g])
 *              acc[m,g,n] = sum_{k in g} A_q[m,k] * (v_e[k,n] - 8)  (int32, exact)
 *              qsum[m,g]  = sum_{k in g} A_q[m,k]                    (int32, exact)
 *              (the delta term only with w_delta), in fp32, one rounding to
 *              fp16 at the end.
 * acc_debug    NULL, or [M_total,G,N] int32 out receiving acc exactly.
 * Tails (K or N not a multiple of 128, packs from pack_int4_weights of that
 *              shape: each [K_padded*N_padded/8], scales [G,N_padded]): A_q
 *              is copied with zero columns into the workspace, the product is
 *              formed on the padded shape and cropped into C; acc_debug is
 *              then QG_ERR_UNSUPPORTED.
 * workspace/workspace_bytes: qg_workspace_bytes(QG_OP_W4A8, M_total, N, K,
 *              group_size, E, 0) bytes, 256-byte aligned: 0 (pass NULL, 0)
 *              unless the shape has tails.  The first
 *              QG_W4A16_WS_COUNTER_BYTES bytes are never touched (they are
 *              the W4A16 split-K counters' place), so one zero-filled
 *              workspace may serve W4A16 and W4A8 calls in turn on one
 *              stream.                                                      */
int qgemm_w4a8(const int8_t *A_q, const float *a_scale, const uint32_t *w_packed,
               const uint16_t *w_scale, const uint16_t *w_delta,
               const int32_t *expert_offsets, int num_experts,
               int M_total, int max_rows_per_expert, int N, int K, int group_size,
               uint16_t *C, int32_t *acc_debug, void *workspace, size_t workspace_bytes,
               unsigned flags, void *stream);

/* ---- per-token int8 activation quantization, the input stage of
 *      qgemm_w4a8 ([HyperQwen] "why int8 activation quantization (W4A8) is
 *      worth doing": activations are quantized per token to int8) ----
 * A        [M,K] fp16 activations, 16-byte aligned; K % 8 == 0 (else
 *          QG_ERR_UNSUPPORTED).
 * A_q      [M,K] int8 out, 8-byte aligned; a_scale [M] fp32 out:
 *            a_scale[m] = max_k |A[m,k]| / 127
 *            A_q[m,k]   = clamp(round_half_even(A[m,k] / a_scale[m]), -127, 127)
 *          both divisions single IEEE binary32 operations (round to nearest
 *          even); a row of zeros gets a_scale 0 and codes 0.  The outputs
 *          are exactly qgemm_w4a8's A_q and a_scale.  Non-finite inputs give
 *          unspecified codes.
 * One kernel on `stream`. No workspace.                                     */
int quantize_rows_int8(const uint16_t *A, int M, int K, int8_t *A_q, float *a_scale,
                       void *stream);

#ifdef __cplusplus
}
#endif

#endif /* QGEMM_H */
