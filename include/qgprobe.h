/* Achievable-peak probes used by the measurement harness (bench.py); not part
 * of the GEMM library.  Built as libqgprobe.so next to libqgemm.so.
 *
 * All pointers are device pointers; `stream` is a hipStream_t (NULL = the
 * default stream).  Calls only enqueue work; the caller times them (HIP
 * events on the same stream).  Return 0 on success, 1 for invalid arguments,
 * 5 if the launch failed.
 */
#ifndef QGPROBE_H
#define QGPROBE_H

#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Matrix-core loop: `workgroups` workgroups of 256 threads; every wave runs
 * `iters` rounds of independent fp16 MFMA chains (shape 16: sixteen chains of
 * 16x16x32; shape 32: four chains of 32x32x16).  `out` receives one float per
 * thread (workgroups * 256 floats, caller-allocated) so the work is not
 * discarded. */
int qgprobe_mfma_f16(int shape, float *out, int workgroups, int iters, void *stream);

/* int8 matrix-core loop: as qgprobe_mfma_f16 with sixteen chains of
 * 16x16x64 int8 MFMAs; `out` receives one int per thread. */
int qgprobe_mfma_i8(int *out, int workgroups, int iters, void *stream);

/* Operations (multiply and add counted separately) of one launch:
 * shape 16 or 32 = qgprobe_mfma_f16 with that shape, 64 = qgprobe_mfma_i8;
 * 0 for any other value. */
long long qgprobe_mfma_flops(int shape, int workgroups, int iters);

/* Streaming read of `bytes` (rounded down to whole KiB) from `buf`:
 * `workgroups` workgroups of 4 waves, each wave reading one contiguous run of
 * 1 KiB blocks in batches of `unroll` (1, 2, 4, 8 or 16) blocks, one batch in flight
 * ahead of the one it consumes.  `out` receives one word per lane
 * (workgroups * 256 words, caller-allocated). */
int qgprobe_hbm_read(const void *buf, size_t bytes, unsigned *out, int workgroups, int unroll, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* QGPROBE_H */
