// C ABI of the packed-int4 GEMM library: host-side validation, then launches.
// Nothing is launched and nothing is written unless every check passes.
#include "qgemm.h"

#include <hip/hip_runtime.h>

#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <mutex>
#include <set>
#include <string>

#include "qg_launch.h"

namespace {

thread_local char g_err[512] = "";

int fail(int status, const char *fmt, ...)
{
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_err, sizeof(g_err), fmt, ap);
    va_end(ap);
    return status;
}

int ok()
{
    g_err[0] = '\0';
    return QG_OK;
}

bool aligned(const void *p, size_t a) { return ((uintptr_t)p % a) == 0; }

// gfx950 check of the current device; cached per device id.
int check_device()
{
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0)
        return fail(QG_ERR_DEVICE, "no HIP device is current");
    if (!qg_device_supported(dev))
        return fail(QG_ERR_DEVICE, "device %d is not a gfx950 GPU", dev);
    return QG_OK;
}

// QG_DEBUG_SYNC: the library built with it set (libqgemm_debugsync.so, for
// race checks) also waits for each call's kernels and reports a failed kernel
// as that call's error; it must not be used under stream capture.
#ifndef QG_DEBUG_SYNC
#define QG_DEBUG_SYNC 0
#endif

int launch_status(hipError_t e, const char *what, hipStream_t st)
{
    if (e != hipSuccess)
        return fail(QG_ERR_LAUNCH, "%s: launch failed: %s", what, hipGetErrorString(e));
    if (QG_DEBUG_SYNC) {
        e = hipStreamSynchronize(st);
        if (e != hipSuccess)
            return fail(QG_ERR_LAUNCH, "%s: kernel failed: %s", what, hipGetErrorString(e));
    }
    return ok();
}

// With QGEMM_LOG set (and not "0"): one stderr line for the first successful
// launch of each distinct call description, as the pages' integration logs its
// first dispatch ("Marlin INT4 on Ada - how it works", "End-to-end result on
// RTX 4090").
bool log_enabled()
{
    static const bool on = [] {
        const char *e = getenv("QGEMM_LOG");
        return e && *e && strcmp(e, "0") != 0;
    }();
    return on;
}

void log_first(const char *fmt, ...)
{
    if (!log_enabled()) return;
    char line[320];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(line, sizeof(line), fmt, ap);
    va_end(ap);
    static std::mutex mu;
    static std::set<std::string> seen;
    std::lock_guard<std::mutex> lk(mu);
    if (seen.insert(line).second) fprintf(stderr, "[qgemm] first dispatch ok: %s\n", line);
}

// The kernels address a tile's activation rows and a scale row with 32-bit
// byte offsets: K < 2^22 and ceil(K/g) * N * 2 < 2^31 keep every one in
// range (far beyond any layer; larger shapes are refused, not miscomputed).
int check_offsets(const char *what, int N, int K, int g)
{
    const long long groups = (K + (long long)g - 1) / g;
    if (K >= (1 << 22) || groups * N * 2 >= (1ll << 31))
        return fail(QG_ERR_UNSUPPORTED, "%s: K=%d, N=%d too large for 32-bit offsets", what, K, N);
    return QG_OK;
}

// Shape rules shared by every GEMM-like entry point.  Normalises the per-column
// sentinel -1 to K.
int check_shape(const char *what, int M, int N, int K, int *g)
{
    if (M < 1 || N < 1 || K < 1)
        return fail(QG_ERR_INVALID_ARG, "%s: M, N, K must be >= 1 (got %d, %d, %d)", what, M, N, K);
    if (K % 128 != 0 || N % 128 != 0)
        return fail(QG_ERR_UNSUPPORTED, "%s: K and N must be multiples of 128 (got K=%d N=%d)",
                    what, K, N);
    if (*g == -1) *g = K;
    if (*g < 1 || K % *g != 0)
        return fail(QG_ERR_INVALID_ARG, "%s: group_size %d does not divide K=%d", what, *g, K);
    if (*g != K && *g % 128 != 0 && *g != 64 && *g != 32)
        return fail(QG_ERR_UNSUPPORTED,
                    "%s: group_size %d unsupported (must be 32, 64, a multiple of 128, K, or -1)",
                    what, *g);
    if ((long long)M * K > (1ll << 40) || (long long)K * N > (1ll << 40))
        return fail(QG_ERR_UNSUPPORTED, "%s: shape too large", what);
    return check_offsets(what, N, K, *g);
}

// Shape rules of the entry points that take tails (pack_int4_weights,
// qgemm_w4a16): K and N any positive size; group_size 32, 64, a multiple of
// 128 (the last group may be partial), K, or -1 (normalised to K).
int check_shape_tail(const char *what, int M, int N, int K, int *g)
{
    if (M < 1 || N < 1 || K < 1)
        return fail(QG_ERR_INVALID_ARG, "%s: M, N, K must be >= 1 (got %d, %d, %d)", what, M, N, K);
    if (*g == -1) *g = K;
    if (*g < 1)
        return fail(QG_ERR_INVALID_ARG, "%s: group_size %d", what, *g);
    if (*g != K && *g % 128 != 0 && *g != 64 && *g != 32) {
        if (K % *g != 0)
            return fail(QG_ERR_INVALID_ARG, "%s: group_size %d does not divide K=%d", what, *g, K);
        return fail(QG_ERR_UNSUPPORTED,
                    "%s: group_size %d unsupported (must be 32, 64, a multiple of 128, K, or -1)",
                    what, *g);
    }
    if (K > (1 << 28) || N > (1 << 28) || (long long)M * K > (1ll << 40) ||
        (long long)K * N > (1ll << 40))
        return fail(QG_ERR_UNSUPPORTED, "%s: shape too large", what);
    return check_offsets(what, N, K, *g);
}

size_t corr_ws_bytes(int M, int K, int g) { return (size_t)M * (size_t)(K / g) * sizeof(float); }

size_t align256(size_t n) { return (n + 255) / 256 * 256; }

// W4A16 workspace: [counters][decode partial sums][correction a_sum when
// separate].  The counter region is always first, whatever the call, so a
// workspace shared by different shapes never has group sums or partials
// written over a counter.
size_t w4a16_gemm_ws_bytes(int M, int N, int K, int g, bool separate)
{
    const size_t gemm = qg::w4a16_workspace_bytes(M, N, K, g);
    if (gemm) return gemm;
    return separate ? qg::W4A16_WS_COUNTER_BYTES : 0;
}

size_t w4a16_ws_bytes(int M, int N, int K, int g, bool separate)
{
    const size_t gemm = w4a16_gemm_ws_bytes(M, N, K, g, separate);
    if (!separate) return gemm;
    return align256(gemm) + corr_ws_bytes(M, K, g);
}

// Host checks of a W4A16 call shared by qgemm_w4a16 and qgemm_w4a16_noalloc:
// shape, pointers, alignment and flags; fills the group size, the path and
// the scratch bytes the call needs.
struct W4A16Call {
    int g;
    bool separate, tail;
    size_t need;
};

int w4a16_check(const char *what, const uint16_t *A, const uint32_t *w_packed,
                const uint16_t *scale, const uint16_t *delta, const uint16_t *C, int M, int N,
                int K, int group_size, unsigned flags, W4A16Call *call)
{
    int g = group_size;
    int rc = check_shape_tail(what, M, N, K, &g);
    if (rc) return rc;
    if (!A || !w_packed || !scale || !C)
        return fail(QG_ERR_INVALID_ARG, "%s: NULL A/w_packed/scale/C", what);
    if (!aligned(A, 16) || !aligned(w_packed, 16) || !aligned(scale, 2) || !aligned(C, 2) ||
        (delta && !aligned(delta, 2)))
        return fail(QG_ERR_INVALID_ARG, "%s: misaligned pointer", what);
    if (flags & ~QG_CORR_SEPARATE)
        return fail(QG_ERR_INVALID_ARG, "%s: unknown flags 0x%x", what, flags);
    call->g = g;
    call->separate = (flags & QG_CORR_SEPARATE) && delta;
    call->tail = qg::is_tail_shape(N, K, g);
    if (call->tail && call->separate)
        return fail(QG_ERR_UNSUPPORTED, "%s: QG_CORR_SEPARATE needs K, N multiples of 128", what);
    call->need = call->tail ? qg::tail_workspace_bytes(M, N, K, g)
                            : w4a16_ws_bytes(M, N, K, g, call->separate);
    return QG_OK;
}

// The launches of a checked W4A16 call; `workspace` holds call.need bytes.
int w4a16_launch(const char *what, const W4A16Call &call, const uint16_t *A,
                 const uint32_t *w_packed, const uint16_t *scale, const uint16_t *delta,
                 uint16_t *C, int M, int N, int K, void *workspace, hipStream_t st)
{
    const int g = call.g;
    int rc;
    if (call.tail) {
        rc = launch_status(qg::launch_w4a16_tail(A, w_packed, scale, delta, C, M, N, K, g, true,
                                                 workspace, st),
                           what, st);
    } else {
        const size_t gemm_ws = w4a16_gemm_ws_bytes(M, N, K, g, call.separate);
        hipError_t e = qg::launch_w4a16(A, w_packed, scale, delta, C, M, N, K, g, !call.separate,
                                        qg::w4a16_workspace_bytes(M, N, K, g) ? workspace : nullptr, st);
        if (e == hipSuccess && call.separate)
            e = qg::launch_group_sum_correction(A, delta, C, M, N, K, g,
                                                (float *)((char *)workspace + align256(gemm_ws)), st);
        rc = launch_status(e, what, st);
    }
    if (rc == QG_OK && log_enabled()) {
        int Kp = K, Np = N, gp = g;
        if (call.tail) qg::padded_shape(K, N, g, &Kp, &Np, &gp);
        char kern[160];
        qg::describe_w4a16(M, Np, Kp, gp, delta && !call.separate, false, kern, sizeof(kern));
        log_first("%s M=%d N=%d K=%d gs=%d %s: %s%s%s", what, M, N, K, g,
                  delta ? (call.separate ? "asymmetric (separate correction)" : "asymmetric")
                        : "symmetric",
                  call.tail ? "padded shape, " : "", kern,
                  call.separate ? " + group sums + correction" : "");
    }
    return rc;
}

} // namespace

extern "C" {

int qg_padded_shape(int K, int N, int group_size, int *K_padded, int *N_padded, int *groups)
{
    int g = group_size;
    int rc = check_shape_tail("qg_padded_shape", 1, N, K, &g);
    if (rc) return rc;
    int Kp, Np, gp;
    qg::padded_shape(K, N, g, &Kp, &Np, &gp);
    if (K_padded) *K_padded = Kp;
    if (N_padded) *N_padded = Np;
    if (groups) *groups = Kp / gp;
    return ok();
}

int qg_device_supported(int device)
{
    int n = 0;
    if (hipGetDeviceCount(&n) != hipSuccess || device < 0 || device >= n) return 0;
    static std::mutex mu;
    static int cache[64];
    static bool cached[64];
    if (device < 64) {
        std::lock_guard<std::mutex> lk(mu);
        if (cached[device]) return cache[device];
    }
    hipDeviceProp_t p;
    if (hipGetDeviceProperties(&p, device) != hipSuccess) return 0;
    int yes = strncmp(p.gcnArchName, "gfx950", 6) == 0 ? 1 : 0;
    if (device < 64) {
        std::lock_guard<std::mutex> lk(mu);
        cache[device] = yes;
        cached[device] = true;
    }
    return yes;
}

const char *qg_status_string(int status)
{
    switch (status) {
    case QG_OK: return "ok";
    case QG_ERR_INVALID_ARG: return "invalid argument";
    case QG_ERR_UNSUPPORTED: return "unsupported shape or group size";
    case QG_ERR_WORKSPACE: return "workspace missing or too small";
    case QG_ERR_DEVICE: return "no supported (gfx950) device";
    case QG_ERR_LAUNCH: return "kernel launch failed";
    default: return "unknown status";
    }
}

const char *qg_last_error(void) { return g_err; }

size_t qg_workspace_bytes(int op, int M, int N, int K, int group_size, int num_experts,
                          unsigned flags)
{
    (void)num_experts;
    int g = group_size;
    switch (op) {
    case QG_OP_W4A16:
        if (check_shape_tail("qg_workspace_bytes", M, N, K, &g) != QG_OK) return (size_t)-1;
        if (qg::is_tail_shape(N, K, g)) {
            if (flags & QG_CORR_SEPARATE) {
                fail(QG_ERR_UNSUPPORTED, "qg_workspace_bytes: QG_CORR_SEPARATE needs K, N multiples of 128");
                return (size_t)-1;
            }
            return qg::tail_workspace_bytes(M, N, K, g);
        }
        return w4a16_ws_bytes(M, N, K, g, (flags & QG_CORR_SEPARATE) != 0);
    case QG_OP_W4A16_SWIGLU:
        if (check_shape("qg_workspace_bytes", M, N, K, &g) != QG_OK) return (size_t)-1;
        if (N > 0x3FFFFFFF) return (size_t)-1;
        return qg::swiglu_workspace_bytes(M, N, K, g);
    case QG_OP_GROUP_SUM_CORRECTION:
        if (check_shape("qg_workspace_bytes", M, N, K, &g) != QG_OK) return (size_t)-1;
        return corr_ws_bytes(M, K, g);
    case QG_OP_W4A8:
        if (check_shape_tail("qg_workspace_bytes", M < 1 ? 1 : M, N, K, &g) != QG_OK) return (size_t)-1;
        return qg::is_tail_shape(N, K, g) ? qg::w4a8_tail_workspace_bytes(M < 1 ? 1 : M, N, K, g) : 0;
    case QG_OP_PACK:
        if (check_shape("qg_workspace_bytes", M < 1 ? 1 : M, N, K, &g) != QG_OK) return (size_t)-1;
        return 0;
    default:
        fail(QG_ERR_INVALID_ARG, "qg_workspace_bytes: unknown op %d", op);
        return (size_t)-1;
    }
}

int pack_int4_weights(const uint8_t *q, const uint16_t *scale, const uint16_t *zero, int K,
                      int N, int group_size, unsigned flags, uint32_t *w_packed,
                      uint16_t *scale_out, uint16_t *delta_out, void *stream)
{
    int g = group_size;
    int rc = check_shape_tail("pack_int4_weights", 1, N, K, &g);
    if (rc) return rc;
    if (!q || !scale || !w_packed || !scale_out)
        return fail(QG_ERR_INVALID_ARG, "pack_int4_weights: NULL q/scale/w_packed/scale_out");
    if (zero && !delta_out)
        return fail(QG_ERR_INVALID_ARG, "pack_int4_weights: delta_out is required with zero");
    if (!aligned(w_packed, 16) || !aligned(scale, 2) || !aligned(scale_out, 2) ||
        (zero && !aligned(zero, 2)) || (delta_out && !aligned(delta_out, 2)))
        return fail(QG_ERR_INVALID_ARG, "pack_int4_weights: misaligned pointer");
    if (flags & ~QG_PACK_FOLD_NEG_SCALES)
        return fail(QG_ERR_INVALID_ARG, "pack_int4_weights: unknown flags 0x%x", flags);
    if ((const void *)scale_out == (const void *)scale) {
        int Kp, Np, gp;
        qg::padded_shape(K, N, g, &Kp, &Np, &gp);
        if (Np != N || Kp / gp != (K + g - 1) / g)
            return fail(QG_ERR_INVALID_ARG,
                        "pack_int4_weights: scale_out may alias scale only when the padded "
                        "shape adds no columns and no groups");
    }
    if ((rc = check_device())) return rc;
    hipError_t e = qg::launch_pack(q, scale, zero, K, N, g, (flags & QG_PACK_FOLD_NEG_SCALES) != 0,
                                   w_packed, scale_out, zero ? delta_out : nullptr,
                                   (hipStream_t)stream);
    rc = launch_status(e, "pack_int4_weights", (hipStream_t)stream);
    if (rc == QG_OK)
        log_first("pack_int4_weights K=%d N=%d gs=%d %s%s", K, N, g, zero ? "asymmetric" : "symmetric",
                  (flags & QG_PACK_FOLD_NEG_SCALES) ? ", negative scales folded" : "");
    return rc;
}

int qgemm_w4a16(const uint16_t *A, const uint32_t *w_packed, const uint16_t *scale,
                const uint16_t *delta, uint16_t *C, int M, int N, int K, int group_size,
                unsigned flags, void *workspace, size_t workspace_bytes, void *stream)
{
    W4A16Call call;
    int rc = w4a16_check("qgemm_w4a16", A, w_packed, scale, delta, C, M, N, K, group_size, flags,
                         &call);
    if (rc) return rc;
    if (call.need > 0) {
        if (!workspace || workspace_bytes < call.need)
            return fail(QG_ERR_WORKSPACE, "qgemm_w4a16: workspace of %zu bytes needed, got %zu",
                        call.need, workspace ? workspace_bytes : (size_t)0);
        if (!aligned(workspace, 256))
            return fail(QG_ERR_INVALID_ARG, "qgemm_w4a16: workspace must be 256-byte aligned");
    }
    if ((rc = check_device())) return rc;
    return w4a16_launch("qgemm_w4a16", call, A, w_packed, scale, delta, C, M, N, K, workspace,
                        (hipStream_t)stream);
}

int qgemm_w4a16_noalloc(const uint16_t *A, const uint32_t *w_packed, const uint16_t *scale,
                        const uint16_t *delta, uint16_t *C, int M, int N, int K, int group_size,
                        unsigned flags, void *stream)
{
    W4A16Call call;
    int rc = w4a16_check("qgemm_w4a16_noalloc", A, w_packed, scale, delta, C, M, N, K, group_size,
                         flags, &call);
    if (rc) return rc;
    if (call.need > QG_NOALLOC_SCRATCH_BYTES)
        return fail(QG_ERR_WORKSPACE,
                    "qgemm_w4a16_noalloc: this call needs %zu bytes of scratch, more than the "
                    "library's static scratch of %zu bytes (use qgemm_w4a16 with a workspace)",
                    call.need, (size_t)QG_NOALLOC_SCRATCH_BYTES);
    if ((rc = check_device())) return rc;
    void *ws = nullptr;
    if (call.need > 0) {
        hipError_t e = qg::noalloc_scratch((hipStream_t)stream, &ws);
        if (e != hipSuccess)
            return fail(QG_ERR_LAUNCH, "qgemm_w4a16_noalloc: static scratch unavailable: %s",
                        hipGetErrorString(e));
    }
    return w4a16_launch("qgemm_w4a16_noalloc", call, A, w_packed, scale, delta, C, M, N, K, ws,
                        (hipStream_t)stream);
}

int qgemm_w4a16_swiglu(const uint16_t *A, const uint32_t *w_packed, const uint16_t *scale,
                       const uint16_t *delta, uint16_t *H, int M, int N, int K, int group_size,
                       unsigned flags, void *workspace, size_t workspace_bytes, void *stream)
{
    int g = group_size;
    int rc = check_shape("qgemm_w4a16_swiglu", M, N, K, &g);
    if (rc) return rc;
    if (N > 0x3FFFFFFF || (size_t)K * 2 * (size_t)N / 8 > 0x7FFFFFFFull * 16)
        return fail(QG_ERR_UNSUPPORTED, "qgemm_w4a16_swiglu: shape too large");
    if ((rc = check_offsets("qgemm_w4a16_swiglu", 2 * N, K, g))) return rc;   // the pair's width
    if (!A || !w_packed || !scale || !H)
        return fail(QG_ERR_INVALID_ARG, "qgemm_w4a16_swiglu: NULL A/w_packed/scale/H");
    if (!aligned(A, 16) || !aligned(w_packed, 16) || !aligned(scale, 2) || !aligned(H, 16) ||
        (delta && !aligned(delta, 2)))
        return fail(QG_ERR_INVALID_ARG, "qgemm_w4a16_swiglu: misaligned pointer");
    if (flags != 0)
        return fail(QG_ERR_INVALID_ARG, "qgemm_w4a16_swiglu: unknown flags 0x%x", flags);
    const size_t need = qg::swiglu_workspace_bytes(M, N, K, g);
    if (need > 0) {
        if (!workspace || workspace_bytes < need)
            return fail(QG_ERR_WORKSPACE, "qgemm_w4a16_swiglu: workspace of %zu bytes needed, got %zu",
                        need, workspace ? workspace_bytes : (size_t)0);
        if (!aligned(workspace, 256))
            return fail(QG_ERR_INVALID_ARG, "qgemm_w4a16_swiglu: workspace must be 256-byte aligned");
    }
    if ((rc = check_device())) return rc;
    hipError_t e = qg::launch_w4a16_swiglu(A, w_packed, scale, delta, H, M, N, K, g,
                                           need ? workspace : nullptr, (hipStream_t)stream);
    rc = launch_status(e, "qgemm_w4a16_swiglu", (hipStream_t)stream);
    if (rc == QG_OK && log_enabled()) {
        char kern[160];
        qg::describe_w4a16(M, N, K, g, delta != nullptr, true, kern, sizeof(kern));
        log_first("qgemm_w4a16_swiglu M=%d N=%d (pair %d) K=%d gs=%d %s: %s", M, N, 2 * N, K, g,
                  delta ? "asymmetric" : "symmetric", kern);
    }
    return rc;
}

int group_sum_correction(const uint16_t *A, const uint16_t *delta, uint16_t *C, int M, int N,
                         int K, int group_size, void *workspace, size_t workspace_bytes,
                         void *stream)
{
    int g = group_size;
    int rc = check_shape("group_sum_correction", M, N, K, &g);
    if (rc) return rc;
    if (!A || !delta || !C)
        return fail(QG_ERR_INVALID_ARG, "group_sum_correction: NULL A/delta/C");
    if (!aligned(A, 2) || !aligned(delta, 2) || !aligned(C, 2))
        return fail(QG_ERR_INVALID_ARG, "group_sum_correction: misaligned pointer");
    size_t need = corr_ws_bytes(M, K, g);
    if (!workspace || workspace_bytes < need)
        return fail(QG_ERR_WORKSPACE, "group_sum_correction: workspace of %zu bytes needed, got %zu",
                    need, workspace ? workspace_bytes : (size_t)0);
    if (!aligned(workspace, 4))
        return fail(QG_ERR_INVALID_ARG, "group_sum_correction: misaligned workspace");
    if ((rc = check_device())) return rc;
    hipError_t e = qg::launch_group_sum_correction(A, delta, C, M, N, K, g, (float *)workspace,
                                                   (hipStream_t)stream);
    rc = launch_status(e, "group_sum_correction", (hipStream_t)stream);
    if (rc == QG_OK) log_first("group_sum_correction M=%d N=%d K=%d gs=%d", M, N, K, g);
    return rc;
}

int qgemm_w4a8(const int8_t *A_q, const float *a_scale, const uint32_t *w_packed,
               const uint16_t *w_scale, const uint16_t *w_delta,
               const int32_t *expert_offsets, int num_experts,
               int M_total, int max_rows_per_expert, int N, int K, int group_size, uint16_t *C,
               int32_t *acc_debug, void *workspace, size_t workspace_bytes, unsigned flags,
               void *stream)
{
    int g = group_size;
    int rc = check_shape_tail("qgemm_w4a8", M_total, N, K, &g);
    if (rc) return rc;
    const bool tail = qg::is_tail_shape(N, K, g);
    if (!A_q || !a_scale || !w_packed || !w_scale || !C)
        return fail(QG_ERR_INVALID_ARG, "qgemm_w4a8: NULL A_q/a_scale/w_packed/w_scale/C");
    if (num_experts < 1 || num_experts > 65535)
        return fail(QG_ERR_INVALID_ARG, "qgemm_w4a8: num_experts %d out of range", num_experts);
    if (!expert_offsets && num_experts != 1)
        return fail(QG_ERR_INVALID_ARG, "qgemm_w4a8: expert_offsets is required when E > 1");
    if (max_rows_per_expert < 1)
        return fail(QG_ERR_INVALID_ARG, "qgemm_w4a8: max_rows_per_expert must be >= 1");
    if (!expert_offsets && max_rows_per_expert < M_total)
        return fail(QG_ERR_INVALID_ARG, "qgemm_w4a8: max_rows_per_expert < M_total with one expert");
    if (K > 131072)
        return fail(QG_ERR_UNSUPPORTED, "qgemm_w4a8: K > 131072 would overflow int32 accumulators");
    if (!aligned(A_q, 8) || !aligned(a_scale, 4) || !aligned(w_packed, 16) ||
        !aligned(w_scale, 2) || (w_delta && !aligned(w_delta, 2)) || !aligned(C, 2) ||
        (acc_debug && !aligned(acc_debug, 4)) ||
        (expert_offsets && !aligned(expert_offsets, 4)))
        return fail(QG_ERR_INVALID_ARG, "qgemm_w4a8: misaligned pointer");
    if (flags != 0) return fail(QG_ERR_INVALID_ARG, "qgemm_w4a8: unknown flags 0x%x", flags);
    if (tail) {
        if (acc_debug)
            return fail(QG_ERR_UNSUPPORTED, "qgemm_w4a8: acc_debug needs K, N multiples of 128");
        const size_t need = qg::w4a8_tail_workspace_bytes(M_total, N, K, g);
        if (!workspace || workspace_bytes < need)
            return fail(QG_ERR_WORKSPACE, "qgemm_w4a8: workspace of %zu bytes needed, got %zu", need,
                        workspace ? workspace_bytes : (size_t)0);
        if (!aligned(workspace, 256))
            return fail(QG_ERR_INVALID_ARG, "qgemm_w4a8: workspace must be 256-byte aligned");
    }
    if ((rc = check_device())) return rc;
    int max_rows = max_rows_per_expert > M_total ? M_total : max_rows_per_expert;
    const hipError_t e =
        tail ? qg::launch_w4a8_tail(A_q, a_scale, w_packed, w_scale, w_delta, expert_offsets,
                                    num_experts, M_total, max_rows, N, K, g, C, workspace,
                                    (hipStream_t)stream)
             : qg::launch_w4a8(A_q, a_scale, w_packed, w_scale, w_delta, expert_offsets, num_experts,
                               M_total, max_rows, N, K, g, C, acc_debug, (hipStream_t)stream);
    rc = launch_status(e, "qgemm_w4a8", (hipStream_t)stream);
    if (rc == QG_OK)
        log_first("qgemm_w4a8 experts=%d M_total=%d max_rows=%d N=%d K=%d gs=%d %s%s%s", num_experts,
                  M_total, max_rows_per_expert, N, K, g, w_delta ? "zero-points" : "symmetric",
                  tail ? ", padded shape" : "", acc_debug ? ", acc_debug" : "");
    return rc;
}

int quantize_rows_int8(const uint16_t *A, int M, int K, int8_t *A_q, float *a_scale,
                       void *stream)
{
    if (!A || !A_q || !a_scale)
        return fail(QG_ERR_INVALID_ARG, "quantize_rows_int8: NULL A/A_q/a_scale");
    if (M < 1 || K < 1)
        return fail(QG_ERR_INVALID_ARG, "quantize_rows_int8: M and K must be >= 1 (got %d, %d)", M, K);
    if (K % 8)
        return fail(QG_ERR_UNSUPPORTED, "quantize_rows_int8: K must be a multiple of 8 (got %d)", K);
    if (!aligned(A, 16) || !aligned(A_q, 8) || !aligned(a_scale, 4))
        return fail(QG_ERR_INVALID_ARG, "quantize_rows_int8: misaligned pointer");
    int rc = check_device();
    if (rc) return rc;
    hipError_t e = qg::launch_quantize_rows_int8(A, M, K, A_q, a_scale, (hipStream_t)stream);
    rc = launch_status(e, "quantize_rows_int8", (hipStream_t)stream);
    if (rc == QG_OK) log_first("quantize_rows_int8 M=%d K=%d", M, K);
    return rc;
}

} // extern "C"
