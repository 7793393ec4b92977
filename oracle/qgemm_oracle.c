/*
 * Plain CPU oracle for the packed-int4 weight GEMM.  TEST INFRASTRUCTURE ONLY:
 * only the tests, the smoke check and the benchmark's CPU-baseline leg may load
 * this library.  It shares no code, header, table or constant with the HIP
 * library: it reads the LOGICAL inputs (one 4-bit code per byte, fp16 scales
 * and zeros as raw IEEE binary16 bits) and never the packed layout.
 *
 * Everything is computed in fp64 with naive loops, in the order the method is
 * defined.  Sources (web pages; cited by title and section):
 *   [Marlin-Ada]  "Marlin INT4 on Ada - how it works" (TinyLoop docs)
 *   [HyperQwen]   "HyperQwen int8 tensor-core fix of the Marlin W4A8 negative
 *                 scale bug and per-layer activation quantization" (kwkr.cn)
 *
 * Every function here is pinned by the CPU test-suite against values fixed by
 * the pages and by mathematics (exact rational brute force, closed-form
 * identities, invariants, hand-worked fixtures); none is "parity unpinned".
 */
#include <stdint.h>
#include <stddef.h>
#include <stdlib.h>
#include <math.h>
#include <string.h>

/* ---- IEEE 754 binary16 <-> binary64, written from the format definition ----
 * binary16: 1 sign bit, 5 exponent bits (bias 15), 10 fraction bits.
 * exponent 0 -> subnormal (f * 2^-24); exponent 31 -> inf / NaN.            */
double oracle_f16_to_f64(uint16_t h)
{
    int sign = (h >> 15) & 1;
    int e = (h >> 10) & 0x1f;
    int f = h & 0x3ff;
    double v;
    if (e == 0)
        v = ldexp((double)f, -24);
    else if (e == 31)
        v = f ? NAN : INFINITY;
    else
        v = ldexp((double)(1024 + f), e - 25);
    return sign ? -v : v;
}

/* Round an fp64 value to the nearest binary16, ties to even.  Values whose
 * magnitude rounds past 65504 become infinity.                               */
uint16_t oracle_f64_to_f16(double x)
{
    uint16_t sign = (uint16_t)(signbit(x) ? 0x8000 : 0);
    double a = fabs(x);
    if (isnan(x)) return (uint16_t)(sign | 0x7e00);
    if (a == 0.0) return sign;
    /* choose the quantum of the binade that contains a (subnormals: 2^-24) */
    int ex;
    frexp(a, &ex);                 /* a = m * 2^ex, m in [0.5, 1) */
    int e_unb = ex - 1;            /* a in [2^e_unb, 2^(e_unb+1)) */
    if (e_unb < -14) e_unb = -14;  /* subnormal range shares the 2^-24 quantum */
    double quantum = ldexp(1.0, e_unb - 10);
    double q = a / quantum;        /* exact: power-of-two division */
    double fl = floor(q);
    double rem = q - fl;
    double n;
    if (rem > 0.5) n = fl + 1.0;
    else if (rem < 0.5) n = fl;
    else n = (fmod(fl, 2.0) == 0.0) ? fl : fl + 1.0;
    double r = n * quantum;
    if (r > 65504.0) return (uint16_t)(sign | 0x7c00);
    /* encode r exactly */
    if (r < ldexp(1.0, -14)) {     /* subnormal (or rounded up to min normal) */
        long m = (long)(r / ldexp(1.0, -24));
        return (uint16_t)(sign | (uint16_t)m);  /* m == 1024 encodes 2^-14 */
    }
    int ex2;
    double m2 = frexp(r, &ex2);    /* r = m2 * 2^ex2, m2 in [0.5,1) */
    int biased = ex2 - 1 + 15;
    long frac = (long)((m2 * 2.0 - 1.0) * 1024.0);
    return (uint16_t)(sign | (uint16_t)(biased << 10) | (uint16_t)frac);
}

/* Groups of g consecutive k: k belongs to group k / g, and when g does not
 * divide K the last group is partial (K not a multiple of 128 is a supported
 * shape; the pages' dispatcher requires the multiple, so a partial group is
 * this library's own reading of "one scale per group of g k").            */
static int n_groups(int K, int g) { return (K + g - 1) / g; }

/* ---- [HyperQwen] section "hidden landmine: the negative group scale bug" ----
 * For every (group, column) whose scale is strictly negative, flip the scale's
 * sign and replace each code v of that group by 16 - v; the code 0 (value -8)
 * would become 16, which does not fit in 4 bits, and is clamped to 15.
 * Operates in place on copies owned by the caller.  Returns how many codes
 * were clamped.                                                              */
long oracle_fold_negative_scales(uint8_t *q, uint16_t *s, int K, int N, int g)
{
    long clamped = 0;
    int G = n_groups(K, g);
    for (int gi = 0; gi < G; ++gi) {
        for (int n = 0; n < N; ++n) {
            double sv = oracle_f16_to_f64(s[(size_t)gi * N + n]);
            if (!(sv < 0.0)) continue;          /* strict: -0.0 is not folded */
            s[(size_t)gi * N + n] ^= 0x8000;    /* s -> -s (exact in binary16) */
            for (int k = gi * g; k < (gi + 1) * g && k < K; ++k) {
                int v = q[(size_t)k * N + n];
                int nv = 16 - v;
                if (nv > 15) { nv = 15; ++clamped; }
                q[(size_t)k * N + n] = (uint8_t)nv;
            }
        }
    }
    return clamped;
}

/* ---- [Marlin-Ada] "The core mismatch: symmetric vs asymmetric" ----
 * symmetric offset-binary:  W[k,n] = (q[k,n] - 8) * scale[g,n]               */
void oracle_dequant_sym(const uint8_t *q, const uint16_t *s, int K, int N, int g,
                        double *W)
{
    for (int k = 0; k < K; ++k)
        for (int n = 0; n < N; ++n)
            W[(size_t)k * N + n] = ((double)q[(size_t)k * N + n] - 8.0) *
                                   oracle_f16_to_f64(s[(size_t)(k / g) * N + n]);
}

/* asymmetric min-max:  W[k,n] = q[k,n] * scale[g,n] + zero[g,n]             */
void oracle_dequant_asym(const uint8_t *q, const uint16_t *s, const uint16_t *z,
                         int K, int N, int g, double *W)
{
    for (int k = 0; k < K; ++k)
        for (int n = 0; n < N; ++n) {
            size_t gi = (size_t)(k / g) * N + n;
            W[(size_t)k * N + n] = (double)q[(size_t)k * N + n] * oracle_f16_to_f64(s[gi]) +
                                   oracle_f16_to_f64(z[gi]);
        }
}

/* delta[g,n] = zero[g,n] + 8 * scale[g,n]: the per-cell residual between the
 * asymmetric and the symmetric dequantization.  Returned exactly in fp64
 * (the sum of two binary16 values is exact in binary64) and rounded once to
 * binary16 (ties to even).  Either output pointer may be NULL.               */
void oracle_delta(const uint16_t *s, const uint16_t *z, int G, int N,
                  double *delta_exact, uint16_t *delta_f16)
{
    for (size_t i = 0; i < (size_t)G * N; ++i) {
        double d = oracle_f16_to_f64(z[i]) + 8.0 * oracle_f16_to_f64(s[i]);
        if (delta_exact) delta_exact[i] = d;
        if (delta_f16) delta_f16[i] = oracle_f64_to_f16(d);
    }
}

/* Plain product C[M,N] = A[M,K] . W[K,N] (row-major), fp64, loop order m-k-n,
 * rows shared out over OpenMP threads.  No blocking and no reordering beyond
 * the definition of the matrix product.                                      */
void oracle_matmul(const double *A, const double *W, int M, int N, int K, double *C)
{
#pragma omp parallel for schedule(static)
    for (int m = 0; m < M; ++m) {
        double *c = C + (size_t)m * N;
        for (int n = 0; n < N; ++n) c[n] = 0.0;
        for (int k = 0; k < K; ++k) {
            double a = A[(size_t)m * K + k];
            const double *w = W + (size_t)k * N;
            for (int n = 0; n < N; ++n) c[n] += a * w[n];
        }
    }
}

static double *f16_matrix_to_f64(const uint16_t *h, size_t count)
{
    double *d = (double *)malloc(count * sizeof(double));
    if (!d) return NULL;
    for (size_t i = 0; i < count; ++i) d[i] = oracle_f16_to_f64(h[i]);
    return d;
}

/* W4A16 GEMM, C[M,N] = A[M,K] . W[K,N] with W dequantized from 4-bit codes.
 *   z == NULL : symmetric; if fold != 0, negative scales are first folded
 *               into the codes ([HyperQwen] negative-scale section).
 *   z != NULL : asymmetric, W = q*s + z (direct form; [Marlin-Ada]).
 * A is binary16 bits.  Returns 0, or -1 on allocation failure.               */
int oracle_w4a16(const uint16_t *A, const uint8_t *q, const uint16_t *s,
                 const uint16_t *z, int M, int N, int K, int g, int fold, double *C)
{
    int G = n_groups(K, g);
    size_t KN = (size_t)K * N, GN = (size_t)G * N;
    uint8_t *qc = (uint8_t *)malloc(KN);
    uint16_t *sc = (uint16_t *)malloc(GN * sizeof(uint16_t));
    double *W = (double *)malloc(KN * sizeof(double));
    double *Ad = f16_matrix_to_f64(A, (size_t)M * K);
    if (!qc || !sc || !W || !Ad) { free(qc); free(sc); free(W); free(Ad); return -1; }
    memcpy(qc, q, KN);
    memcpy(sc, s, GN * sizeof(uint16_t));
    if (z == NULL) {
        if (fold) oracle_fold_negative_scales(qc, sc, K, N, g);
        oracle_dequant_sym(qc, sc, K, N, g, W);
    } else {
        oracle_dequant_asym(qc, sc, z, K, N, g, W);
    }
    oracle_matmul(Ad, W, M, N, K, C);
    free(qc); free(sc); free(W); free(Ad);
    return 0;
}

/* Same product evaluated only at the listed output cells (rows[i], cols[i]),
 * one dot product per cell: for full-size shapes where the dense oracle is
 * too slow.  Codes, scales and zeros are the caller's logical inputs; the
 * fold (symmetric only) is applied to the cells' columns as above.           */
int oracle_w4a16_cells(const uint16_t *A, const uint8_t *q, const uint16_t *s,
                       const uint16_t *z, int M, int N, int K, int g, int fold,
                       int n_cells, const int *rows, const int *cols, double *out)
{
    (void)M;
#pragma omp parallel for schedule(static)
    for (int i = 0; i < n_cells; ++i) {
        int m = rows[i], n = cols[i];
        double acc = 0.0;
        for (int k = 0; k < K; ++k) {
            size_t gi = (size_t)(k / g) * N + n;
            double sv = oracle_f16_to_f64(s[gi]);
            int v = q[(size_t)k * N + n];
            double w;
            if (z != NULL) {
                w = (double)v * sv + oracle_f16_to_f64(z[gi]);
            } else {
                if (fold && sv < 0.0) {   /* fold, as oracle_fold_negative_scales */
                    sv = -sv;
                    v = 16 - v;
                    if (v > 15) v = 15;
                }
                w = ((double)v - 8.0) * sv;
            }
            acc += oracle_f16_to_f64(A[(size_t)m * K + k]) * w;
        }
        out[i] = acc;
    }
    return 0;
}

/* ---- [Marlin-Ada] "The pipeline, end to end", a_group_sum stage ----
 * a_sum[m, g] = sum over k in group g of A[m, k], in fp64.                   */
void oracle_group_sum(const uint16_t *A, int M, int K, int g, double *a_sum)
{
    int G = n_groups(K, g);
    for (int m = 0; m < M; ++m)
        for (int gi = 0; gi < G; ++gi) {
            double acc = 0.0;
            for (int k = gi * g; k < (gi + 1) * g && k < K; ++k)
                acc += oracle_f16_to_f64(A[(size_t)m * K + k]);
            a_sum[(size_t)m * G + gi] = acc;
        }
}

/* correction_accum stage: C_out[m,n] = C_in[m,n] + sum_g a_sum[m,g] * delta[g,n]
 * with C_in and delta binary16 bits, result kept in fp64.                    */
int oracle_group_sum_correction(const uint16_t *A, const uint16_t *delta,
                                const uint16_t *C_in, int M, int N, int K, int g,
                                double *C_out)
{
    int G = n_groups(K, g);
    double *as = (double *)malloc((size_t)M * G * sizeof(double));
    if (!as) return -1;
    oracle_group_sum(A, M, K, g, as);
    for (int m = 0; m < M; ++m)
        for (int n = 0; n < N; ++n) {
            double acc = oracle_f16_to_f64(C_in[(size_t)m * N + n]);
            for (int gi = 0; gi < G; ++gi)
                acc += as[(size_t)m * G + gi] * oracle_f16_to_f64(delta[(size_t)gi * N + n]);
            C_out[(size_t)m * N + n] = acc;
        }
    free(as);
    return 0;
}

/* ---- [HyperQwen] "why int8 activation quantization (W4A8) is worth doing" ----
 * Grouped W4A8: expert e owns rows offsets[e] .. offsets[e+1]-1 of A_q and its
 * own 4-bit weights (codes q_e [K,N], scales s_e [G,N]; zeros z_e [G,N] for
 * an asymmetric weight, z == NULL for a symmetric one).  Per row m of expert
 * e, per group g and column n, the integer partial product
 *     acc[m,g,n] = sum_{k in g} A_q[m,k] * (v_e[k,n] - 8)
 * is exact (int64 here), and the output is
 *     symmetric:   C[m,n] = a_scale[m] * sum_g s_e[g,n] * acc[m,g,n]
 *     asymmetric:  C[m,n] = a_scale[m] * sum_k A_q[m,k] * (v_e[k,n] s_e[g,n] + z_e[g,n])
 *                         = a_scale[m] * sum_g (s_e[g,n] P[m,g,n] + z_e[g,n] Q[m,g])
 * with the exact integer sums P = sum_{k in g} A_q v and Q = sum_{k in g} A_q
 * (the asymmetric form is [HyperQwen] "how to verify", point 2: zero-point
 * uint4 weights with int8 activations), all in fp64.  Negative scales are
 * folded first when fold != 0, for a symmetric weight only (an asymmetric
 * weight is never folded).  acc may be NULL.  Returns 0, or -1 on allocation
 * failure.                                                                   */
int oracle_w4a8(const int8_t *Aq, const float *a_scale, const uint8_t *q,
                const uint16_t *s, const uint16_t *z, const int32_t *offsets, int E,
                int M_total, int N, int K, int g, int fold, int64_t *acc, double *C)
{
    int G = n_groups(K, g);
    size_t KN = (size_t)K * N, GN = (size_t)G * N;
    uint8_t *qc = (uint8_t *)malloc(KN);
    uint16_t *sc = (uint16_t *)malloc(GN * sizeof(uint16_t));
    int64_t *row_acc = (int64_t *)malloc(GN * sizeof(int64_t));
    int64_t *row_p = (int64_t *)malloc(GN * sizeof(int64_t));
    int64_t *row_q = (int64_t *)malloc((size_t)G * sizeof(int64_t));
    if (!qc || !sc || !row_acc || !row_p || !row_q) {
        free(qc); free(sc); free(row_acc); free(row_p); free(row_q);
        return -1;
    }
    (void)M_total;
    for (int e = 0; e < E; ++e) {
        const uint16_t *ze = z ? z + (size_t)e * GN : NULL;
        memcpy(qc, q + (size_t)e * KN, KN);
        memcpy(sc, s + (size_t)e * GN, GN * sizeof(uint16_t));
        if (fold && !ze) oracle_fold_negative_scales(qc, sc, K, N, g);
        for (int m = offsets[e]; m < offsets[e + 1]; ++m) {
            for (size_t i = 0; i < GN; ++i) row_acc[i] = row_p[i] = 0;
            for (int gi = 0; gi < G; ++gi) row_q[gi] = 0;
            for (int k = 0; k < K; ++k) {
                int64_t a = Aq[(size_t)m * K + k];
                int64_t *ra = row_acc + (size_t)(k / g) * N;
                int64_t *rp = row_p + (size_t)(k / g) * N;
                const uint8_t *qr = qc + (size_t)k * N;
                row_q[k / g] += a;
                for (int n = 0; n < N; ++n) {
                    ra[n] += a * ((int64_t)qr[n] - 8);
                    rp[n] += a * (int64_t)qr[n];
                }
            }
            if (acc) memcpy(acc + (size_t)m * GN, row_acc, GN * sizeof(int64_t));
            for (int n = 0; n < N; ++n) {
                double t = 0.0;
                for (int gi = 0; gi < G; ++gi) {
                    size_t i = (size_t)gi * N + n;
                    double sv = oracle_f16_to_f64(sc[i]);
                    if (ze)
                        t += sv * (double)row_p[i] + oracle_f16_to_f64(ze[i]) * (double)row_q[gi];
                    else
                        t += sv * (double)row_acc[i];
                }
                C[(size_t)m * N + n] = (double)a_scale[m] * t;
            }
        }
    }
    free(qc); free(sc); free(row_acc); free(row_p); free(row_q);
    return 0;
}

/* ---- [HyperQwen] "why int8 activation quantization (W4A8) is worth doing":
 * the activations of the W4A8 path are quantized per token (per row) to int8.
 * The page names no rule; this is the plain symmetric absmax one:
 *     a_scale[m] = max_k |A[m,k]| / 127
 *     A_q[m,k]   = clamp(round_half_even(A[m,k] / a_scale[m]), -127, 127)
 * and a row of zeros gets a_scale 0 and codes 0.  Floating point decides the
 * integer codes here, so the precision is part of the definition: both
 * divisions are single IEEE binary32 operations rounded to nearest even (the
 * precision the GPU kernel takes them in).  binary16 values convert to
 * binary32 exactly.                                                          */
void oracle_quantize_rows_int8(const uint16_t *A, int M, int K, int8_t *Aq, float *a_scale)
{
    for (int m = 0; m < M; ++m) {
        const uint16_t *a = A + (size_t)m * K;
        float amax = 0.0f;
        for (int k = 0; k < K; ++k) {
            float v = fabsf((float)oracle_f16_to_f64(a[k]));
            if (v > amax) amax = v;
        }
        float sc = amax / 127.0f;
        a_scale[m] = sc;
        for (int k = 0; k < K; ++k) {
            int8_t c = 0;
            if (sc > 0.0f) {
                float r = rintf((float)oracle_f16_to_f64(a[k]) / sc);
                if (r > 127.0f) r = 127.0f;
                if (r < -127.0f) r = -127.0f;
                c = (int8_t)r;
            }
            Aq[(size_t)m * K + k] = c;
        }
    }
}

/* ---- [Marlin-Ada] "Gaps and follow-ups": the fused SwiGLU of an MLP's gate
 * and up projections (mlp_gate and mlp_up in one kernel).  The page does not
 * define it; the standard definition is used:
 *     H[m,n] = silu(G[m,n]) * U[m,n],   silu(x) = x / (1 + exp(-x))
 * where G = C[:, 0:N] and U = C[:, N:2N] are the two halves of the product
 * C = A . [W_gate | W_up]  ([M, 2N], row-major, fp64).                      */
void oracle_silu_mul(const double *C, int M, int N, double *H)
{
    for (int m = 0; m < M; ++m)
        for (int n = 0; n < N; ++n) {
            double g = C[(size_t)m * 2 * N + n];
            double u = C[(size_t)m * 2 * N + N + n];
            H[(size_t)m * N + n] = g / (1.0 + exp(-g)) * u;
        }
}
