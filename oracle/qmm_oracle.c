/*
 * qmm_oracle.c -- plain CPU oracle for the W4A16 group-128 quantized matmul,
 * its split-K form, the split-K partial reduction and the dense bf16 variant.
 *
 * TEST INFRASTRUCTURE. Only the test suite, the smoke check and the benchmark's
 * CPU-baseline leg load this library. It shares no code, header, table or helper
 * with the GPU library and includes no HIP header. It is slow on purpose: every
 * function is the plain definition of what it computes, written so that it can
 * be checked against the pages by eye.
 *
 * What it computes, and where that is defined:
 *
 *   q[n,k] = nibble (k mod 8) of word Wq[n][k/8], low bits first
 *            (the packed uint4 layout: eight 4-bit values per 32-bit word along K;
 *             tiny-llm's page prints no order inside a word; lowest field first is the
 *             reading taken).
 *   w[n,k] = scale[n,g] * q[n,k] + bias[n,g],  g = k / 128
 *            (tiny-llm "Week 2 Day 7: Split-K Prefill", Task 2: the W4A16 g128
 *             loader and dequantizer; per-(row, 128-group) bf16 scale and bias.)
 *   C[m,n] = sum_k A[m,k] * w[n,k]                        (the product C = A @ W.T,
 *            "Why Split the Reduction Dimension?")
 *   split:  C[m,n] = sum_p ( sum_{k in partition p} A[m,k] * w[n,k] )
 *            with s partitions of equal length on 128-value group boundaries
 *            (Task 2: same reduction length, group-aligned start and end).
 *   reduce: C_bf16[m,n] = bf16_rne( fp32 sum over p = 0..s-1 of partial[p,m,n] )
 *            (Task 4: one thread per output, sum all partitions in FP32, cast once).
 *   other weight formats (skillsdirectory "Optimize Prefill vs Decode Kernels",
 *   step 6: weight-only W4A16 and W8A16, dequantisation fused into the matmul):
 *            q[n,k] = field (k mod (32/b)) of word Wq[n][k/(32/b)], b = 4 or 8 bits,
 *            lowest bits first; w[n,k] = scale[n, k/gs] * q[n,k] + bias[n, k/gs]
 *            for a group size gs of 32, 64 or 128; the split partitions stay on
 *            128-value boundaries (which are group boundaries for every gs).
 *   decode attention (skillsdirectory "Optimize Prefill vs Decode Kernels", step 4
 *   and the correctness notes on split-KV with an LSE combine): for request b, query
 *   token i of Mq and query head h,
 *            allowed keys j < L_b - Mq + 1 + i (the query's own position and before),
 *            s_j = scale * sum_d Q[b,i,h,d] * K[b,h/G,j,d]   (G = Hq/Hkv query heads per
 *            key/value head), O[b,i,h,:] = sum_j softmax(s)_j * V[b,h/G,j,:].
 *            The oracle is this plain definition in fp64; the split into key ranges
 *            and their merge are the GPU method's business.
 *   dense:  C[m,n] = sum_k A[m,k] * B[n,k], split into s near-equal partitions of
 *            64-value units when K is a multiple of 64, else of 32-value granules
 *            (gpu-kernels-explained "Split-K, streams and overlap", Concept / Maths: k
 *            cut into s slices, a second pass adds the partials).
 *
 * All matmul arithmetic is fp64 in ascending k (inner) and ascending p (outer).
 * The reduce is fp32 because the page fixes FP32 for that sum.
 * Parity is pinned by the tests in tests/test_oracle_pins.py (brute force in exact
 * rationals, closed forms, library routines, the split invariance).
 */
#include <math.h>
#include <pthread.h>
#include <stddef.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORACLE_GROUP 128
#define ORACLE_GRANULE 32

/* ---- scalar definitions ------------------------------------------------- */

/* The real number a bf16 bit pattern denotes (bf16 = the top 16 bits of an
 * IEEE binary32); exact in double. */
double oracle_bf16_value(uint16_t bits)
{
    uint32_t u = (uint32_t)bits << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

/* Nearest bf16 to a finite x, ties to the even significand (round-to-nearest-
 * even), written from the definition: bf16 keeps 8 significant bits and shares
 * binary32's exponent range, so the spacing of bf16 values around |x| in
 * [2^e, 2^(e+1)) is 2^(e-7), and never below 2^-133 (the subnormal spacing).
 * Values beyond the largest finite bf16 round to infinity. */
uint16_t oracle_bf16_round(double x)
{
    if (x == 0.0) return signbit(x) ? 0x8000u : 0x0000u;
    if (isnan(x)) return 0x7fc0u;
    int sign = x < 0.0;
    double ax = fabs(x);
    int e;
    frexp(ax, &e);                     /* ax = f * 2^e, f in [0.5, 1) -> ax in [2^(e-1), 2^e) */
    int spacing_exp = (e - 1) - 7;     /* 8 significant bits */
    if (spacing_exp < -133) spacing_exp = -133;
    double t = ldexp(ax, -spacing_exp); /* exact: power-of-two scaling */
    double fl = floor(t);
    double frac = t - fl;               /* exact */
    if (frac > 0.5 || (frac == 0.5 && fmod(fl, 2.0) != 0.0)) fl += 1.0;
    double r = ldexp(fl, spacing_exp);  /* a bf16 value, or 2^128 on overflow */
    float rf = (float)r;                /* exact: at most 8 significant bits */
    uint32_t u;
    memcpy(&u, &rf, sizeof u);
    if (r >= 0x1p128) u = 0x7f800000u;  /* overflow -> infinity */
    uint16_t b = (uint16_t)(u >> 16);
    return sign ? (uint16_t)(b | 0x8000u) : b;
}

/* q[n,k]: nibble (k mod 8) of word Wq[n][k/8], low nibble first. */
int oracle_nibble(const uint32_t *Wq, int K, int n, int k)
{
    uint32_t word = Wq[(size_t)n * (size_t)(K / 8) + (size_t)(k / 8)];
    return (int)((word >> (4 * (k % 8))) & 0xFu);
}

/* w[n,k] = scale[n,g] * q[n,k] + bias[n,g] for the whole matrix, in fp64. */
void oracle_dequant_w4a16(const uint32_t *Wq, const uint16_t *scale, const uint16_t *bias,
                          int N, int K, double *w)
{
    int G = K / ORACLE_GROUP;
    for (int n = 0; n < N; ++n)
        for (int k = 0; k < K; ++k) {
            int g = k / ORACLE_GROUP;
            double sc = oracle_bf16_value(scale[(size_t)n * G + g]);
            double bi = oracle_bf16_value(bias[(size_t)n * G + g]);
            w[(size_t)n * K + k] = sc * (double)oracle_nibble(Wq, K, n, k) + bi;
        }
}

/* Partition p of s over G groups: equal length, group aligned. Returns 0 on
 * success, -1 if s does not divide G (the method requires equal partitions). */
int oracle_partition_groups(int G, int s, int p, int *g_begin, int *g_end)
{
    if (s <= 0 || p < 0 || p >= s || G % s != 0) return -1;
    *g_begin = p * (G / s);
    *g_end = (p + 1) * (G / s);
    return 0;
}

/* Partition p of s over U granules (dense variant): near-equal, floor bounds. */
int oracle_partition_granules(int U, int s, int p, int *u_begin, int *u_end)
{
    if (s <= 0 || s > U || p < 0 || p >= s) return -1;
    *u_begin = (int)(((long long)p * U) / s);
    *u_end = (int)(((long long)(p + 1) * U) / s);
    return 0;
}

/* ---- the matmuls (row-parallel over host threads) ---------------------- */

typedef struct {
    const double *a;    /* [M][K] */
    const double *b;    /* [N][K] (w for W4A16, B for dense) */
    int M, N, K;
    const int *kb;      /* s+1 partition bounds in k */
    int s;
    double *C;          /* [M][N] */
    int m0, m1;
} job_t;

static void *run_rows(void *arg)
{
    job_t *j = (job_t *)arg;
    for (int m = j->m0; m < j->m1; ++m) {
        const double *arow = j->a + (size_t)m * j->K;
        for (int n = 0; n < j->N; ++n) {
            const double *brow = j->b + (size_t)n * j->K;
            double total = 0.0;
            for (int p = 0; p < j->s; ++p) {
                double part = 0.0;
                for (int k = j->kb[p]; k < j->kb[p + 1]; ++k) part += arow[k] * brow[k];
                total = (p == 0) ? part : total + part;
            }
            j->C[(size_t)m * j->N + n] = total;
        }
    }
    return NULL;
}

static int run_threads(const double *a, const double *b, int M, int N, int K,
                       const int *kb, int s, double *C, int nthreads)
{
    if (nthreads < 1) nthreads = 1;
    if (nthreads > M) nthreads = M;
    pthread_t *th = (pthread_t *)calloc((size_t)nthreads, sizeof *th);
    job_t *jobs = (job_t *)calloc((size_t)nthreads, sizeof *jobs);
    if (!th || !jobs) { free(th); free(jobs); return -2; }
    for (int t = 0; t < nthreads; ++t) {
        jobs[t] = (job_t){a, b, M, N, K, kb, s, C,
                          (int)(((long long)t * M) / nthreads),
                          (int)(((long long)(t + 1) * M) / nthreads)};
    }
    int started = 0;
    for (int t = 1; t < nthreads; ++t)
        if (pthread_create(&th[t], NULL, run_rows, &jobs[t]) == 0) started = t; else break;
    run_rows(&jobs[0]);
    for (int t = 1; t <= started; ++t) pthread_join(th[t], NULL);
    for (int t = started + 1; t < nthreads; ++t) run_rows(&jobs[t]);  /* thread start failed */
    free(th);
    free(jobs);
    return 0;
}

static double *bf16_matrix_to_f64(const uint16_t *x, size_t count)
{
    double *d = (double *)malloc(count * sizeof *d);
    if (!d) return NULL;
    for (size_t i = 0; i < count; ++i) d[i] = oracle_bf16_value(x[i]);
    return d;
}

/* C[M][N] (fp64) = the W4A16 g128 product, summed per partition (s equal
 * group-aligned partitions, s = 1 for the plain sum). Returns 0, or -1 on a
 * bad shape / split, -2 on allocation failure. */
int oracle_qmm_w4a16(const uint16_t *A, const uint32_t *Wq, const uint16_t *scale,
                     const uint16_t *bias, int M, int N, int K, int s, double *C, int nthreads)
{
    if (M <= 0 || N <= 0 || K <= 0 || K % ORACLE_GROUP != 0) return -1;
    int G = K / ORACLE_GROUP;
    int *kb = (int *)malloc(((size_t)s + 1) * sizeof *kb);
    if (!kb) return -2;
    for (int p = 0; p < s; ++p) {
        int gb, ge;
        if (oracle_partition_groups(G, s, p, &gb, &ge) != 0) { free(kb); return -1; }
        kb[p] = gb * ORACLE_GROUP;
        kb[p + 1] = ge * ORACLE_GROUP;
    }
    double *a = bf16_matrix_to_f64(A, (size_t)M * K);
    double *w = (double *)malloc((size_t)N * K * sizeof *w);
    if (!a || !w) { free(a); free(w); free(kb); return -2; }
    oracle_dequant_w4a16(Wq, scale, bias, N, K, w);
    int rc = run_threads(a, w, M, N, K, kb, s, C, nthreads);
    free(a); free(w); free(kb);
    return rc;
}

/* Selected outputs C[ms[i], ns[i]] of the unsplit W4A16 product, each computed
 * on its own (for shapes too large for the full product). */
int oracle_qmm_w4a16_points(const uint16_t *A, const uint32_t *Wq, const uint16_t *scale,
                            const uint16_t *bias, int M, int N, int K, int count,
                            const int *ms, const int *ns, double *out)
{
    if (M <= 0 || N <= 0 || K <= 0 || K % ORACLE_GROUP != 0) return -1;
    int G = K / ORACLE_GROUP;
    for (int i = 0; i < count; ++i) {
        int m = ms[i], n = ns[i];
        if (m < 0 || m >= M || n < 0 || n >= N) return -1;
        double total = 0.0;
        for (int k = 0; k < K; ++k) {
            int g = k / ORACLE_GROUP;
            double w = oracle_bf16_value(scale[(size_t)n * G + g]) * (double)oracle_nibble(Wq, K, n, k)
                     + oracle_bf16_value(bias[(size_t)n * G + g]);
            total += oracle_bf16_value(A[(size_t)m * K + k]) * w;
        }
        out[i] = total;
    }
    return 0;
}

/* C[M][N] (fp64) = A @ B.T for bf16 A[M][K], B[N][K], summed per partition over
 * s near-equal partitions of 64-value units (K a multiple of 64) or of 32-value granules. */
int oracle_qmm_dense(const uint16_t *A, const uint16_t *B, int M, int N, int K, int s,
                     double *C, int nthreads)
{
    if (M <= 0 || N <= 0 || K <= 0 || K % ORACLE_GRANULE != 0) return -1;
    const int unit = K % (2 * ORACLE_GRANULE) == 0 ? 2 * ORACLE_GRANULE : ORACLE_GRANULE;
    int U = K / unit;
    int *kb = (int *)malloc(((size_t)s + 1) * sizeof *kb);
    if (!kb) return -2;
    for (int p = 0; p < s; ++p) {
        int ub, ue;
        if (oracle_partition_granules(U, s, p, &ub, &ue) != 0) { free(kb); return -1; }
        kb[p] = ub * unit;
        kb[p + 1] = ue * unit;
    }
    double *a = bf16_matrix_to_f64(A, (size_t)M * K);
    double *b = bf16_matrix_to_f64(B, (size_t)N * K);
    if (!a || !b) { free(a); free(b); free(kb); return -2; }
    int rc = run_threads(a, b, M, N, K, kb, s, C, nthreads);
    free(a); free(b); free(kb);
    return rc;
}

/* ---- other weight formats ------------------------------------------------- */

/* q[n,k] of a b-bit code (b = 4 or 8): field (k mod (32/b)) of word
 * Wq[n][k/(32/b)], lowest bits first. */
int oracle_code(const uint32_t *Wq, int bits, int K, int n, int k)
{
    int per_word = 32 / bits;
    uint32_t word = Wq[(size_t)n * (size_t)(K / per_word) + (size_t)(k / per_word)];
    return (int)((word >> (bits * (k % per_word))) & ((1u << bits) - 1u));
}

static int format_ok(int bits, int group, int K)
{
    if (bits != 4 && bits != 8) return 0;
    if (group != 32 && group != 64 && group != 128) return 0;
    return K > 0 && K % ORACLE_GROUP == 0;
}

/* w[n,k] = scale[n, k/group] * q[n,k] + bias[n, k/group], in fp64. */
static double wq_weight(const uint32_t *Wq, int bits, int group, const uint16_t *scale,
                        const uint16_t *bias, int K, int n, int k)
{
    int G = K / group;
    int g = k / group;
    double sc = oracle_bf16_value(scale[(size_t)n * G + g]);
    double bi = oracle_bf16_value(bias[(size_t)n * G + g]);
    return sc * (double)oracle_code(Wq, bits, K, n, k) + bi;
}

/* The whole dequantised matrix w[N][K] of a (bits, group) format. Returns 0, or -1
 * for an unsupported format. */
int oracle_dequant_wq(const uint32_t *Wq, int bits, int group, const uint16_t *scale,
                      const uint16_t *bias, int N, int K, double *w)
{
    if (!format_ok(bits, group, K)) return -1;
    for (int n = 0; n < N; ++n)
        for (int k = 0; k < K; ++k) w[(size_t)n * K + k] = wq_weight(Wq, bits, group, scale, bias, K, n, k);
    return 0;
}

/* C[M][N] (fp64) of a (bits, group) weight format, summed per partition: s equal
 * partitions of the K/128 blocks of 128 values. Returns 0, -1 on a bad format,
 * shape or split, -2 on allocation failure. */
int oracle_qmm_wq(int bits, int group, const uint16_t *A, const uint32_t *Wq, const uint16_t *scale,
                  const uint16_t *bias, int M, int N, int K, int s, double *C, int nthreads)
{
    if (M <= 0 || N <= 0 || !format_ok(bits, group, K)) return -1;
    int B = K / ORACLE_GROUP;
    int *kb = (int *)malloc(((size_t)s + 1) * sizeof *kb);
    if (!kb) return -2;
    for (int p = 0; p < s; ++p) {
        int bb, be;
        if (oracle_partition_groups(B, s, p, &bb, &be) != 0) { free(kb); return -1; }
        kb[p] = bb * ORACLE_GROUP;
        kb[p + 1] = be * ORACLE_GROUP;
    }
    double *a = bf16_matrix_to_f64(A, (size_t)M * K);
    double *w = (double *)malloc((size_t)N * K * sizeof *w);
    if (!a || !w) { free(a); free(w); free(kb); return -2; }
    oracle_dequant_wq(Wq, bits, group, scale, bias, N, K, w);
    int rc = run_threads(a, w, M, N, K, kb, s, C, nthreads);
    free(a); free(w); free(kb);
    return rc;
}

/* Selected outputs C[ms[i], ns[i]] of the unsplit product of a (bits, group) format. */
int oracle_qmm_wq_points(int bits, int group, const uint16_t *A, const uint32_t *Wq,
                         const uint16_t *scale, const uint16_t *bias, int M, int N, int K, int count,
                         const int *ms, const int *ns, double *out)
{
    if (M <= 0 || N <= 0 || !format_ok(bits, group, K)) return -1;
    for (int i = 0; i < count; ++i) {
        int m = ms[i], n = ns[i];
        if (m < 0 || m >= M || n < 0 || n >= N) return -1;
        double total = 0.0;
        for (int k = 0; k < K; ++k)
            total += oracle_bf16_value(A[(size_t)m * K + k]) * wq_weight(Wq, bits, group, scale, bias, K, n, k);
        out[i] = total;
    }
    return 0;
}

/* ---- decode attention ------------------------------------------------------ */

/* O[b][i][h][:] (fp64) for bf16 Q[B][Mq][Hq][D], K and V [B][Hkv][Lmax][D], key counts
 * len[b] (Mq <= len[b] <= Lmax): softmax over the allowed keys of the scaled dot
 * products, then the weighted sum of the value rows, every step in fp64. Returns 0,
 * or -1 on a bad argument. */
int oracle_attn_decode(const uint16_t *Q, const uint16_t *K, const uint16_t *V, const int *len,
                       int B, int Mq, int Hq, int Hkv, int Lmax, int D, double scale, double *O)
{
    if (B <= 0 || Mq <= 0 || Hq <= 0 || Hkv <= 0 || Lmax <= 0 || D <= 0 || Hq % Hkv != 0) return -1;
    int G = Hq / Hkv;
    double *sc = (double *)malloc((size_t)Lmax * sizeof *sc);
    if (!sc) return -1;
    for (int b = 0; b < B; ++b) {
        if (len[b] < Mq || len[b] > Lmax) { free(sc); return -1; }
        for (int i = 0; i < Mq; ++i) {
            int nkeys = len[b] - Mq + 1 + i;
            for (int h = 0; h < Hq; ++h) {
                const uint16_t *q = Q + (((size_t)b * Mq + i) * Hq + h) * D;
                size_t kv = ((size_t)b * Hkv + (size_t)(h / G)) * (size_t)Lmax * (size_t)D;
                double mx = -INFINITY;
                for (int j = 0; j < nkeys; ++j) {
                    double dot = 0.0;
                    for (int d = 0; d < D; ++d)
                        dot += oracle_bf16_value(q[d]) * oracle_bf16_value(K[kv + (size_t)j * D + d]);
                    sc[j] = scale * dot;
                    if (sc[j] > mx) mx = sc[j];
                }
                double denom = 0.0;
                for (int j = 0; j < nkeys; ++j) {
                    sc[j] = exp(sc[j] - mx);
                    denom += sc[j];
                }
                double *o = O + (((size_t)b * Mq + i) * Hq + h) * D;
                for (int d = 0; d < D; ++d) {
                    double acc = 0.0;
                    for (int j = 0; j < nkeys; ++j) acc += sc[j] * oracle_bf16_value(V[kv + (size_t)j * D + d]);
                    o[d] = acc / denom;
                }
            }
        }
    }
    free(sc);
    return 0;
}

/* ---- the split-K reduction ------------------------------------------------ */

/* C[i] = bf16_rne( ((partial[0][i] + partial[1][i]) + ...) + partial[s-1][i] )
 * with every addition in binary32, for bf16 partial planes [s][MN]. */
void oracle_reduce_bf16(const uint16_t *partials, int s, size_t MN, uint16_t *C)
{
    for (size_t i = 0; i < MN; ++i) {
        float acc = (float)oracle_bf16_value(partials[i]);
        for (int p = 1; p < s; ++p) acc = acc + (float)oracle_bf16_value(partials[(size_t)p * MN + i]);
        C[i] = oracle_bf16_round((double)acc);
    }
}

/* Same for fp32 partial planes (the dense variant). */
void oracle_reduce_f32(const float *partials, int s, size_t MN, uint16_t *C)
{
    for (size_t i = 0; i < MN; ++i) {
        float acc = partials[i];
        for (int p = 1; p < s; ++p) acc = acc + partials[(size_t)p * MN + i];
        C[i] = oracle_bf16_round((double)acc);
    }
}
