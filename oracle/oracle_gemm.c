/*
 * oracle_gemm.c -- TEST INFRASTRUCTURE ONLY.
 *
 * A plain, slow CPU reference for the dense contraction
 *
 *     C[b][i][j] = alpha * sum_{k=0}^{K-1} A[b][i][k] * B[b][k][j]  +  beta * C0[b][i][j]
 *
 * evaluated in IEEE binary64.  Only tests/, the smoke check and the benchmark's
 * CPU-baseline leg may load this file's library; the GPU product path never
 * touches it, and the two share no code, headers or tables.
 *
 * What it follows:
 *  - OCANNL "Module Ir.Schedule", Tensorize: the micro-kernel being replaced is
 *    the single accumulation d[i,j] += a[i,k] * b[k,j] over operands that are
 *    row-major in their last two axes and not transposed.  Every schedule op on
 *    that page (Split, Partition, Pad, Stage, Privatize, Tensorize, epilogue
 *    fusion) is stated to preserve this value, up to the reassociation that
 *    Interchange licenses, so the oracle is the un-scheduled definition.
 *  - LuisaCompute "Execution Nests and coordinates", structured-region calculus
 *    and "Logical anchor and execution frontier": matmul is acc = mma(a, b, acc)
 *    with a reduce region over k; reduce may regroup, so the oracle fixes the
 *    plainest order, k increasing.
 *  - The alpha/beta epilogue is not on the pages; the reading taken is the BLAS
 *    one: beta == 0 means C0 is not read at all (NaN in C0 cannot leak).
 *
 * Numerics: every product of two fp32/bf16/fp16 values is exact in binary64
 * (each significand has at most 24 bits), so only the running sum rounds.
 * Inputs are decoded here from their bit patterns, by code written from the
 * IEEE-754 binary16 definition and the bfloat16 definition (the top half of a
 * binary32).
 *
 * Loop order: for each output row the k loop is outermost and the j loop
 * innermost, s[j] += a[i][k] * b[k][j].  Each s[j] still sees k = 0, 1, ...,
 * K-1 in order, so this is the same sequence of binary64 operations per output
 * as the textbook i-j-k triple loop; it only makes B row reads contiguous.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORACLE_F32 0
#define ORACLE_BF16 1
#define ORACLE_F16 2

/* bfloat16: the upper 16 bits of an IEEE binary32. */
double oracle_decode_bf16(uint16_t h) {
    uint32_t u = ((uint32_t)h) << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

/* IEEE-754 binary16: 1 sign bit, 5 exponent bits (bias 15), 10 fraction bits. */
double oracle_decode_f16(uint16_t h) {
    int sign = (h >> 15) & 1;
    int expo = (h >> 10) & 0x1f;
    int frac = h & 0x3ff;
    double v;
    if (expo == 0) {
        v = ldexp((double)frac, -24);                 /* zero and subnormals: f * 2^-24 */
    } else if (expo == 31) {
        v = frac ? NAN : INFINITY;
    } else {
        v = ldexp((double)(frac | 0x400), expo - 25); /* (1.f) * 2^(e-15) */
    }
    return sign ? -v : v;
}

double oracle_decode_f32(uint32_t bits) {
    float f;
    memcpy(&f, &bits, sizeof f);
    return (double)f;
}

/* Table for binary16, filled once from oracle_decode_f16 (a cache of it). */
static double f16_table[65536];
static int f16_table_ready = 0;

static void ensure_f16_table(void) {
    if (f16_table_ready) return;
    for (int h = 0; h < 65536; ++h) f16_table[h] = oracle_decode_f16((uint16_t)h);
    f16_table_ready = 1;
}

static inline double elem(const void *base, int dtype, int64_t idx) {
    if (dtype == ORACLE_F32) return (double)((const float *)base)[idx];
    uint16_t h = ((const uint16_t *)base)[idx];
    if (dtype == ORACLE_BF16) return oracle_decode_bf16(h);
    return f16_table[h];
}

static int bad_args(int64_t batch, int64_t M, int64_t N, int64_t K, int dtype,
                    int64_t lda, int64_t ldb, int64_t ldc) {
    if (batch < 0 || M < 0 || N < 0 || K < 0) return 1;
    if (dtype != ORACLE_F32 && dtype != ORACLE_BF16 && dtype != ORACLE_F16) return 1;
    if (lda < (K > 1 ? K : 1) || ldb < (N > 1 ? N : 1) || ldc < (N > 1 ? N : 1)) return 1;
    return 0;
}

/*
 * Full result.  out is binary64, laid out out[b*sO + i*ldo + j].
 * C0 is fp32 (ldc, sC); it is not read when beta == 0.
 * If absden is non-null it receives sum_k |A[i,k]| * |B[k,j]| (the parity
 * metric's denominator), with the same layout as out.
 * Returns 0 on success, 1 on bad arguments, 2 on allocation failure.
 */
int oracle_gemm(int64_t batch, int64_t M, int64_t N, int64_t K, int dtype,
                const void *A, int64_t lda, int64_t sA,
                const void *B, int64_t ldb, int64_t sB,
                const float *C0, int64_t ldc, int64_t sC,
                double alpha, double beta,
                double *out, int64_t ldo, int64_t sO, double *absden) {
    if (bad_args(batch, M, N, K, dtype, lda, ldb, ldc) || ldo < N) return 1;
    if (dtype == ORACLE_F16) ensure_f16_table();
    int failed = 0;
#pragma omp parallel
    {
        double *s = (double *)malloc(sizeof(double) * (size_t)(N > 0 ? N : 1));
        double *t = (double *)malloc(sizeof(double) * (size_t)(N > 0 ? N : 1));
        if (!s || !t) {
#pragma omp atomic write
            failed = 1;
        } else {
#pragma omp for collapse(2) schedule(dynamic, 1)
            for (int64_t b = 0; b < batch; ++b) {
                for (int64_t i = 0; i < M; ++i) {
                    const char *Ab = (const char *)A + (size_t)(b * sA) * (dtype == ORACLE_F32 ? 4 : 2);
                    const char *Bb = (const char *)B + (size_t)(b * sB) * (dtype == ORACLE_F32 ? 4 : 2);
                    for (int64_t j = 0; j < N; ++j) { s[j] = 0.0; t[j] = 0.0; }
                    for (int64_t k = 0; k < K; ++k) {
                        double a = elem(Ab, dtype, i * lda + k);
                        for (int64_t j = 0; j < N; ++j) {
                            double bv = elem(Bb, dtype, k * ldb + j);
                            s[j] += a * bv;
                            if (absden) t[j] += fabs(a) * fabs(bv);
                        }
                    }
                    for (int64_t j = 0; j < N; ++j) {
                        double c = alpha * s[j];
                        if (beta != 0.0) c += beta * (double)C0[b * sC + i * ldc + j];
                        out[b * sO + i * ldo + j] = c;
                        if (absden) absden[b * sO + i * ldo + j] = t[j];
                    }
                }
            }
        }
        free(s);
        free(t);
    }
    return failed ? 2 : 0;
}

/*
 * Sampled result: the same definition at npts chosen outputs (pb[p], pi[p],
 * pj[p]), one dot product each, k increasing.  For full-size problems whose
 * complete oracle would take hours.  out[p] and absden[p] (if non-null) are
 * binary64.  Returns 0, or 1 on bad arguments / an out-of-range point.
 */
int oracle_gemm_points(int64_t batch, int64_t M, int64_t N, int64_t K, int dtype,
                       const void *A, int64_t lda, int64_t sA,
                       const void *B, int64_t ldb, int64_t sB,
                       const float *C0, int64_t ldc, int64_t sC,
                       double alpha, double beta,
                       int64_t npts, const int64_t *pb, const int64_t *pi, const int64_t *pj,
                       double *out, double *absden) {
    if (bad_args(batch, M, N, K, dtype, lda, ldb, ldc) || npts < 0) return 1;
    for (int64_t p = 0; p < npts; ++p)
        if (pb[p] < 0 || pb[p] >= batch || pi[p] < 0 || pi[p] >= M || pj[p] < 0 || pj[p] >= N) return 1;
    if (dtype == ORACLE_F16) ensure_f16_table();
    size_t esz = dtype == ORACLE_F32 ? 4 : 2;
#pragma omp parallel for schedule(dynamic, 16)
    for (int64_t p = 0; p < npts; ++p) {
        const char *Ab = (const char *)A + (size_t)(pb[p] * sA) * esz;
        const char *Bb = (const char *)B + (size_t)(pb[p] * sB) * esz;
        double s = 0.0, t = 0.0;
        for (int64_t k = 0; k < K; ++k) {
            double a = elem(Ab, dtype, pi[p] * lda + k);
            double bv = elem(Bb, dtype, k * ldb + pj[p]);
            s += a * bv;
            t += fabs(a) * fabs(bv);
        }
        double c = alpha * s;
        if (beta != 0.0) c += beta * (double)C0[pb[p] * sC + pi[p] * ldc + pj[p]];
        out[p] = c;
        if (absden) absden[p] = t;
    }
    return 0;
}

/*
 * Fused elementwise tail (OCANNL "Module Ir.Schedule", epilogue fusion: the
 * bias add / activation / residual that follows a reduction, folded into its
 * store-back; it never reorders the reduction).  Applied to a result computed
 * with beta = 0 (out = alpha * sum), in place and in binary64:
 *     out <- act(out + bias) + beta * C0
 * bias_mode 1: one value per column, bias[b * bias_stride + j]; 2: one per
 * row, bias[b * bias_stride + i]; 0: none.  act 1: ReLU, x < 0 ? 0 : x; 2:
 * GELU, x * Phi(x) with the standard normal CDF Phi(x) = (1 + erf(x / sqrt 2)) / 2;
 * 0: none.  C0 (fp32, ldc, sC) is read only when beta != 0.
 */
static double oracle_activation(double x, int act) {
    if (act == 1) return x < 0.0 ? 0.0 : x;
    if (act == 2) return x * 0.5 * (1.0 + erf(x / sqrt(2.0)));
    return x;
}

static double tail_one(double x, int64_t b, int64_t i, int64_t j, const float *bias, int64_t bias_stride,
                       int bias_mode, int act, const float *C0, int64_t ldc, int64_t sC, double beta) {
    if (bias_mode == 1) x += (double)bias[b * bias_stride + j];
    if (bias_mode == 2) x += (double)bias[b * bias_stride + i];
    double y = oracle_activation(x, act);
    if (beta != 0.0) y += beta * (double)C0[b * sC + ldc * i + j];
    return y;
}

static int bad_tail(int bias_mode, int act, const float *bias, int64_t bias_stride) {
    return bias_mode < 0 || bias_mode > 2 || act < 0 || act > 2 || (bias_mode != 0 && !bias) || bias_stride < 0;
}

int oracle_tail(int64_t batch, int64_t M, int64_t N, double *out, int64_t ldo, int64_t sO,
                const float *bias, int64_t bias_stride, int bias_mode, int act,
                const float *C0, int64_t ldc, int64_t sC, double beta) {
    if (bad_tail(bias_mode, act, bias, bias_stride) || batch < 0 || M < 0 || N < 0 || ldo < N) return 1;
    for (int64_t b = 0; b < batch; ++b)
        for (int64_t i = 0; i < M; ++i)
            for (int64_t j = 0; j < N; ++j) {
                double *o = &out[b * sO + i * ldo + j];
                *o = tail_one(*o, b, i, j, bias, bias_stride, bias_mode, act, C0, ldc, sC, beta);
            }
    return 0;
}

int oracle_tail_points(int64_t npts, const int64_t *pb, const int64_t *pi, const int64_t *pj, double *out,
                       const float *bias, int64_t bias_stride, int bias_mode, int act,
                       const float *C0, int64_t ldc, int64_t sC, double beta) {
    if (bad_tail(bias_mode, act, bias, bias_stride) || npts < 0) return 1;
    for (int64_t p = 0; p < npts; ++p)
        out[p] = tail_one(out[p], pb[p], pi[p], pj[p], bias, bias_stride, bias_mode, act, C0, ldc, sC, beta);
    return 0;
}

int oracle_max_threads(void) {
#ifdef _OPENMP
    extern int omp_get_max_threads(void);
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/* Threads for the following calls (n >= 1); a timing control only, the
 * arithmetic of every output is the same on any number of threads. */
void oracle_set_threads(int n) {
#ifdef _OPENMP
    extern void omp_set_num_threads(int);
    if (n >= 1) omp_set_num_threads(n);
#else
    (void)n;
#endif
}
