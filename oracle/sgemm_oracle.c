/*
 * sgemm_oracle.c -- the plain CPU reference for C = alpha*A*B + beta*C.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the
 * benchmark's CPU-baseline leg may load this library.  The GPU library never
 * links, includes or calls it, and it shares no code with the GPU library.
 *
 * What it computes (definition, not an algorithm):
 *   "Show HN: Phobos - A tiny scale-free kernel language with tile-DAG
 *   support", section "Matrix Multiplication": C(MxN) = alpha*A(MxK)*B(KxN)
 *   + beta*C, all operands 32-bit floats; section "Introducing the Phobos
 *   Language": the naive SGEMM keeps one running sum per output element,
 *   adds the K products A[i][k]*B[k][j] in ascending k, then stores
 *   alpha*sum + beta*C[i][j].
 *
 * Precision: every product of two fp32 values is exact in fp64 (24+24 bits
 * fit in 53), each output sums its products in fp64 in ascending k, applies
 * alpha and beta in fp64 and is rounded once to fp32 (round to nearest even,
 * the C default).  The result is within about half an fp32 ulp of the exact
 * real value.
 *
 * Readings where the pages are silent (each also listed in the design notes):
 *   - beta == 0: C is not read (it may hold NaN); the output is alpha*sum.
 *   - K == 0: the sum is 0 and the output is beta*C (the DSL's accumulator
 *     starts at 0.0 and the loop runs zero times).
 *   - Matrices are row-major with leading dimensions lda >= K, ldb >= N,
 *     ldc >= N; elements past the logical width of a row are never read.
 *
 * The error bound (the acceptance rule for every other implementation):
 *   Bnd[i][j] = 2*K*2^-24 * (|alpha| * sum_k |A[i][k]|*|B[k][j]|
 *                            + |beta*C[i][j]|) + 1e-30,
 * with the beta term taken as 0 when beta == 0.  It is accumulated in fp64
 * beside the sum.
 *
 * Loop order: rows i are independent and are shared over OpenMP threads.
 * Within a row the k loop is outside the j loop so that B is walked along its
 * rows; each output element still receives its K products one at a time in
 * ascending k, so every element's sum is the same sequence of fp64 additions
 * as in the textbook i-j-k nest.  The per-entry function below uses the
 * i-j-k nest itself.
 */
#include <stdint.h>
#include <stdlib.h>
#include <math.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define ORACLE_U 5.9604644775390625e-08 /* 2^-24, fp32 unit roundoff */

/* Threads OpenMP will use for the full-matrix routine. */
int oracle_max_threads(void) {
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

static double bound_of(int64_t K, float alpha, float beta, double abs_sum, float c) {
    double beta_term = (beta == 0.0f) ? 0.0 : fabs((double)beta * (double)c);
    return 2.0 * (double)K * ORACLE_U * (fabs((double)alpha) * abs_sum + beta_term) + 1e-30;
}

static float finish(float alpha, float beta, double sum, float c) {
    double t = (double)alpha * sum;
    if (beta != 0.0f) t += (double)beta * (double)c;
    return (float)t;
}

/*
 * Full matrix.  Cref (ld = ldr) receives the fp32 result, Bnd (ld = ldb_nd,
 * may be NULL) the bound.  C may be NULL only when beta == 0.  Returns 0, or
 * -1 when a work buffer cannot be allocated, -2 on bad arguments.
 */
int oracle_sgemm(int64_t M, int64_t N, int64_t K, float alpha,
                 const float* A, int64_t lda, const float* B, int64_t ldb,
                 float beta, const float* C, int64_t ldc,
                 float* Cref, int64_t ldr, double* Bnd, int64_t ldbnd) {
    if (M < 0 || N < 0 || K < 0) return -2;
    if (M == 0 || N == 0) return 0;
    if (ldr < N || (Bnd && ldbnd < N)) return -2;
    if (K > 0 && (lda < K || ldb < N)) return -2;
    if (beta != 0.0f && (C == NULL || ldc < N)) return -2;
    int failed = 0;
#pragma omp parallel
    {
        double* s = (double*)malloc(sizeof(double) * (size_t)N);
        double* sa = (double*)malloc(sizeof(double) * (size_t)N);
        if (!s || !sa) {
#pragma omp atomic write
            failed = 1;
        } else {
#pragma omp for schedule(dynamic, 1)
            for (int64_t i = 0; i < M; ++i) {
                for (int64_t j = 0; j < N; ++j) { s[j] = 0.0; sa[j] = 0.0; }
                for (int64_t k = 0; k < K; ++k) {
                    const double a = (double)A[i * lda + k];
                    const float* brow = B + k * ldb;
                    for (int64_t j = 0; j < N; ++j) {
                        const double p = a * (double)brow[j];
                        s[j] += p;
                        sa[j] += fabs(p);
                    }
                }
                for (int64_t j = 0; j < N; ++j) {
                    const float c = (beta != 0.0f) ? C[i * ldc + j] : 0.0f;
                    Cref[i * ldr + j] = finish(alpha, beta, s[j], c);
                    if (Bnd) Bnd[i * ldbnd + j] = bound_of(K, alpha, beta, sa[j], c);
                }
            }
        }
        free(s);
        free(sa);
    }
    return failed ? -1 : 0;
}

/*
 * Selected entries (rows[t], cols[t]) for t < count, each by the i-j-k
 * definition: one fp64 running sum over ascending k.  For checks at sizes
 * where the full product would take too long on a CPU.
 */
int oracle_sgemm_entries(int64_t M, int64_t N, int64_t K, float alpha,
                         const float* A, int64_t lda, const float* B, int64_t ldb,
                         float beta, const float* C, int64_t ldc,
                         int64_t count, const int64_t* rows, const int64_t* cols,
                         float* out, double* bnd) {
    if (M < 0 || N < 0 || K < 0 || count < 0) return -2;
    for (int64_t t = 0; t < count; ++t)
        if (rows[t] < 0 || rows[t] >= M || cols[t] < 0 || cols[t] >= N) return -2;
#pragma omp parallel for schedule(static)
    for (int64_t t = 0; t < count; ++t) {
        const int64_t i = rows[t], j = cols[t];
        double s = 0.0, sa = 0.0;
        for (int64_t k = 0; k < K; ++k) {
            const double p = (double)A[i * lda + k] * (double)B[k * ldb + j];
            s += p;
            sa += fabs(p);
        }
        const float c = (beta != 0.0f) ? C[i * ldc + j] : 0.0f;
        out[t] = finish(alpha, beta, s, c);
        if (bnd) bnd[t] = bound_of(K, alpha, beta, sa, c);
    }
    return 0;
}

/*
 * Matrix-core variant ("Show HN: Phobos", section "Are we cuBLAS yet?", the
 * side-quest on tensor cores): every fp32 element of A and B is first
 * rounded to a 16-bit format, the products of the rounded values are
 * accumulated in a 32-bit (here: fp64) accumulator, and alpha, beta and C
 * stay fp32.  The pages do not name the rounding; the reading taken is IEEE
 * round to nearest, ties to even, for both formats.
 *
 * Formats (fmt): 1 = IEEE binary16 (11-bit significand, minimum normal
 * exponent -14, largest finite 65504), 2 = bfloat16 (8-bit significand, the
 * exponent range of fp32, largest finite (2 - 2^-7) * 2^127).
 *
 * The bound is the same rule as above, applied to the rounded inputs:
 *   2*K*2^-24 * (|alpha| * sum_k |A'[i][k]|*|B'[k][j]| + |beta*C[i][j]|) + 1e-30.
 */
#define ORACLE_F16 1
#define ORACLE_BF16 2

/*
 * Round x to the nearest number with a p-bit significand and minimum
 * exponent emin (below it the spacing stays that of the smallest normal
 * binade: subnormals), ties to even; a result above `max` in magnitude
 * becomes an infinity of x's sign.  NaN, infinities and zeros are returned
 * unchanged.  Every step is exact in fp64 for an fp32 x: the spacing q is a
 * power of two, x/q and r*q only shift exponents, and nearbyint rounds half
 * to even in the default rounding mode.
 */
static double round_to_format(float x, int p, int emin, double max) {
    if (isnan(x) || isinf(x) || x == 0.0f) return (double)x;
    int e;
    (void)frexp((double)x, &e);   /* |x| in [2^(e-1), 2^e) */
    int lead = e - 1;             /* exponent of the leading bit */
    if (lead < emin) lead = emin;
    const double q = ldexp(1.0, lead - (p - 1));
    const double r = nearbyint((double)x / q) * q;
    if (fabs(r) > max) return copysign(INFINITY, (double)x);
    return r;
}

static double round_fmt(int fmt, float x) {
    if (fmt == ORACLE_F16) return round_to_format(x, 11, -14, 65504.0);
    return round_to_format(x, 8, -126, ldexp(255.0, 120));   /* (2 - 2^-7) * 2^127 */
}

/* out[t] = in[t] rounded to format fmt (as an fp32 value), t < n. */
int oracle_round(int fmt, int64_t n, const float* in, float* out) {
    if ((fmt != ORACLE_F16 && fmt != ORACLE_BF16) || n < 0) return -2;
    for (int64_t t = 0; t < n; ++t) out[t] = (float)round_fmt(fmt, in[t]);
    return 0;
}

/*
 * Full matrix of the variant: A and B are rounded element by element into
 * packed copies (lda' = K, ldb' = N), then the fp32 definition above is
 * applied to the copies.
 */
int oracle_sgemm_tc(int fmt, int64_t M, int64_t N, int64_t K, float alpha,
                    const float* A, int64_t lda, const float* B, int64_t ldb,
                    float beta, const float* C, int64_t ldc,
                    float* Cref, int64_t ldr, double* Bnd, int64_t ldbnd) {
    if (fmt != ORACLE_F16 && fmt != ORACLE_BF16) return -2;
    if (M < 0 || N < 0 || K < 0) return -2;
    if (M == 0 || N == 0) return 0;
    if (K > 0 && (lda < K || ldb < N)) return -2;
    float* Ar = (float*)malloc(sizeof(float) * (size_t)(M * K > 0 ? M * K : 1));
    float* Br = (float*)malloc(sizeof(float) * (size_t)(K * N > 0 ? K * N : 1));
    if (!Ar || !Br) {
        free(Ar);
        free(Br);
        return -1;
    }
    for (int64_t i = 0; i < M; ++i)
        for (int64_t k = 0; k < K; ++k) Ar[i * K + k] = (float)round_fmt(fmt, A[i * lda + k]);
    for (int64_t k = 0; k < K; ++k)
        for (int64_t j = 0; j < N; ++j) Br[k * N + j] = (float)round_fmt(fmt, B[k * ldb + j]);
    const int rc = oracle_sgemm(M, N, K, alpha, Ar, K > 0 ? K : 1, Br, N, beta, C, ldc,
                                Cref, ldr, Bnd, ldbnd);
    free(Ar);
    free(Br);
    return rc;
}

/* Selected entries of the variant, each by the i-j-k definition. */
int oracle_sgemm_tc_entries(int fmt, int64_t M, int64_t N, int64_t K, float alpha,
                            const float* A, int64_t lda, const float* B, int64_t ldb,
                            float beta, const float* C, int64_t ldc,
                            int64_t count, const int64_t* rows, const int64_t* cols,
                            float* out, double* bnd) {
    if (fmt != ORACLE_F16 && fmt != ORACLE_BF16) return -2;
    if (M < 0 || N < 0 || K < 0 || count < 0) return -2;
    for (int64_t t = 0; t < count; ++t)
        if (rows[t] < 0 || rows[t] >= M || cols[t] < 0 || cols[t] >= N) return -2;
#pragma omp parallel for schedule(static)
    for (int64_t t = 0; t < count; ++t) {
        const int64_t i = rows[t], j = cols[t];
        double s = 0.0, sa = 0.0;
        for (int64_t k = 0; k < K; ++k) {
            const double p = round_fmt(fmt, A[i * lda + k]) * round_fmt(fmt, B[k * ldb + j]);
            s += p;
            sa += fabs(p);
        }
        const float c = (beta != 0.0f) ? C[i * ldc + j] : 0.0f;
        out[t] = finish(alpha, beta, s, c);
        if (bnd) bnd[t] = bound_of(K, alpha, beta, sa, c);
    }
    return 0;
}
