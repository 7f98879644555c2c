/*
 * attention_oracle.c -- the plain CPU reference for the pages' second
 * @cluster example, flash attention.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the
 * benchmark's CPU-baseline leg may load this library.  The GPU library never
 * links, includes or calls it, and it shares no code with the GPU library.
 *
 * What it computes: the "@cluster" page (sections "The same names at two
 * levels" and the Flash Attention example) declares
 *   flash_attention(Q: f32[Nq, D], K: f32[Nk, D], V: f32[Nk, D],
 *                   O: f32[Nq, D], scale: f32)
 * and cites the FlashAttention paper; its body is not on the pages.  The
 * reading taken is exact (unmasked) attention:
 *   S[i][j] = scale * sum_d Q[i][d] * K[j][d]
 *   P[i][j] = exp(S[i][j] - max_j S[i][j]) / sum_j exp(S[i][j] - max_j S[i][j])
 *   O[i][d] = sum_j P[i][j] * V[j][d]
 * i.e. a row softmax over the keys.  Each query row is computed in fp64 in
 * two passes (scores and their maximum, then weights, sum and output) and
 * rounded once to fp32.
 *
 * The bound (the acceptance rule for an fp32 implementation that forms S
 * with fp32 products and sums, takes exp of scores less a running maximum,
 * and accumulates the weighted sum and the weight sum in fp32):
 *   Bnd[i][d] = sum_j P[i][j] * delta[i][j] * (|V[j][d]| + |O[i][d]|)
 *             + (5*Nk + 8) * u * sum_j P[i][j] * |V[j][d]|  + 1e-30,
 * with u = 2^-24 and the relative error of one weight
 *   delta[i][j] = scale * (2*D*u * sum_d |Q[i][d]*K[j][d]|
 *                          + 2*u * |S0[i][j]| + u * (S0max[i] - S0[i][j])) + 4*u,
 * where S0 = S / scale (the unscaled dot product).  The first sum is the
 * effect of the per-weight errors on the normalised average (first order),
 * the second the fp32 accumulation of the Nk terms of the output and of the
 * weight sum, the rescaling of running sums and the final division.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>

#define ATT_U 5.9604644775390625e-08 /* 2^-24 */

static void attention_row(int64_t i, int64_t Nk, int64_t D, const float* Q, int64_t ldq,
                          const float* K, int64_t ldk, const float* V, int64_t ldv,
                          float scale, double* s0, double* w, double* delta, float* out,
                          double* bnd) {
    const float* q = Q + i * ldq;
    /* pass 1: unscaled dot products and the sum of |products| of each */
    for (int64_t j = 0; j < Nk; ++j) {
        const float* k = K + j * ldk;
        double s = 0.0, a = 0.0;
        for (int64_t d = 0; d < D; ++d) {
            const double p = (double)q[d] * (double)k[d];
            s += p;
            a += fabs(p);
        }
        s0[j] = s;
        delta[j] = a;
    }
    double smax = -INFINITY, s0max = -INFINITY;
    for (int64_t j = 0; j < Nk; ++j) {
        const double ss = (double)scale * s0[j];
        if (ss > smax) smax = ss;
        if (s0[j] > s0max) s0max = s0[j];
    }
    /* pass 2: weights, their sum, and each weight's relative error bound */
    double l = 0.0;
    for (int64_t j = 0; j < Nk; ++j) {
        w[j] = exp((double)scale * s0[j] - smax);
        l += w[j];
        delta[j] = fabs((double)scale) * (2.0 * (double)D * ATT_U * delta[j] +
                                          2.0 * ATT_U * fabs(s0[j]) +
                                          ATT_U * fabs(s0max - s0[j])) +
                   4.0 * ATT_U;
    }
    for (int64_t d = 0; d < D; ++d) {
        double o = 0.0;
        for (int64_t j = 0; j < Nk; ++j) o += w[j] * (double)V[j * ldv + d];
        o /= l;
        out[d] = (float)o;
        if (bnd) {
            double pert = 0.0, mag = 0.0;
            for (int64_t j = 0; j < Nk; ++j) {
                const double p = w[j] / l, av = fabs((double)V[j * ldv + d]);
                pert += p * delta[j] * (av + fabs(o));
                mag += p * av;
            }
            bnd[d] = pert + (5.0 * (double)Nk + 8.0) * ATT_U * mag + 1e-30;
        }
    }
}

/*
 * Rows rows[t] (t < count) of O, into out[t*ldo ...], bounds into bnd[t*ldb
 * ...] (bnd may be NULL).  Returns 0, -1 when a work buffer cannot be
 * allocated, -2 on bad arguments.
 */
int oracle_attention_rows(int64_t Nq, int64_t Nk, int64_t D, const float* Q, int64_t ldq,
                          const float* K, int64_t ldk, const float* V, int64_t ldv, float scale,
                          int64_t count, const int64_t* rows, float* out, int64_t ldo,
                          double* bnd, int64_t ldb) {
    if (Nq < 0 || Nk < 1 || D < 1 || count < 0) return -2;
    if (ldq < D || ldk < D || ldv < D || ldo < D || (bnd && ldb < D)) return -2;
    for (int64_t t = 0; t < count; ++t)
        if (rows[t] < 0 || rows[t] >= Nq) return -2;
    int failed = 0;
#pragma omp parallel
    {
        double* s0 = (double*)malloc(sizeof(double) * (size_t)Nk);
        double* w = (double*)malloc(sizeof(double) * (size_t)Nk);
        double* delta = (double*)malloc(sizeof(double) * (size_t)Nk);
        if (!s0 || !w || !delta) {
#pragma omp atomic write
            failed = 1;
        } else {
#pragma omp for schedule(dynamic, 1)
            for (int64_t t = 0; t < count; ++t)
                attention_row(rows[t], Nk, D, Q, ldq, K, ldk, V, ldv, scale, s0, w, delta,
                              out + t * ldo, bnd ? bnd + t * ldb : NULL);
        }
        free(s0);
        free(w);
        free(delta);
    }
    return failed ? -1 : 0;
}
