/*
 * ikbo_oracle.c -- CPU reference for the IKBO Linear Compression Embedding forward
 * (and, below, its backward).
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
 * benchmark's CPU-baseline leg may load this library.  The product path never
 * links, loads or calls it, and it shares no code with the HIP kernels.
 *
 * What it computes (IKBO recsys blog, "Deep Dive: Linear Compression", the
 * baseline and stage 1; aibriefing article, "kernel deep-dive case 1"):
 * the baseline op is one batched product of the projection W with, for every
 * candidate b, the candidate's input X_b in which the user's request-only rows
 * have been replicated ("materialised broadcast"):
 *
 *     X_b = [ U[map[b]] ; C[b] ]            rows 0..K_u-1 from the user,
 *                                           rows K_u..K_u+K_c-1 from the candidate
 *     W   = [ W_u | W_c ]                   [M, K_u + K_c]
 *     Y[b] = W . X_b                        [M, D]
 *
 * The pages' four optimisation stages (decomposition by linearity, zero
 * K-padding, epilogue fusion, persistent fusion) all reach this same value;
 * this file is the plain definition written out and nothing else.
 *
 * Arithmetic: every stored input value is widened exactly to double
 * (bfloat16 -> double, float -> double); each output element is one double sum
 * over k in ascending order; the result is returned in double, unrounded.
 * Built with -O2 -ffp-contract=off (no fused multiply-add, no reassociation).
 *
 * Layouts (row-major, contiguous):
 *   U   [B_u, K_u, D]     C [B_c, K_c, D]     W_u [M, K_u]     W_c [M, K_c]
 *   map [B_c] int32, 0 <= map[b] < B_u        Y   [n_rows, M, D] double
 */
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#ifdef _OPENMP
#include <omp.h>
#endif

enum { ORACLE_BF16 = 0, ORACLE_F32 = 1 };
enum { ORACLE_OK = 0, ORACLE_ERR_ARG = -1, ORACLE_ERR_MAP = -2, ORACLE_ERR_NOMEM = -3 };

static double widen(const void *base, int64_t i, int dtype)
{
    if (dtype == ORACLE_BF16) {
        uint32_t bits = (uint32_t)((const uint16_t *)base)[i] << 16;
        float f;
        memcpy(&f, &bits, sizeof f);
        return (double)f;
    }
    return (double)((const float *)base)[i];
}

/*
 * Y[r] = W . X_{b_r} for each requested candidate b_r = rows[r] (or b_r = r for
 * all B_c candidates when rows == NULL).  Returns ORACLE_ERR_MAP if any map
 * entry of a requested candidate lies outside [0, B_u).
 */
int ikbo_oracle_lce_f64(const void *U, const void *C, const int32_t *map,
                        const void *W_u, const void *W_c, double *Y,
                        int64_t B_u, int64_t B_c, int64_t K_u, int64_t K_c,
                        int64_t M, int64_t D, int dtype,
                        const int64_t *rows, int64_t n_rows, int nthreads)
{
    if (!U || !C || !map || !W_u || !W_c || !Y) return ORACLE_ERR_ARG;
    if (B_u < 1 || B_c < 0 || K_u < 0 || K_c < 0 || M < 1 || D < 1) return ORACLE_ERR_ARG;
    if (dtype != ORACLE_BF16 && dtype != ORACLE_F32) return ORACLE_ERR_ARG;
    if (rows == NULL) n_rows = B_c;
    for (int64_t r = 0; r < n_rows; ++r) {
        int64_t b = rows ? rows[r] : r;
        if (b < 0 || b >= B_c) return ORACLE_ERR_ARG;
        if (map[b] < 0 || map[b] >= B_u) return ORACLE_ERR_MAP;
    }

    const int64_t K = K_u + K_c;
    /* W = [W_u | W_c], widened. */
    double *W = (double *)malloc(sizeof(double) * (size_t)(M * (K > 0 ? K : 1)));
    if (!W) return ORACLE_ERR_NOMEM;
    for (int64_t m = 0; m < M; ++m) {
        for (int64_t k = 0; k < K_u; ++k) W[m * K + k] = widen(W_u, m * K_u + k, dtype);
        for (int64_t k = 0; k < K_c; ++k) W[m * K + K_u + k] = widen(W_c, m * K_c + k, dtype);
    }

    int status = ORACLE_OK;
#ifdef _OPENMP
    if (nthreads > 0) omp_set_num_threads(nthreads);
#else
    (void)nthreads;
#endif

#pragma omp parallel
    {
        /* Per-thread scratch: one materialised X_b and one output row. */
        double *X = (double *)malloc(sizeof(double) * (size_t)((K > 0 ? K : 1) * D));
        double *acc = (double *)malloc(sizeof(double) * (size_t)D);
        if (!X || !acc) {
#pragma omp atomic write
            status = ORACLE_ERR_NOMEM;
        } else {
#pragma omp for schedule(dynamic, 1)
            for (int64_t r = 0; r < n_rows; ++r) {
                const int64_t b = rows ? rows[r] : r;
                const int64_t u = map[b];
                /* Materialise the broadcast: the user's rows first, then the candidate's. */
                for (int64_t k = 0; k < K_u; ++k)
                    for (int64_t d = 0; d < D; ++d)
                        X[k * D + d] = widen(U, (u * K_u + k) * D + d, dtype);
                for (int64_t k = 0; k < K_c; ++k)
                    for (int64_t d = 0; d < D; ++d)
                        X[(K_u + k) * D + d] = widen(C, (b * K_c + k) * D + d, dtype);
                /* Naive product; each output element sums over k in ascending order. */
                double *Yr = Y + r * M * D;
                for (int64_t m = 0; m < M; ++m) {
                    for (int64_t d = 0; d < D; ++d) acc[d] = 0.0;
                    for (int64_t k = 0; k < K; ++k) {
                        const double w = W[m * K + k];
                        const double *x = X + k * D;
                        for (int64_t d = 0; d < D; ++d) acc[d] += w * x[d];
                    }
                    for (int64_t d = 0; d < D; ++d) Yr[m * D + d] = acc[d];
                }
            }
        }
        free(X);
        free(acc);
    }
    free(W);
    return status;
}

/*
 * Backward of the same materialised product, for an upstream gradient dY [B_c, M, D]
 * (the pages give no formulas for training; this is the adjoint of the definition
 * above, taken step by step):
 *
 *     dX_b   = W^T . dY[b]                       [K_u + K_c, D]
 *     dC[b]  = rows K_u.. of dX_b                (the candidate's own rows)
 *     dU[u] += rows 0..K_u-1 of dX_b  for every b with map[b] = u
 *                                                (the adjoint of the replication is a
 *                                                 scatter-add; users with no candidate
 *                                                 get zero)
 *     dW     = sum_b dY[b] . X_b^T               [M, K_u + K_c] = [dW_u | dW_c]
 *
 * Orders (independent of the thread count): dX_b sums over m ascending; dU adds the
 * candidates of a user in ascending b; dW sums over b ascending, then d ascending.
 * Outputs in double: dU [B_u, K_u, D], dC [B_c, K_c, D], dW_u [M, K_u], dW_c [M, K_c].
 */
int ikbo_oracle_lce_backward_f64(const void *dY, const void *U, const void *C, const int32_t *map,
                                 const void *W_u, const void *W_c, double *dU, double *dC,
                                 double *dW_u, double *dW_c, int64_t B_u, int64_t B_c, int64_t K_u,
                                 int64_t K_c, int64_t M, int64_t D, int dtype, int nthreads)
{
    if (!dY || !U || !C || !map || !W_u || !W_c || !dU || !dC || !dW_u || !dW_c) return ORACLE_ERR_ARG;
    if (B_u < 1 || B_c < 0 || K_u < 0 || K_c < 0 || M < 1 || D < 1) return ORACLE_ERR_ARG;
    if (dtype != ORACLE_BF16 && dtype != ORACLE_F32) return ORACLE_ERR_ARG;
    for (int64_t b = 0; b < B_c; ++b)
        if (map[b] < 0 || map[b] >= B_u) return ORACLE_ERR_MAP;

    const int64_t K = K_u + K_c;
    double *W = (double *)malloc(sizeof(double) * (size_t)(M * (K > 0 ? K : 1)));
    if (!W) return ORACLE_ERR_NOMEM;
    for (int64_t m = 0; m < M; ++m) {
        for (int64_t k = 0; k < K_u; ++k) W[m * K + k] = widen(W_u, m * K_u + k, dtype);
        for (int64_t k = 0; k < K_c; ++k) W[m * K + K_u + k] = widen(W_c, m * K_c + k, dtype);
    }
#ifdef _OPENMP
    if (nthreads > 0) omp_set_num_threads(nthreads);
#else
    (void)nthreads;
#endif
    int status = ORACLE_OK;
    memset(dU, 0, sizeof(double) * (size_t)(B_u * K_u * D));

    /* dX_b = W^T dY[b]: candidate rows into dC[b]; user rows added into dU[map[b]], the
     * candidates of one user taken in ascending b by the thread that owns that user. */
#pragma omp parallel
    {
        double *dX = (double *)malloc(sizeof(double) * (size_t)((K > 0 ? K : 1) * D));
        if (!dX) {
#pragma omp atomic write
            status = ORACLE_ERR_NOMEM;
        } else {
#pragma omp for schedule(dynamic, 1)
            for (int64_t b = 0; b < B_c; ++b) {
                for (int64_t k = K_u; k < K; ++k) {
                    double *out = dC + (b * K_c + (k - K_u)) * D;
                    for (int64_t d = 0; d < D; ++d) out[d] = 0.0;
                    for (int64_t m = 0; m < M; ++m) {
                        const double w = W[m * K + k];
                        for (int64_t d = 0; d < D; ++d) out[d] += w * widen(dY, (b * M + m) * D + d, dtype);
                    }
                }
            }
#pragma omp for schedule(dynamic, 1)
            for (int64_t u = 0; u < B_u; ++u) {
                for (int64_t b = 0; b < B_c; ++b) {
                    if (map[b] != u) continue;
                    for (int64_t k = 0; k < K_u; ++k) {
                        double *x = dX + k * D;
                        for (int64_t d = 0; d < D; ++d) x[d] = 0.0;
                        for (int64_t m = 0; m < M; ++m) {
                            const double w = W[m * K + k];
                            for (int64_t d = 0; d < D; ++d) x[d] += w * widen(dY, (b * M + m) * D + d, dtype);
                        }
                        double *acc = dU + (u * K_u + k) * D;
                        for (int64_t d = 0; d < D; ++d) acc[d] += x[d];
                    }
                }
            }
        }
        free(dX);
    }

    /* dW[m][k] = sum over b (ascending), then d (ascending), of dY[b][m][d] * X_b[k][d]. */
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t m = 0; m < M; ++m) {
        for (int64_t k = 0; k < K; ++k) {
            double acc = 0.0;
            for (int64_t b = 0; b < B_c; ++b) {
                for (int64_t d = 0; d < D; ++d) {
                    const double x = k < K_u ? widen(U, ((int64_t)map[b] * K_u + k) * D + d, dtype)
                                             : widen(C, (b * K_c + (k - K_u)) * D + d, dtype);
                    acc += widen(dY, (b * M + m) * D + d, dtype) * x;
                }
            }
            if (k < K_u) dW_u[m * K_u + k] = acc;
            else dW_c[m * K_c + (k - K_u)] = acc;
        }
    }
    free(W);
    return status;
}

/* Number of threads an OpenMP parallel region would use (1 without OpenMP). */
int ikbo_oracle_max_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}
