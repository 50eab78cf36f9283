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
#include <math.h>
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
 *     dU[u]  = sum over b with map[b] = u of rows 0..K_u-1 of dX_b
 *                                                (the adjoint of the replication is a
 *                                                 scatter-add; users with no candidate
 *                                                 get zero)
 *     dW     = sum_b dY[b] . X_b^T               [M, K_u + K_c] = [dW_u | dW_c]
 *
 * Only the requested outputs are computed, so that large batches can be checked on a
 * sample: dC rows (b, k) and dU rows (u, k) give D values each, dW elements (m, kk)
 * with kk < K_u in dW_u and kk >= K_u in dW_c (column kk - K_u) give one value each.
 * Orders (independent of the thread count): a row of dX_b sums over m ascending; a dU
 * row adds the candidates of its user in ascending b; a dW element sums over b
 * ascending, then d ascending.
 */
int ikbo_oracle_lce_backward_f64(const void *dY, const void *U, const void *C, const int32_t *map,
                                 const void *W_u, const void *W_c, int64_t B_u, int64_t B_c, int64_t K_u,
                                 int64_t K_c, int64_t M, int64_t D, int dtype,
                                 const int64_t *dc_rows, int64_t n_dc, double *dC,
                                 const int64_t *du_rows, int64_t n_du, double *dU,
                                 const int64_t *dw_elems, int64_t n_dw, double *dW, int nthreads)
{
    if (!dY || !U || !C || !map || !W_u || !W_c) return ORACLE_ERR_ARG;
    if ((n_dc && (!dc_rows || !dC)) || (n_du && (!du_rows || !dU)) || (n_dw && (!dw_elems || !dW)))
        return ORACLE_ERR_ARG;
    if (B_u < 1 || B_c < 0 || K_u < 0 || K_c < 0 || M < 1 || D < 1) return ORACLE_ERR_ARG;
    if (dtype != ORACLE_BF16 && dtype != ORACLE_F32) return ORACLE_ERR_ARG;
    for (int64_t b = 0; b < B_c; ++b)
        if (map[b] < 0 || map[b] >= B_u) return ORACLE_ERR_MAP;
    const int64_t K = K_u + K_c;
    for (int64_t i = 0; i < n_dc; ++i)
        if (dc_rows[2 * i] < 0 || dc_rows[2 * i] >= B_c || dc_rows[2 * i + 1] < 0 || dc_rows[2 * i + 1] >= K_c)
            return ORACLE_ERR_ARG;
    for (int64_t i = 0; i < n_du; ++i)
        if (du_rows[2 * i] < 0 || du_rows[2 * i] >= B_u || du_rows[2 * i + 1] < 0 || du_rows[2 * i + 1] >= K_u)
            return ORACLE_ERR_ARG;
    for (int64_t i = 0; i < n_dw; ++i)
        if (dw_elems[2 * i] < 0 || dw_elems[2 * i] >= M || dw_elems[2 * i + 1] < 0 || dw_elems[2 * i + 1] >= K)
            return ORACLE_ERR_ARG;

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

    /* dC rows: row K_u + k of dX_b. */
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t i = 0; i < n_dc; ++i) {
        const int64_t b = dc_rows[2 * i], k = K_u + dc_rows[2 * i + 1];
        double *out = dC + i * D;
        for (int64_t d = 0; d < D; ++d) out[d] = 0.0;
        for (int64_t m = 0; m < M; ++m) {
            const double w = W[m * K + k];
            for (int64_t d = 0; d < D; ++d) out[d] += w * widen(dY, (b * M + m) * D + d, dtype);
        }
    }

    /* dU rows: row k of dX_b, added over the user's candidates in ascending b. */
#pragma omp parallel
    {
        double *x = (double *)malloc(sizeof(double) * (size_t)D);
        if (!x) {
#pragma omp atomic write
            status = ORACLE_ERR_NOMEM;
        } else {
#pragma omp for schedule(dynamic, 1)
            for (int64_t i = 0; i < n_du; ++i) {
                const int64_t u = du_rows[2 * i], k = du_rows[2 * i + 1];
                double *acc = dU + i * D;
                for (int64_t d = 0; d < D; ++d) acc[d] = 0.0;
                for (int64_t b = 0; b < B_c; ++b) {
                    if (map[b] != u) continue;
                    for (int64_t d = 0; d < D; ++d) x[d] = 0.0;
                    for (int64_t m = 0; m < M; ++m) {
                        const double w = W[m * K + k];
                        for (int64_t d = 0; d < D; ++d) x[d] += w * widen(dY, (b * M + m) * D + d, dtype);
                    }
                    for (int64_t d = 0; d < D; ++d) acc[d] += x[d];
                }
            }
        }
        free(x);
    }

    /* dW[m][kk] = sum over b (ascending), then d (ascending), of dY[b][m][d] * X_b[kk][d]. */
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t i = 0; i < n_dw; ++i) {
        const int64_t m = dw_elems[2 * i], k = dw_elems[2 * i + 1];
        double acc = 0.0;
        for (int64_t b = 0; b < B_c; ++b) {
            for (int64_t d = 0; d < D; ++d) {
                const double x = k < K_u ? widen(U, ((int64_t)map[b] * K_u + k) * D + d, dtype)
                                         : widen(C, (b * K_c + (k - K_u)) * D + d, dtype);
                acc += widen(dY, (b * M + m) * D + d, dtype) * x;
            }
        }
        dW[i] = acc;
    }
    free(W);
    return status;
}

/*
 * IKBO target attention (IKBO recsys blog, "Deep Dive: Flash Attention"): the queries of
 * candidate b attend over the keys and values of its user u = map[b], head by head:
 *
 *     K_b = K[map[b]], V_b = V[map[b]]           (the broadcast, materialised here)
 *     s_k = scale * sum_d Q[b,h,q,d] K_b[h,k,d]
 *     O[b,h,q,:] = sum_k softmax(s)_k V_b[h,k,:]
 *
 * Layouts: Q, O [B_c][H][L_q][hd]; K, V [B_u][H][L_kv][hd].  Requested output rows are
 * (b, h, q) triples; each gives hd values.  Per row: the materialised K_b and V_b rows of
 * head h are copied into a buffer, scores summed over d ascending, the maximum score
 * subtracted before exp (the value is the same; it only keeps exp finite), the weights and
 * the weighted sum of V taken over k ascending, then divided by the sum of weights.
 */
int ikbo_oracle_fa_f64(const void *Q, const void *K, const void *V, const int32_t *map, int64_t B_u,
                       int64_t B_c, int64_t H, int64_t L_q, int64_t L_kv, int64_t hd, double scale,
                       int dtype, const int64_t *rows, int64_t n_rows, double *O, int nthreads)
{
    if (!Q || !K || !V || !map || !O || (n_rows && !rows)) return ORACLE_ERR_ARG;
    if (B_u < 1 || B_c < 0 || H < 1 || L_q < 1 || L_kv < 1 || hd < 1) return ORACLE_ERR_ARG;
    if (dtype != ORACLE_BF16 && dtype != ORACLE_F32) return ORACLE_ERR_ARG;
    for (int64_t b = 0; b < B_c; ++b)
        if (map[b] < 0 || map[b] >= B_u) return ORACLE_ERR_MAP;
    for (int64_t i = 0; i < n_rows; ++i)
        if (rows[3 * i] < 0 || rows[3 * i] >= B_c || rows[3 * i + 1] < 0 || rows[3 * i + 1] >= H ||
            rows[3 * i + 2] < 0 || rows[3 * i + 2] >= L_q)
            return ORACLE_ERR_ARG;
#ifdef _OPENMP
    if (nthreads > 0) omp_set_num_threads(nthreads);
#else
    (void)nthreads;
#endif
    int status = ORACLE_OK;
#pragma omp parallel
    {
        double *Kb = (double *)malloc(sizeof(double) * (size_t)(L_kv * hd));
        double *Vb = (double *)malloc(sizeof(double) * (size_t)(L_kv * hd));
        double *sc = (double *)malloc(sizeof(double) * (size_t)L_kv);
        double *qv = (double *)malloc(sizeof(double) * (size_t)hd);
        if (!Kb || !Vb || !sc || !qv) {
#pragma omp atomic write
            status = ORACLE_ERR_NOMEM;
        } else {
#pragma omp for schedule(dynamic, 4)
            for (int64_t i = 0; i < n_rows; ++i) {
                const int64_t b = rows[3 * i], h = rows[3 * i + 1], q = rows[3 * i + 2];
                const int64_t u = map[b];
                for (int64_t k = 0; k < L_kv; ++k)
                    for (int64_t d = 0; d < hd; ++d) {
                        Kb[k * hd + d] = widen(K, ((u * H + h) * L_kv + k) * hd + d, dtype);
                        Vb[k * hd + d] = widen(V, ((u * H + h) * L_kv + k) * hd + d, dtype);
                    }
                for (int64_t d = 0; d < hd; ++d) qv[d] = widen(Q, ((b * H + h) * L_q + q) * hd + d, dtype);
                double mx = -INFINITY;
                for (int64_t k = 0; k < L_kv; ++k) {
                    double t = 0.0;
                    for (int64_t d = 0; d < hd; ++d) t += qv[d] * Kb[k * hd + d];
                    sc[k] = scale * t;
                    if (sc[k] > mx) mx = sc[k];
                }
                double l = 0.0;
                for (int64_t k = 0; k < L_kv; ++k) {
                    sc[k] = exp(sc[k] - mx);
                    l += sc[k];
                }
                double *out = O + i * hd;
                for (int64_t d = 0; d < hd; ++d) out[d] = 0.0;
                for (int64_t k = 0; k < L_kv; ++k)
                    for (int64_t d = 0; d < hd; ++d) out[d] += sc[k] * Vb[k * hd + d];
                for (int64_t d = 0; d < hd; ++d) out[d] /= l;
            }
        }
        free(Kb);
        free(Vb);
        free(sc);
        free(qv);
    }
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
