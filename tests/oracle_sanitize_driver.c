/* Runs every oracle entry point on small shapes with exact-size heap buffers, for a
 * build with -fsanitize=address,undefined: an out-of-bounds access or undefined
 * behaviour anywhere in the oracle stops the program with a report.  Also checks a few
 * results that must hold (a sampled row equals the full result's row; a single key gives
 * O = V).  Exit status 0 when everything ran and held. */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

int ikbo_oracle_lce_f64(const void *U, const void *C, const int32_t *map, const void *W_u, const void *W_c,
                        double *Y, int64_t B_u, int64_t B_c, int64_t K_u, int64_t K_c, int64_t M, int64_t D,
                        int dtype, const int64_t *rows, int64_t n_rows, int nthreads);
int ikbo_oracle_lce_backward_f64(const void *dY, const void *U, const void *C, const int32_t *map,
                                 const void *W_u, const void *W_c, int64_t B_u, int64_t B_c, int64_t K_u,
                                 int64_t K_c, int64_t M, int64_t D, int dtype, const int64_t *dc_rows, int64_t n_dc,
                                 double *dC, const int64_t *du_rows, int64_t n_du, double *dU,
                                 const int64_t *dw_elems, int64_t n_dw, double *dW, int nthreads);
int ikbo_oracle_fa_f64(const void *Q, const void *K, const void *V, const int32_t *map, int64_t B_u, int64_t B_c,
                       int64_t H, int64_t L_q, int64_t L_kv, int64_t hd, double scale, int dtype,
                       const int64_t *rows, int64_t n_rows, double *O, int nthreads);

static uint32_t rng_state = 12345u;
static uint32_t next_u32(void) {   /* xorshift32 */
    rng_state ^= rng_state << 13;
    rng_state ^= rng_state >> 17;
    rng_state ^= rng_state << 5;
    return rng_state;
}
/* n values of element type dtype (0: bf16 bit patterns of small numbers, 1: float32). */
static void *values(int64_t n, int dtype) {
    const size_t esz = dtype == 0 ? 2 : 4;
    void *p = malloc((size_t)(n > 0 ? n : 1) * esz);
    for (int64_t i = 0; i < n; ++i) {
        const float f = (float)((int)(next_u32() % 17u) - 8) / 8.0f;
        if (dtype == 0) {
            uint32_t bits;
            memcpy(&bits, &f, 4);
            ((uint16_t *)p)[i] = (uint16_t)(bits >> 16);   /* exact: f has few mantissa bits */
        } else {
            ((float *)p)[i] = f;
        }
    }
    return p;
}
static int32_t *a_map(int64_t B_c, int64_t B_u) {
    int32_t *m = malloc((size_t)(B_c > 0 ? B_c : 1) * sizeof(int32_t));
    for (int64_t b = 0; b < B_c; ++b) m[b] = (int32_t)(next_u32() % (uint32_t)B_u);
    return m;
}

static int fails = 0;
#define EXPECT(c)                                                           \
    do {                                                                    \
        if (!(c)) {                                                         \
            fprintf(stderr, "%s:%d: expectation failed: %s\n", __FILE__, __LINE__, #c); \
            ++fails;                                                        \
        }                                                                   \
    } while (0)

static void lce_case(int64_t B_u, int64_t B_c, int64_t K_u, int64_t K_c, int64_t M, int64_t D, int dtype) {
    void *U = values(B_u * K_u * D, dtype), *C = values(B_c * K_c * D, dtype);
    void *W_u = values(M * K_u, dtype), *W_c = values(M * K_c, dtype), *dY = values(B_c * M * D, dtype);
    int32_t *map = a_map(B_c, B_u);
    double *Y = malloc((size_t)(B_c * M * D) * sizeof(double));
    EXPECT(ikbo_oracle_lce_f64(U, C, map, W_u, W_c, Y, B_u, B_c, K_u, K_c, M, D, dtype, NULL, 0, 1) == 0);
    const int64_t rows[2] = {B_c - 1, 0};
    double *Yr = malloc((size_t)(2 * M * D) * sizeof(double));
    EXPECT(ikbo_oracle_lce_f64(U, C, map, W_u, W_c, Yr, B_u, B_c, K_u, K_c, M, D, dtype, rows, 2, 1) == 0);
    EXPECT(memcmp(Yr, Y + (B_c - 1) * M * D, (size_t)(M * D) * sizeof(double)) == 0);
    EXPECT(memcmp(Yr + M * D, Y, (size_t)(M * D) * sizeof(double)) == 0);
    /* backward: every dC row, every dU row, every dW element */
    const int64_t n_dc = B_c * K_c, n_du = B_u * K_u, n_dw = M * (K_u + K_c);
    int64_t *dc_rows = malloc((size_t)(2 * (n_dc > 0 ? n_dc : 1)) * sizeof(int64_t));
    int64_t *du_rows = malloc((size_t)(2 * n_du) * sizeof(int64_t));
    int64_t *dw_el = malloc((size_t)(2 * n_dw) * sizeof(int64_t));
    for (int64_t i = 0; i < n_dc; ++i) { dc_rows[2 * i] = i / K_c; dc_rows[2 * i + 1] = i % K_c; }
    for (int64_t i = 0; i < n_du; ++i) { du_rows[2 * i] = i / K_u; du_rows[2 * i + 1] = i % K_u; }
    for (int64_t i = 0; i < n_dw; ++i) { dw_el[2 * i] = i / (K_u + K_c); dw_el[2 * i + 1] = i % (K_u + K_c); }
    double *dC = malloc((size_t)((n_dc > 0 ? n_dc : 1) * D) * sizeof(double));
    double *dU = malloc((size_t)(n_du * D) * sizeof(double));
    double *dW = malloc((size_t)n_dw * sizeof(double));
    EXPECT(ikbo_oracle_lce_backward_f64(dY, U, C, map, W_u, W_c, B_u, B_c, K_u, K_c, M, D, dtype, dc_rows, n_dc,
                                        dC, du_rows, n_du, dU, dw_el, n_dw, dW, 1) == 0);
    for (int64_t i = 0; i < n_dw; ++i) EXPECT(isfinite(dW[i]));
    /* an out-of-range map entry is refused */
    if (B_c > 0) {
        map[0] = (int32_t)B_u;
        EXPECT(ikbo_oracle_lce_f64(U, C, map, W_u, W_c, Y, B_u, B_c, K_u, K_c, M, D, dtype, NULL, 0, 1) != 0);
    }
    free(U); free(C); free(W_u); free(W_c); free(dY); free(map); free(Y); free(Yr);
    free(dc_rows); free(du_rows); free(dw_el); free(dC); free(dU); free(dW);
}

static void fa_case(int64_t B_u, int64_t B_c, int64_t H, int64_t L_q, int64_t L_kv, int64_t hd, int dtype) {
    void *Q = values(B_c * H * L_q * hd, dtype), *K = values(B_u * H * L_kv * hd, dtype);
    void *V = values(B_u * H * L_kv * hd, dtype);
    int32_t *map = a_map(B_c, B_u);
    const int64_t n_all = B_c * H * L_q;   /* every query row, (b, h, q) in order */
    int64_t *all = malloc((size_t)(3 * n_all) * sizeof(int64_t));
    for (int64_t i = 0; i < n_all; ++i) {
        all[3 * i] = i / (H * L_q);
        all[3 * i + 1] = (i / L_q) % H;
        all[3 * i + 2] = i % L_q;
    }
    double *O = malloc((size_t)(n_all * hd) * sizeof(double));
    EXPECT(ikbo_oracle_fa_f64(Q, K, V, map, B_u, B_c, H, L_q, L_kv, hd, 1.0 / sqrt((double)hd), dtype, all, n_all, O,
                              1) == 0);
    if (L_kv == 1)   /* a single key: every output row is that key's V row */
        for (int64_t i = 0; i < n_all; ++i) {
            const int64_t u = map[all[3 * i]], h = all[3 * i + 1];
            for (int64_t d = 0; d < hd; ++d) {
                const int64_t e = (u * H + h) * hd + d;
                double v;
                if (dtype == 0) {
                    const uint32_t bits = (uint32_t)((const uint16_t *)V)[e] << 16;
                    float f;
                    memcpy(&f, &bits, 4);
                    v = f;
                } else {
                    v = ((const float *)V)[e];
                }
                EXPECT(O[i * hd + d] == v);
            }
        }
    const int64_t rows[3] = {B_c - 1, H - 1, L_q - 1};
    double *Or = malloc((size_t)hd * sizeof(double));
    EXPECT(ikbo_oracle_fa_f64(Q, K, V, map, B_u, B_c, H, L_q, L_kv, hd, 1.0 / sqrt((double)hd), dtype, rows, 1, Or,
                              1) == 0);
    EXPECT(memcmp(Or, O + (((B_c - 1) * H + H - 1) * L_q + L_q - 1) * hd, (size_t)hd * sizeof(double)) == 0);
    free(Q); free(K); free(V); free(map); free(O); free(Or); free(all);
}

int main(void) {
    for (int dtype = 0; dtype < 2; ++dtype) {
        lce_case(1, 1, 1, 1, 1, 1, dtype);
        lce_case(2, 5, 3, 2, 3, 4, dtype);
        lce_case(3, 7, 13, 11, 17, 8, dtype);
        lce_case(2, 4, 5, 0, 3, 2, dtype);   /* no candidate features */
        fa_case(1, 1, 1, 1, 1, 1, dtype);
        fa_case(2, 5, 2, 3, 7, 4, dtype);
    }
    if (fails) fprintf(stderr, "%d expectations failed\n", fails);
    else printf("oracle sanitizer run: ok\n");
    return fails ? 1 : 0;
}
