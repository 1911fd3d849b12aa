/* Runs every oracle entry point on small inputs, for a build of the oracle with the
 * address and undefined-behaviour sanitizers (tests/test_oracle_sanitize.py compiles
 * this file together with oracle/tcq_oracle.c with gcc).  Any out-of-bounds access,
 * leak or undefined operation aborts the run; a clean run prints "oracle sanitize ok". */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

double oracle_inv_normal_cdf(double p);
uint64_t oracle_splitmix64_next(uint64_t *state);
int oracle_make_codebook(int L, int V, uint64_t seed, float *out);
void oracle_decode_block(const uint32_t *bits, uint32_t s0, const float *C, int L, int k,
                         int V, int T, float *out);
float oracle_path_cost(const float *w, const float *d, const float *C, int L, int k, int V,
                       int T, const uint32_t *bits, uint32_t s0);
int oracle_encode_block(const float *w, const float *d, const float *C, int L, int k, int V,
                        int T, int fixed_s0, uint32_t *bits, uint32_t *s0_out,
                        float *cost_out);
int oracle_two_best_block(const float *w, const float *d, const float *C, int L, int k,
                          int V, int T, int fixed_s0, float *best_out, float *second_out);
int oracle_ldlq_row(const float *w, const float *U, long ldu, const float *d, const float *C,
                    int L, int k, int V, int T, long N, uint32_t *bits, uint32_t *s0_out,
                    float *cost_out, float *what, float *target);
int oracle_bcjr_block(const double *w, const double *d, const float *C, int L, int k, int V,
                      int T, double tau, double *soft_out, double *logz_out);
int oracle_hadamard_row(const double *x, long len, long n, const double *sigma, int inverse,
                        double *y);
int oracle_scale_field(const float *W, long M, long N, long ldw, double *a, double *b,
                       double *Wn);

static uint64_t rng = 12345;
static double unif(void) { return (double)(oracle_splitmix64_next(&rng) >> 11) * 0x1.0p-53; }
static double gauss(void) { return oracle_inv_normal_cdf(0.001 + 0.998 * unif()); }

#define CHECK(c)                                                       \
    do {                                                               \
        if (!(c)) {                                                    \
            fprintf(stderr, "check failed at line %d: %s\n", __LINE__, #c); \
            return 1;                                                  \
        }                                                              \
    } while (0)

/* encode, decode and recompute the cost of one block of each shape */
static int one_shape(int L, int k, int V, int T, int weighted) {
    const int rows = 1 << L;
    float *C = malloc(sizeof(float) * rows * V);
    float *w = malloc(sizeof(float) * T), *d = malloc(sizeof(float) * T);
    float *rec = malloc(sizeof(float) * T);
    const int nw = (k * T + 31) / 32;
    uint32_t *bits = calloc((size_t)nw, sizeof(uint32_t));
    CHECK(C && w && d && rec && bits);
    CHECK(oracle_make_codebook(L, V, 7, C) == 0);
    for (int i = 0; i < T; ++i) {
        w[i] = (float)gauss();
        d[i] = (float)(0.5 + unif());
    }
    for (int fixed = -1; fixed <= 0; ++fixed) {
        uint32_t s0 = 0;
        float cost = 0.0f, best = 0.0f, second = 0.0f;
        CHECK(oracle_encode_block(w, weighted ? d : NULL, C, L, k, V, T, fixed, bits, &s0,
                                  &cost) == 0);
        oracle_decode_block(bits, s0, C, L, k, V, T, rec);
        CHECK(oracle_path_cost(w, weighted ? d : NULL, C, L, k, V, T, bits, s0) == cost);
        CHECK(oracle_two_best_block(w, weighted ? d : NULL, C, L, k, V, T, fixed, &best,
                                    &second) == 0);
        CHECK(best == cost && second >= best);
    }
    free(C); free(w); free(d); free(rec); free(bits);
    return 0;
}

int main(void) {
    CHECK(one_shape(6, 2, 1, 12, 0) == 0);
    CHECK(one_shape(6, 2, 1, 12, 1) == 0);
    CHECK(one_shape(8, 1, 2, 10, 1) == 0);
    CHECK(one_shape(5, 3, 1, 9, 1) == 0);
    CHECK(one_shape(4, 4, 1, 3, 0) == 0);  /* kV = L: every state reachable in one step */

    /* error feedback over a row of 3 blocks */
    {
        const int L = 6, k = 2, V = 1, T = 8;
        const long N = 24;
        float *C = malloc(sizeof(float) << L), *w = malloc(sizeof(float) * N);
        float *U = calloc((size_t)(N * N), sizeof(float)), *d = malloc(sizeof(float) * N);
        float *what = malloc(sizeof(float) * N), *target = malloc(sizeof(float) * N);
        float cost[3];
        uint32_t bits[3], s0[3];
        CHECK(C && w && U && d && what && target);
        CHECK(oracle_make_codebook(L, V, 9, C) == 0);
        for (long i = 0; i < N; ++i) {
            w[i] = (float)gauss();
            d[i] = (float)(0.5 + unif());
            U[i * N + i] = 1.0f;
            for (long c = i + 1; c < N; ++c) U[i * N + c] = (float)(0.1 * gauss());
        }
        CHECK(oracle_ldlq_row(w, U, N, d, C, L, k, V, T, N, bits, s0, cost, what, target) == 0);
        free(C); free(w); free(U); free(d); free(what); free(target);
    }

    /* soft trellis */
    {
        const int L = 6, k = 2, V = 1, T = 8;
        float *C = malloc(sizeof(float) << L);
        double w[8], d[8], soft[8], logz = 0.0;
        CHECK(C);
        CHECK(oracle_make_codebook(L, V, 11, C) == 0);
        for (int i = 0; i < T; ++i) {
            w[i] = gauss();
            d[i] = 0.5 + unif();
        }
        CHECK(oracle_bcjr_block(w, d, C, L, k, V, T, 0.5, soft, &logz) == 0);
        CHECK(isfinite(logz));
        free(C);
    }

    /* pre-processing */
    {
        double x[32], sg[32], y[32], z[32];
        for (int i = 0; i < 32; ++i) {
            x[i] = gauss();
            sg[i] = (oracle_splitmix64_next(&rng) & 1) ? 1.0 : -1.0;
        }
        CHECK(oracle_hadamard_row(x, 32, 16, sg, 0, y) == 0);
        CHECK(oracle_hadamard_row(y, 32, 16, sg, 1, z) == 0);
        for (int i = 0; i < 32; ++i) CHECK(fabs(z[i] - x[i]) < 1e-12);
        const long M = 5, N = 7, ldw = 9;
        float W[45];
        double a[5], b[7], Wn[35];
        for (int i = 0; i < 45; ++i) W[i] = (float)gauss();
        for (int c = 0; c < N; ++c) W[2 * ldw + c] = 0.0f; /* an all-zero row */
        CHECK(oracle_scale_field(W, M, N, ldw, a, b, Wn) == 0);
        CHECK(a[2] == 1.0);
    }
    printf("oracle sanitize ok\n");
    return 0;
}
