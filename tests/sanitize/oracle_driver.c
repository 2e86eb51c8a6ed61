/*
 * Sanitizer driver for the CPU oracle (built with -fsanitize=address,undefined
 * by tests/test_sanitize.py; test infrastructure only).  Runs every exported
 * oracle function on small problems -- ragged and empty experts, M = 0,
 * explicit index lists, invalid offsets and indices -- so that an
 * out-of-bounds access or undefined behaviour in the oracle is reported.
 * Prints "ok" and returns 0 when every call returned what it should.
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

int oracle_threads(void);
int oracle_fwd(const uint16_t *X, const uint16_t *W, const int32_t *offs, int32_t E, int64_t M, int64_t N,
               int64_t K, const int64_t *idx, int64_t count, double *out, double *q);
int oracle_dgrad(const uint16_t *G, const uint16_t *W, const int32_t *offs, int32_t E, int64_t M, int64_t N,
                 int64_t K, const int64_t *idx, int64_t count, double *out, double *q);
int oracle_wgrad(const uint16_t *X, const uint16_t *G, const int32_t *offs, int32_t E, int64_t M, int64_t N,
                 int64_t K, const int64_t *idx, int64_t count, double *out, double *q);
void oracle_round_f32(const double *in, float *out, int64_t n);
void oracle_round_bf16(const double *in, uint16_t *out, int64_t n);
int oracle_router_exact(const float *X, const float *Wr, int64_t M, int64_t N, int64_t K, const int64_t *idx,
                        int64_t count, double *out);
int oracle_router_bf16x3(const float *X, const float *Wr, int64_t M, int64_t N, int64_t K, const int64_t *idx,
                         int64_t count, double *out);

static int fails = 0;
#define CHECK(c)                                                  \
    do {                                                          \
        if (!(c)) {                                               \
            fprintf(stderr, "check failed line %d: %s\n", __LINE__, #c); \
            ++fails;                                              \
        }                                                         \
    } while (0)

/* small integers as BF16 bit patterns (exact) */
static uint16_t bf16_of_int(int v) {
    float f = (float)v;
    uint32_t u;
    memcpy(&u, &f, sizeof u);
    return (uint16_t)(u >> 16);
}

static uint16_t *rand_bf16(int64_t n, unsigned *seed) {
    uint16_t *a = malloc((size_t)(n > 0 ? n : 1) * sizeof *a);
    for (int64_t i = 0; i < n; ++i) a[i] = bf16_of_int((int)(rand_r(seed) % 9) - 4);
    return a;
}

int main(void) {
    unsigned seed = 7;
    CHECK(oracle_threads() >= 1);
    const int32_t E = 4;
    const int64_t M = 37, N = 24, K = 16;
    const int32_t offs[5] = {0, 10, 10, 31, 37};     /* expert 1 empty */
    uint16_t *X = rand_bf16(M * K, &seed), *W = rand_bf16(E * N * K, &seed), *G = rand_bf16(M * N, &seed);
    double *out = malloc(sizeof(double) * (size_t)(E * N * K)), *q = malloc(sizeof(double) * (size_t)(E * N * K));
    CHECK(oracle_fwd(X, W, offs, E, M, N, K, NULL, M * N, out, q) == 0);
    CHECK(oracle_dgrad(G, W, offs, E, M, N, K, NULL, M * K, out, q) == 0);
    CHECK(oracle_wgrad(X, G, offs, E, M, N, K, NULL, E * N * K, out, q) == 0);
    for (int64_t i = 0; i < N * K; ++i) CHECK(out[N * K + i] == 0.0 && !signbit(out[N * K + i]));
    /* explicit index lists: first, last, and a few in between */
    int64_t idx[4] = {0, 5, M * N - 1, 100};
    CHECK(oracle_fwd(X, W, offs, E, M, N, K, idx, 4, out, q) == 0);
    int64_t widx[3] = {0, E * N * K - 1, N * K + 3};
    CHECK(oracle_wgrad(X, G, offs, E, M, N, K, widx, 3, out, q) == 0);
    /* out-of-range indices and invalid offsets are refused, not read */
    int64_t bad_idx[1] = {M * N};
    CHECK(oracle_fwd(X, W, offs, E, M, N, K, bad_idx, 1, out, q) != 0);
    const int32_t bad_offs[5] = {0, 12, 10, 31, 37};
    CHECK(oracle_dgrad(G, W, bad_offs, E, M, N, K, NULL, M * K, out, q) != 0);
    const int32_t short_offs[5] = {0, 10, 10, 31, 36};
    CHECK(oracle_wgrad(X, G, short_offs, E, M, N, K, NULL, E * N * K, out, q) != 0);
    /* no tokens */
    const int32_t zero_offs[5] = {0, 0, 0, 0, 0};
    CHECK(oracle_fwd(X, W, zero_offs, E, 0, N, K, NULL, 0, out, q) == 0);
    CHECK(oracle_wgrad(X, G, zero_offs, E, 0, N, K, NULL, E * N * K, out, q) == 0);
    for (int64_t i = 0; i < E * N * K; ++i) CHECK(out[i] == 0.0);
    /* rounding, including specials */
    double vals[6] = {1.0, -0.0, 1e-45, 3.4e38 * 2, NAN, 1.00390625};
    float f[6];
    uint16_t b[6];
    oracle_round_f32(vals, f, 6);
    oracle_round_bf16(vals, b, 6);
    CHECK(f[0] == 1.0f && b[0] == 0x3F80);
    /* router, both oracles */
    const int64_t RM = 9, RN = 8, RK = 24;
    float *Xr = malloc(sizeof(float) * (size_t)(RM * RK)), *Wr = malloc(sizeof(float) * (size_t)(RN * RK));
    for (int64_t i = 0; i < RM * RK; ++i) Xr[i] = (float)rand_r(&seed) / (float)RAND_MAX - 0.5f;
    for (int64_t i = 0; i < RN * RK; ++i) Wr[i] = (float)rand_r(&seed) / (float)RAND_MAX - 0.5f;
    double *ro = malloc(sizeof(double) * (size_t)(RM * RN)), *re = malloc(sizeof(double) * (size_t)(RM * RN));
    CHECK(oracle_router_exact(Xr, Wr, RM, RN, RK, NULL, RM * RN, re) == 0);
    CHECK(oracle_router_bf16x3(Xr, Wr, RM, RN, RK, NULL, RM * RN, ro) == 0);
    for (int64_t i = 0; i < RM * RN; ++i) CHECK(fabs(ro[i] - re[i]) <= 1e-3 * (1.0 + fabs(re[i])));
    int64_t rbad[1] = {-1};
    CHECK(oracle_router_exact(Xr, Wr, RM, RN, RK, rbad, 1, re) != 0);
    free(X); free(W); free(G); free(out); free(q); free(Xr); free(Wr); free(ro); free(re);
    if (fails) return 1;
    printf("ok\n");
    return 0;
}
