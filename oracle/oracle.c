/*
 * oracle.c -- the CPU oracle for the ragged BF16 grouped GEMM.
 *
 * TEST INFRASTRUCTURE ONLY.  This file is the plain, slow, obviously correct
 * definition that the GPU kernels are checked against.  Only the test suite,
 * the smoke check and the CPU-baseline leg of the benchmark may load it; the
 * product library never links, loads or calls it, and it shares no code,
 * header or table with the product.
 *
 * What it computes (flashinfer PR #8258, "run the split k512 wgrad tail whole
 * on the least-loaded clusters on sm_107a", opening summary paragraph):
 * experts own contiguous token ranges; every program accumulates exactly
 * and rounds once.
 *
 *   forward          y[t,n]   = sum_k  x[t,k] * w[e(t),n,k]
 *   data gradient    dx[t,k]  = sum_n  g[t,n] * w[e(t),n,k]
 *   weight gradient  dw[e,n,k]= sum_{t in expert e} g[t,n] * x[t,k]
 *
 * with e(t) the expert whose token range holds t.  Token ranges come from
 * group offsets o[0..E] (o[0] = 0, non-decreasing, o[E] = M); expert e owns
 * tokens o[e] .. o[e+1]-1.  An expert with no tokens has dw[e] = +0.
 * The dense projection GEMM of flashinfer PR #8363 ("run the deterministic
 * program at the sm_107a token counts its new plans win", Summary) is the
 * E = 1 case.
 *
 * Precision: the inputs are BF16, so each product of two inputs is exact in
 * binary64; the sums run in binary64 in increasing reduction index.  The
 * result is returned unrounded (double) together with
 *   q = sqrt(sum of squared products),
 * the scale that the BF16 tolerance floor uses.  Separate functions round a
 * double once to FP32 or to BF16 (round to nearest, ties to even, straight
 * from the double so there is no double rounding).
 *
 * The FP32 router GEMM (PR #8363, Summary: 256 experts, FP32 emulated with
 * three BF16 products) has two oracles here: the exact FP32 x FP32
 * product summed in binary64, and the BF16x3 emulation written out step by
 * step: hi = bf16(x), lo = bf16(x - hi) for both operands, and the sum of
 * hi*hi + hi*lo + lo*hi (the lo*lo term is dropped), in binary64.
 *
 * Build: plain C99, no -ffast-math, -ffp-contract=off.  OpenMP only splits
 * the list of requested output elements across threads; each element is
 * computed by one thread in one fixed order, so the result does not depend
 * on the thread count.
 */
#include <math.h>
#include <stdint.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

enum { OR_OK = 0, OR_BAD_OFFSETS = 1, OR_BAD_INDEX = 2, OR_BAD_SHAPE = 3 };

int oracle_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/* A BF16 value is the high half of an IEEE binary32; widening is exact. */
static double bf16_value(uint16_t bits)
{
    uint32_t u = (uint32_t)bits << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

/* Offsets must start at 0, never decrease and end at M. */
static int offsets_ok(const int32_t *o, int32_t E, int64_t M)
{
    if (E < 1 || o[0] != 0 || (int64_t)o[E] != M)
        return 0;
    for (int32_t e = 0; e < E; ++e)
        if (o[e + 1] < o[e])
            return 0;
    return 1;
}

/* The expert whose token range [o[e], o[e+1]) holds token t. */
static int32_t expert_of(const int32_t *o, int32_t E, int64_t t)
{
    for (int32_t e = 0; e < E; ++e)
        if (t < (int64_t)o[e + 1])
            return e;
    return -1;
}

/* ---- the three programs, one output element at a time ------------------ */

static void fwd_element(const uint16_t *X, const uint16_t *W, const int32_t *o,
                        int32_t E, int64_t N, int64_t K, int64_t t, int64_t n,
                        double *val, double *q)
{
    int32_t e = expert_of(o, E, t);
    const uint16_t *x = X + t * K;
    const uint16_t *w = W + ((int64_t)e * N + n) * K;
    double s = 0.0, ss = 0.0;
    for (int64_t k = 0; k < K; ++k) {
        double p = bf16_value(x[k]) * bf16_value(w[k]);
        s += p;
        ss += p * p;
    }
    *val = s;
    *q = sqrt(ss);
}

static void dgrad_element(const uint16_t *G, const uint16_t *W, const int32_t *o,
                          int32_t E, int64_t N, int64_t K, int64_t t, int64_t k,
                          double *val, double *q)
{
    int32_t e = expert_of(o, E, t);
    const uint16_t *g = G + t * N;
    const uint16_t *w = W + (int64_t)e * N * K;
    double s = 0.0, ss = 0.0;
    for (int64_t n = 0; n < N; ++n) {
        double p = bf16_value(g[n]) * bf16_value(w[n * K + k]);
        s += p;
        ss += p * p;
    }
    *val = s;
    *q = sqrt(ss);
}

static void wgrad_element(const uint16_t *X, const uint16_t *G, const int32_t *o,
                          int64_t N, int64_t K, int32_t e, int64_t n, int64_t k,
                          double *val, double *q)
{
    double s = 0.0, ss = 0.0;
    for (int64_t t = o[e]; t < (int64_t)o[e + 1]; ++t) {
        double p = bf16_value(G[t * N + n]) * bf16_value(X[t * K + k]);
        s += p;
        ss += p * p;
    }
    /* no tokens: the sum is empty and the result is +0 */
    *val = s;
    *q = sqrt(ss);
}

/*
 * Each entry point evaluates the output elements whose flat row-major
 * indices are listed in idx[0..count-1] (all of them, in order, when idx is
 * NULL and count equals the output size).  out[i] and q[i] receive the
 * value and scale of element idx[i].  Returns OR_OK or an error code; on
 * error nothing is written.
 */
int oracle_fwd(const uint16_t *X, const uint16_t *W, const int32_t *offs,
               int32_t E, int64_t M, int64_t N, int64_t K,
               const int64_t *idx, int64_t count, double *out, double *q)
{
    if (M < 0 || N < 0 || K < 0)
        return OR_BAD_SHAPE;
    if (!offsets_ok(offs, E, M))
        return OR_BAD_OFFSETS;
    int64_t size = M * N;
    if (!idx && count != size)
        return OR_BAD_INDEX;
    for (int64_t i = 0; idx && i < count; ++i)
        if (idx[i] < 0 || idx[i] >= size)
            return OR_BAD_INDEX;
#pragma omp parallel for schedule(dynamic, 64)
    for (int64_t i = 0; i < count; ++i) {
        int64_t f = idx ? idx[i] : i;
        fwd_element(X, W, offs, E, N, K, f / N, f % N, &out[i], &q[i]);
    }
    return OR_OK;
}

int oracle_dgrad(const uint16_t *G, const uint16_t *W, const int32_t *offs,
                 int32_t E, int64_t M, int64_t N, int64_t K,
                 const int64_t *idx, int64_t count, double *out, double *q)
{
    if (M < 0 || N < 0 || K < 0)
        return OR_BAD_SHAPE;
    if (!offsets_ok(offs, E, M))
        return OR_BAD_OFFSETS;
    int64_t size = M * K;
    if (!idx && count != size)
        return OR_BAD_INDEX;
    for (int64_t i = 0; idx && i < count; ++i)
        if (idx[i] < 0 || idx[i] >= size)
            return OR_BAD_INDEX;
#pragma omp parallel for schedule(dynamic, 64)
    for (int64_t i = 0; i < count; ++i) {
        int64_t f = idx ? idx[i] : i;
        dgrad_element(G, W, offs, E, N, K, f / K, f % K, &out[i], &q[i]);
    }
    return OR_OK;
}

int oracle_wgrad(const uint16_t *X, const uint16_t *G, const int32_t *offs,
                 int32_t E, int64_t M, int64_t N, int64_t K,
                 const int64_t *idx, int64_t count, double *out, double *q)
{
    if (M < 0 || N < 0 || K < 0)
        return OR_BAD_SHAPE;
    if (!offsets_ok(offs, E, M))
        return OR_BAD_OFFSETS;
    int64_t size = (int64_t)E * N * K;
    if (!idx && count != size)
        return OR_BAD_INDEX;
    for (int64_t i = 0; idx && i < count; ++i)
        if (idx[i] < 0 || idx[i] >= size)
            return OR_BAD_INDEX;
#pragma omp parallel for schedule(dynamic, 64)
    for (int64_t i = 0; i < count; ++i) {
        int64_t f = idx ? idx[i] : i;
        int64_t nk = N * K;
        int32_t e = (int32_t)(f / nk);
        int64_t r = f % nk;
        wgrad_element(X, G, offs, N, K, e, r / K, r % K, &out[i], &q[i]);
    }
    return OR_OK;
}

/* ---- rounding a double once ------------------------------------------- */

/* To binary32: C's conversion rounds to nearest, ties to even. */
void oracle_round_f32(const double *in, float *out, int64_t n)
{
    for (int64_t i = 0; i < n; ++i)
        out[i] = (float)in[i];
}

/*
 * To BF16 (8-bit significand, binary32 exponent range), round to nearest,
 * ties to even, directly from the double.  The spacing of BF16 values near
 * |x| is 2^(e-7) for a normal x in [2^e, 2^(e+1)) and 2^-133 below 2^-126;
 * x / spacing is an exact power-of-two scaling, rint() rounds it to the
 * nearest integer with ties to even, and the product is the rounded value.
 * Values that round to 2^128 or beyond become infinities; NaN stays NaN.
 */
static uint16_t round_to_bf16(double x)
{
    float f;
    uint32_t u;
    if (isnan(x)) {
        u = 0x7fc00000u;
        return (uint16_t)(u >> 16);
    }
    double a = fabs(x);
    double r;
    if (isinf(x)) {
        r = x;
    } else {
        double spacing;
        if (a >= ldexp(1.0, -126)) {
            int ex;
            frexp(a, &ex);                  /* a = m * 2^ex, m in [0.5, 1) */
            spacing = ldexp(1.0, (ex - 1) - 7);
        } else {
            spacing = ldexp(1.0, -133);
        }
        r = rint(x / spacing) * spacing;
        if (fabs(r) >= ldexp(1.0, 128))
            r = x < 0 ? -INFINITY : INFINITY;
    }
    f = (float)r;                           /* exact: r is a BF16 value */
    memcpy(&u, &f, sizeof u);
    return (uint16_t)(u >> 16);
}

void oracle_round_bf16(const double *in, uint16_t *out, int64_t n)
{
    for (int64_t i = 0; i < n; ++i)
        out[i] = round_to_bf16(in[i]);
}

/* ---- FP32 router GEMM: out[m,n] = sum_k x[m,k] * wr[n,k] ---------------- */

int oracle_router_exact(const float *X, const float *Wr, int64_t M, int64_t N,
                        int64_t K, const int64_t *idx, int64_t count, double *out)
{
    if (M < 0 || N < 0 || K < 0)
        return OR_BAD_SHAPE;
    int64_t size = M * N;
    if (!idx && count != size)
        return OR_BAD_INDEX;
    for (int64_t i = 0; idx && i < count; ++i)
        if (idx[i] < 0 || idx[i] >= size)
            return OR_BAD_INDEX;
#pragma omp parallel for schedule(dynamic, 64)
    for (int64_t i = 0; i < count; ++i) {
        int64_t f = idx ? idx[i] : i;
        const float *x = X + (f / N) * K;
        const float *w = Wr + (f % N) * K;
        double s = 0.0;
        for (int64_t k = 0; k < K; ++k)
            s += (double)x[k] * (double)w[k];
        out[i] = s;
    }
    return OR_OK;
}

/* The BF16 split of one FP32 value: hi = bf16(v), lo = bf16(v - hi). */
static void split_bf16x2(float v, double *hi, double *lo)
{
    *hi = bf16_value(round_to_bf16((double)v));
    *lo = bf16_value(round_to_bf16((double)v - *hi));   /* v - hi is exact */
}

int oracle_router_bf16x3(const float *X, const float *Wr, int64_t M, int64_t N,
                         int64_t K, const int64_t *idx, int64_t count, double *out)
{
    if (M < 0 || N < 0 || K < 0)
        return OR_BAD_SHAPE;
    int64_t size = M * N;
    if (!idx && count != size)
        return OR_BAD_INDEX;
    for (int64_t i = 0; idx && i < count; ++i)
        if (idx[i] < 0 || idx[i] >= size)
            return OR_BAD_INDEX;
#pragma omp parallel for schedule(dynamic, 64)
    for (int64_t i = 0; i < count; ++i) {
        int64_t f = idx ? idx[i] : i;
        const float *x = X + (f / N) * K;
        const float *w = Wr + (f % N) * K;
        double s = 0.0;
        for (int64_t k = 0; k < K; ++k) {
            double xh, xl, wh, wl;
            split_bf16x2(x[k], &xh, &xl);
            split_bf16x2(w[k], &wh, &wl);
            s += xh * wh + xh * wl + xl * wh;
        }
        out[i] = s;
    }
    return OR_OK;
}
