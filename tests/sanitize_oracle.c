/*
 * sanitize_oracle.c -- drives the C oracle (oracle/attn_oracle.c and
 * oracle/attn_bwd_oracle.c) through every index path on small inputs, for a
 * build with AddressSanitizer and UndefinedBehaviorSanitizer
 * (tests/test_sanitizers.py).  TEST INFRASTRUCTURE.
 *
 * Cases: ragged shapes (Nq != Nk, Nk < Nq, a single key, a single query),
 * both masks, several (batch, head) pairs, all rows and row subsets (in
 * reverse and repeated), head / query / key selections of the backward, and
 * the argument checks (out-of-range rows and heads, null pointers).  Each
 * computed value is checked against properties that hold exactly: forward
 * O against a direct evaluation of the definition in this file, LSE = m +
 * ln l; backward: the sums over keys of dK (0) and of dV (sum over
 * queries of dO), and selections equal to the full computation.
 * Prints "OK" and exits 0, else exits 1.
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

int oracle_attention_rows(const float *q, const float *k, const float *v, int64_t B, int64_t H, int64_t Nq,
                          int64_t Nk, int64_t d, double scale, int causal, const int64_t *rows, int64_t nrows,
                          double *out, double *lse, int nthreads);
int oracle_attention_bwd(const float *q, const float *k, const float *v, const float *dout, int64_t B, int64_t H,
                         int64_t Nq, int64_t Nk, int64_t d, double scale, int causal, const int64_t *heads,
                         int64_t nheads, const int64_t *qsel, int64_t nqsel, const int64_t *ksel, int64_t nksel,
                         double *dq, double *dk, double *dv, double *delta, int nthreads);

static int g_fail = 0;
#define CHECK(cond, ...)                          \
    do {                                          \
        if (!(cond)) {                            \
            fprintf(stderr, "FAIL: " __VA_ARGS__); \
            fprintf(stderr, "\n");                \
            g_fail = 1;                           \
        }                                         \
    } while (0)

static uint64_t g_state = 88172645463325252ull;
static float rnd(void) /* xorshift64, uniform in [-1, 1) */
{
    g_state ^= g_state << 13;
    g_state ^= g_state >> 7;
    g_state ^= g_state << 17;
    return (float)((double)(g_state >> 11) / 9007199254740992.0 * 2.0 - 1.0);
}

static float *make(int64_t n, float sigma)
{
    float *x = (float *)malloc(sizeof(float) * (size_t)n);
    for (int64_t i = 0; i < n; ++i)
        x[i] = sigma * rnd();
    return x;
}

/* direct definition for one row: O = sum_j softmax_j v_j */
static void direct_row(const float *q, const float *K, const float *V, int64_t nvis, int64_t d, double scale,
                       double *o, double *lse)
{
    double m = -INFINITY, l = 0.0;
    for (int64_t j = 0; j < nvis; ++j) {
        double s = 0.0;
        for (int64_t t = 0; t < d; ++t)
            s += (double)q[t] * K[j * d + t];
        s *= scale;
        if (s > m)
            m = s;
    }
    for (int64_t t = 0; t < d; ++t)
        o[t] = 0.0;
    for (int64_t j = 0; j < nvis; ++j) {
        double s = 0.0;
        for (int64_t t = 0; t < d; ++t)
            s += (double)q[t] * K[j * d + t];
        const double p = exp(s * scale - m);
        l += p;
        for (int64_t t = 0; t < d; ++t)
            o[t] += p * V[j * d + t];
    }
    for (int64_t t = 0; t < d; ++t)
        o[t] /= l;
    *lse = m + log(l);
}

static void forward_case(int64_t B, int64_t H, int64_t Nq, int64_t Nk, int64_t d, int causal, double scale)
{
    const int64_t nr = B * H * Nq;
    float *q = make(nr * d, 2.0f), *k = make(B * H * Nk * d, 1.0f), *v = make(B * H * Nk * d, 1.0f);
    double *out = (double *)malloc(sizeof(double) * (size_t)(nr * d)), *lse = (double *)malloc(sizeof(double) * (size_t)nr);
    double *o1 = (double *)malloc(sizeof(double) * (size_t)d);
    CHECK(oracle_attention_rows(q, k, v, B, H, Nq, Nk, d, scale, causal, NULL, nr, out, lse, 3) == 0, "forward rc");
    for (int64_t r = 0; r < nr; ++r) {
        const int64_t bh = r / Nq, i = r % Nq;
        const int64_t nvis = causal ? (i + 1 < Nk ? i + 1 : Nk) : Nk;
        double l1;
        direct_row(q + r * d, k + bh * Nk * d, v + bh * Nk * d, nvis, d, scale, o1, &l1);
        for (int64_t t = 0; t < d; ++t)
            CHECK(fabs(out[r * d + t] - o1[t]) <= 1e-12, "O row %lld", (long long)r);
        CHECK(fabs(lse[r] - l1) <= 1e-12 * (1 + fabs(l1)), "LSE row %lld", (long long)r);
    }
    /* a subset of rows, reversed and repeated; then invalid rows */
    int64_t rows[5] = {nr - 1, 0, nr / 2, nr - 1, 0};
    double *os = (double *)malloc(sizeof(double) * 5 * (size_t)d), ls[5];
    CHECK(oracle_attention_rows(q, k, v, B, H, Nq, Nk, d, scale, causal, rows, 5, os, ls, 2) == 0, "subset rc");
    for (int n = 0; n < 5; ++n) {
        CHECK(memcmp(os + n * d, out + rows[n] * d, sizeof(double) * (size_t)d) == 0, "subset O %d", n);
        CHECK(ls[n] == lse[rows[n]], "subset LSE %d", n);
    }
    int64_t bad[2] = {0, nr};
    CHECK(oracle_attention_rows(q, k, v, B, H, Nq, Nk, d, scale, causal, bad, 2, os, ls, 2) == -1, "bad row");
    CHECK(oracle_attention_rows(NULL, k, v, B, H, Nq, Nk, d, scale, causal, NULL, nr, out, lse, 1) == -1, "null q");
    free(q), free(k), free(v), free(out), free(lse), free(o1), free(os);
}

static void backward_case(int64_t B, int64_t H, int64_t Nq, int64_t Nk, int64_t d, int causal, double scale)
{
    const int64_t BH = B * H;
    float *q = make(BH * Nq * d, 1.5f), *k = make(BH * Nk * d, 1.0f), *v = make(BH * Nk * d, 1.0f);
    float *g = make(BH * Nq * d, 1.0f);
    double *dq = (double *)malloc(sizeof(double) * (size_t)(BH * Nq * d));
    double *dk = (double *)malloc(sizeof(double) * (size_t)(BH * Nk * d));
    double *dv = (double *)malloc(sizeof(double) * (size_t)(BH * Nk * d));
    double *delta = (double *)malloc(sizeof(double) * (size_t)(BH * Nq));
    CHECK(oracle_attention_bwd(q, k, v, g, B, H, Nq, Nk, d, scale, causal, NULL, BH, NULL, Nq, NULL, Nk, dq, dk, dv,
                               delta, 3) == 0,
          "backward rc");
    for (int64_t h = 0; h < BH; ++h) {
        for (int64_t t = 0; t < d; ++t) {
            double sk = 0.0, sv = 0.0, sg = 0.0, ak = 0.0;
            for (int64_t j = 0; j < Nk; ++j) {
                sk += dk[(h * Nk + j) * d + t];
                ak += fabs(dk[(h * Nk + j) * d + t]);
                sv += dv[(h * Nk + j) * d + t];
            }
            /* keys that no query sees (causal, Nk > Nq) carry no dV */
            for (int64_t i = 0; i < Nq; ++i)
                sg += g[(h * Nq + i) * d + t];
            CHECK(fabs(sk) <= 1e-10 * (1 + ak), "sum of dK head %lld", (long long)h);
            CHECK(fabs(sv - sg) <= 1e-10 * (1 + fabs(sg)), "sum of dV head %lld", (long long)h);
        }
    }
    /* selections: the last head first, queries and keys reversed */
    int64_t heads[2] = {BH - 1, 0}, qs[3] = {Nq - 1, 0, Nq / 2}, ks[3] = {Nk - 1, 0, Nk / 2};
    double *sq = (double *)malloc(sizeof(double) * 2 * 3 * (size_t)d);
    double *sk = (double *)malloc(sizeof(double) * 2 * 3 * (size_t)d);
    double *sv = (double *)malloc(sizeof(double) * 2 * 3 * (size_t)d);
    CHECK(oracle_attention_bwd(q, k, v, g, B, H, Nq, Nk, d, scale, causal, heads, 2, qs, 3, ks, 3, sq, sk, sv, NULL,
                               2) == 0,
          "selection rc");
    for (int a = 0; a < 2; ++a)
        for (int b = 0; b < 3; ++b)
            for (int64_t t = 0; t < d; ++t) {
                CHECK(fabs(sq[(a * 3 + b) * d + t] - dq[(heads[a] * Nq + qs[b]) * d + t]) <= 1e-13, "sel dQ");
                CHECK(fabs(sk[(a * 3 + b) * d + t] - dk[(heads[a] * Nk + ks[b]) * d + t]) <= 1e-13, "sel dK");
                CHECK(fabs(sv[(a * 3 + b) * d + t] - dv[(heads[a] * Nk + ks[b]) * d + t]) <= 1e-13, "sel dV");
            }
    int64_t badh[1] = {BH};
    CHECK(oracle_attention_bwd(q, k, v, g, B, H, Nq, Nk, d, scale, causal, badh, 1, NULL, Nq, NULL, Nk, dq, dk, dv,
                               NULL, 1) == -1,
          "bad head");
    int64_t badq[1] = {Nq};
    CHECK(oracle_attention_bwd(q, k, v, g, B, H, Nq, Nk, d, scale, causal, NULL, BH, badq, 1, NULL, Nk, dq, dk, dv,
                               NULL, 1) == -1,
          "bad query");
    free(q), free(k), free(v), free(g), free(dq), free(dk), free(dv), free(delta), free(sq), free(sk), free(sv);
}

int main(void)
{
    const int64_t shapes[][4] = {{1, 1, 5, 7}, {2, 3, 9, 4}, {1, 2, 1, 6}, {1, 1, 6, 1}, {2, 1, 17, 17}, {1, 2, 3, 11}};
    const int64_t dims[] = {1, 3, 8};
    for (size_t s = 0; s < sizeof(shapes) / sizeof(shapes[0]); ++s)
        for (size_t di = 0; di < sizeof(dims) / sizeof(dims[0]); ++di)
            for (int causal = 0; causal <= 1; ++causal) {
                const double scale = (s % 3 == 0) ? -0.4 : (s % 3 == 1 ? 0.0 : 0.35);
                forward_case(shapes[s][0], shapes[s][1], shapes[s][2], shapes[s][3], dims[di], causal, scale);
                backward_case(shapes[s][0], shapes[s][1], shapes[s][2], shapes[s][3], dims[di], causal, scale);
            }
    if (g_fail)
        return 1;
    printf("OK\n");
    return 0;
}
