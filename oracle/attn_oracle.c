/*
 * attn_oracle.c -- plain fp64 reference for exact softmax attention.
 *
 * TEST INFRASTRUCTURE ONLY.  This is the correctness oracle for the
 * io_aware_amd FlashAttention forward.  Only tests/, __graft_entry__.smoke()
 * and bench.py's cpu_baseline leg may load it.  It shares no code, header,
 * table or helper with the HIP library, and the HIP library never calls it.
 *
 * What it computes, per query row i of every (batch b, head h) pair, from
 * the definition of the numerically safe softmax followed by the weighted sum
 * of value rows:
 *
 *   S_ij   = scale * sum_t q_it * k_jt              (scaled dot products)
 *   J_i    = { j < Nk : !causal || j <= i }         (causal mask: M_ij = 0 for
 *                                                    j <= i, -inf otherwise)
 *   m_i    = max_{j in J_i} S_ij                    (pass 1: the row max)
 *   l_i    = sum_{j in J_i} exp(S_ij - m_i)         (pass 2: sum of exps)
 *   O_i    = sum_{j in J_i} (exp(S_ij - m_i) / l_i) * v_j
 *                                                   (pass 3: normalise, then P.V)
 *   LSE_i  = m_i + ln(l_i)                          (natural-log logsumexp)
 *
 * Sources (the pages this build follows):
 *  - "6. FlashAttention 分块逻辑" (lowentro.cn), section 1.1: the three-pass
 *    safe softmax (max, then sum of exp(x - m), then divide);
 *  - the same page, section 4.1: the causal mask M_ij;
 *  - "9.4 FlashAttention 与 FlashMLA" (llm-fullstack-book), section 9.4.2: the
 *    safe-softmax formula with m = max_j x_j; section 9.4.5: the stored
 *    statistic is m + log(l) (natural log).
 *
 * Conventions taken where the pages are silent:
 *  - the scale is applied to the scores before max/exp;
 *  - causal alignment is top-left (key j visible iff j <= i) for any Nq, Nk;
 *  - a row with no visible key (possible only if Nk == 0 or, in a general
 *    setting, never for Nk >= 1) gives O = 0 and LSE = -inf.
 *
 * Arithmetic is IEEE double throughout: the inputs arrive as float32 arrays
 * that hold exactly the values the GPU receives (bf16 and fp16 values are
 * exactly representable in float32) and are widened to double before any
 * arithmetic.  exp and log are the C library's double-precision functions.
 * Build with -O2 and WITHOUT -ffast-math.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* One query row: q is [d], K and V are [nvis, d] (the visible prefix of the
 * key/value rows of this (b, h)), s is scratch for nvis scores. */
static void attention_one_row(const float *q, const float *K, const float *V,
                              int64_t nvis, int64_t d, double scale,
                              double *s, double *o, double *lse)
{
    int64_t j, t;
    double m, l;

    for (t = 0; t < d; ++t)
        o[t] = 0.0;
    if (nvis <= 0) {
        *lse = -INFINITY;
        return;
    }

    /* pass 1: scaled scores and their maximum */
    m = -INFINITY;
    for (j = 0; j < nvis; ++j) {
        double acc = 0.0;
        const float *kj = K + j * d;
        for (t = 0; t < d; ++t)
            acc += (double)q[t] * (double)kj[t];
        s[j] = scale * acc;
        if (s[j] > m)
            m = s[j];
    }

    /* pass 2: the normaliser l = sum exp(s_j - m) */
    l = 0.0;
    for (j = 0; j < nvis; ++j)
        l += exp(s[j] - m);

    /* pass 3: probabilities p_j = exp(s_j - m) / l, then O = sum p_j v_j */
    for (j = 0; j < nvis; ++j) {
        const double p = exp(s[j] - m) / l;
        const float *vj = V + j * d;
        for (t = 0; t < d; ++t)
            o[t] += p * (double)vj[t];
    }
    *lse = m + log(l);
}

/*
 * oracle_attention_rows
 *
 * q: [B, H, Nq, d] float32, k and v: [B, H, Nk, d] float32, all contiguous.
 * rows: flat row indices r = (b * H + h) * Nq + i into the [B*H*Nq] query
 *       rows, or NULL for all rows in order (then nrows must be B*H*Nq).
 * out:  [nrows, d] double; lse: [nrows] double (may be NULL).
 * nthreads: OpenMP threads to use (<= 0: the runtime default).
 *
 * Returns 0 on success, -1 on a bad argument (including a row index out of
 * range), -2 if scratch allocation fails.
 */
int oracle_attention_rows(const float *q, const float *k, const float *v,
                          int64_t B, int64_t H, int64_t Nq, int64_t Nk,
                          int64_t d, double scale, int causal,
                          const int64_t *rows, int64_t nrows,
                          double *out, double *lse, int nthreads)
{
    int failed = 0;
    int64_t n;

    if (!q || !k || !v || !out || B < 1 || H < 1 || Nq < 1 || Nk < 0 ||
        d < 1 || nrows < 0 || (causal != 0 && causal != 1))
        return -1;
    if (!rows && nrows != B * H * Nq)
        return -1;

#ifdef _OPENMP
    if (nthreads <= 0)
        nthreads = omp_get_max_threads();
#pragma omp parallel num_threads(nthreads) reduction(| : failed)
#endif
    {
        double *s = (double *)malloc(sizeof(double) * (size_t)(Nk > 0 ? Nk : 1));
        double lse_row;
        /* every thread reaches the worksharing loop, even without scratch */
#ifdef _OPENMP
#pragma omp for schedule(dynamic, 16)
#endif
        for (n = 0; n < nrows; ++n) {
            const int64_t r = rows ? rows[n] : n;
            const int64_t bh = r / Nq;
            const int64_t i = r % Nq;
            int64_t nvis = Nk;
            if (!s) {
                failed |= 2;
                continue;
            }
            if (r < 0 || r >= B * H * Nq) {
                failed |= 1;
                continue;
            }
            if (causal)
                nvis = (i + 1 < Nk) ? i + 1 : Nk;
            attention_one_row(q + r * d, k + bh * Nk * d, v + bh * Nk * d,
                              nvis, d, scale, s, out + n * d, &lse_row);
            if (lse)
                lse[n] = lse_row;
        }
        free(s);
    }
    return (failed & 1) ? -1 : (failed & 2) ? -2 : 0;
}

/* The number of OpenMP threads a parallel region would use by default. */
int oracle_default_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}
