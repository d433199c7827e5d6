/*
 * attn_bwd_oracle.c -- plain fp64 reference for the gradients of exact
 * softmax attention.
 *
 * TEST INFRASTRUCTURE ONLY, like attn_oracle.c: only tests/,
 * __graft_entry__.smoke() and bench.py's cpu_baseline leg may load it; it
 * shares nothing with the HIP library.
 *
 * With the forward O = P V, P = softmax(S) row by row, S = scale * Q K^T
 * (+ causal mask), and an upstream gradient dO of the loss with respect to
 * O, the gradients are ("6. FlashAttention 分块逻辑" section 7.1; "9.4
 * FlashAttention 与 FlashMLA" section 9.4.5):
 *
 *   dV_j  = sum_i P_ij dO_i                       (dV = P^T dO)
 *   dP_ij = dO_i . v_j                            (dP = dO V^T)
 *   D_i   = sum_j P_ij dP_ij = dO_i . O_i         (the softmax term, a full-row sum)
 *   dS_ij = P_ij (dP_ij - D_i)
 *   dQ_i  = scale * sum_j dS_ij k_j               (dQ = scale dS K)
 *   dK_j  = scale * sum_i dS_ij q_i               (dK = scale dS^T Q)
 *
 * with sums over visible pairs only (key j visible to query i iff j < Nk and,
 * under the causal mask, j <= i: top-left alignment).  P is formed from the
 * definition: the row max m_i, l_i = sum_j exp(S_ij - m_i), P_ij =
 * exp(S_ij - m_i) / l_i, and O_i = sum_j P_ij v_j exactly; D_i is taken as
 * dO_i . O_i with that exact O.  Everything is IEEE double; inputs are
 * float32 arrays holding exactly the values the GPU receives.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#ifdef _OPENMP
#include <omp.h>
#endif

static double dot(const float *a, const float *b, int64_t d)
{
    double acc = 0.0;
    int64_t t;
    for (t = 0; t < d; ++t)
        acc += (double)a[t] * (double)b[t];
    return acc;
}

/* keys visible to query i */
static int64_t visible(int64_t i, int64_t Nk, int causal)
{
    if (!causal)
        return Nk;
    return (i + 1 < Nk) ? i + 1 : Nk;
}

/*
 * oracle_attention_bwd
 *
 * q, dout: [B, H, Nq, d]; k, v: [B, H, Nk, d]; float32, contiguous.
 * heads: flat (b * H + h) indices to evaluate (NULL: all B*H in order, then
 *        nheads must be B*H).
 * qsel:  query indices i within a head whose dQ is wanted (NULL: all Nq,
 *        then nqsel must be Nq); ksel: key indices j for dK and dV
 *        (NULL: all Nk, then nksel must be Nk).
 * dq:    [nheads, nqsel, d] double; dk, dv: [nheads, nksel, d] double;
 * delta: [nheads, Nq] double or NULL (D_i of every query of the head).
 *
 * Returns 0, -1 on a bad argument (an index out of range included), -2 if
 * an allocation fails.
 */
int oracle_attention_bwd(const float *q, const float *k, const float *v, const float *dout,
                         int64_t B, int64_t H, int64_t Nq, int64_t Nk, int64_t d,
                         double scale, int causal,
                         const int64_t *heads, int64_t nheads,
                         const int64_t *qsel, int64_t nqsel,
                         const int64_t *ksel, int64_t nksel,
                         double *dq, double *dk, double *dv, double *delta, int nthreads)
{
    int64_t hn;
    int failed = 0;
    double *m, *l, *D;

    if (!q || !k || !v || !dout || !dq || !dk || !dv || B < 1 || H < 1 || Nq < 1 ||
        Nk < 1 || d < 1 || nheads < 0 || nqsel < 0 || nksel < 0 ||
        (causal != 0 && causal != 1))
        return -1;
    if ((!heads && nheads != B * H) || (!qsel && nqsel != Nq) || (!ksel && nksel != Nk))
        return -1;
#ifdef _OPENMP
    if (nthreads <= 0)
        nthreads = omp_get_max_threads();
#endif
    m = (double *)malloc(sizeof(double) * (size_t)Nq);
    l = (double *)malloc(sizeof(double) * (size_t)Nq);
    D = (double *)malloc(sizeof(double) * (size_t)Nq);
    if (!m || !l || !D) {
        free(m);
        free(l);
        free(D);
        return -2;
    }

    for (hn = 0; hn < nheads && !failed; ++hn) {
        const int64_t bh = heads ? heads[hn] : hn;
        const float *Q, *K, *V, *dO;
        int64_t n;
        if (bh < 0 || bh >= B * H) {
            failed = 1;
            break;
        }
        Q = q + bh * Nq * d;
        dO = dout + bh * Nq * d;
        K = k + bh * Nk * d;
        V = v + bh * Nk * d;

        /* row statistics m_i, l_i and D_i = dO_i . O_i for every query */
#ifdef _OPENMP
#pragma omp parallel for num_threads(nthreads) schedule(dynamic, 8) reduction(| : failed)
#endif
        for (n = 0; n < Nq; ++n) {
            const int64_t nv = visible(n, Nk, causal);
            const float *qi = Q + n * d;
            double *o = (double *)calloc((size_t)d, sizeof(double));
            int64_t j, t;
            double mi = -INFINITY, li = 0.0, Di = 0.0;
            if (!o) {
                failed |= 2;
                continue;
            }
            for (j = 0; j < nv; ++j) {
                const double s = scale * dot(qi, K + j * d, d);
                if (s > mi)
                    mi = s;
            }
            for (j = 0; j < nv; ++j)
                li += exp(scale * dot(qi, K + j * d, d) - mi);
            /* O_i = sum_j P_ij v_j, then D_i = dO_i . O_i */
            for (j = 0; j < nv; ++j) {
                const double p = exp(scale * dot(qi, K + j * d, d) - mi) / li;
                for (t = 0; t < d; ++t)
                    o[t] += p * (double)V[j * d + t];
            }
            for (t = 0; t < d; ++t)
                Di += (double)dO[n * d + t] * o[t];
            free(o);
            m[n] = mi;
            l[n] = li;
            D[n] = Di;
        }
        if (failed)
            break;
        if (delta) {
            for (n = 0; n < Nq; ++n)
                delta[hn * Nq + n] = D[n];
        }

        /* dQ_i = scale * sum_j P_ij (dP_ij - D_i) k_j */
#ifdef _OPENMP
#pragma omp parallel for num_threads(nthreads) schedule(dynamic, 4) reduction(| : failed)
#endif
        for (n = 0; n < nqsel; ++n) {
            const int64_t i = qsel ? qsel[n] : n;
            double *out = dq + (hn * nqsel + n) * d;
            int64_t j, t, nv;
            for (t = 0; t < d; ++t)
                out[t] = 0.0;
            if (i < 0 || i >= Nq) {
                failed |= 1;
                continue;
            }
            nv = visible(i, Nk, causal);
            for (j = 0; j < nv; ++j) {
                const double p = exp(scale * dot(Q + i * d, K + j * d, d) - m[i]) / l[i];
                const double dp = dot(dO + i * d, V + j * d, d);
                const double ds = p * (dp - D[i]);
                for (t = 0; t < d; ++t)
                    out[t] += scale * ds * (double)K[j * d + t];
            }
        }

        /* dV_j = sum_i P_ij dO_i and dK_j = scale * sum_i P_ij (dP_ij - D_i) q_i */
#ifdef _OPENMP
#pragma omp parallel for num_threads(nthreads) schedule(dynamic, 4) reduction(| : failed)
#endif
        for (n = 0; n < nksel; ++n) {
            const int64_t j = ksel ? ksel[n] : n;
            double *gk = dk + (hn * nksel + n) * d;
            double *gv = dv + (hn * nksel + n) * d;
            int64_t i, t;
            for (t = 0; t < d; ++t) {
                gk[t] = 0.0;
                gv[t] = 0.0;
            }
            if (j < 0 || j >= Nk) {
                failed |= 1;
                continue;
            }
            for (i = causal ? j : 0; i < Nq; ++i) {
                const double p = exp(scale * dot(Q + i * d, K + j * d, d) - m[i]) / l[i];
                const double dp = dot(dO + i * d, V + j * d, d);
                const double ds = p * (dp - D[i]);
                for (t = 0; t < d; ++t) {
                    gv[t] += p * (double)dO[i * d + t];
                    gk[t] += scale * ds * (double)Q[i * d + t];
                }
            }
        }
    }
    free(m);
    free(l);
    free(D);
    return (failed & 2) ? -2 : failed ? -1 : 0;
}
