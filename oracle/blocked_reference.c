/*
 * blocked_reference.c -- an independent fp64 CPU implementation of the tiled,
 * online-softmax attention forward pass.
 *
 * TEST INFRASTRUCTURE ONLY, like attention_oracle.c, with which it shares no code.
 * Its job is to pin the online-softmax recurrence: it must agree with the naive
 * two-pass oracle to 1e-12 at every tiling, including tilings that do not divide N.
 *
 * It follows the merge equations of "MCU 上 Transformer 模型的 Flash Attention 实现…"
 * §二 (the aligned equation block), which merge a block's statistics through its own
 * local maximum:
 *     m_new = max(m_old, rowmax(S_i))
 *     l_new = e^(m_old - m_new) l_old + e^(rowmax(S_i) - m_new) rowsum(e^(S_i - rowmax(S_i)))
 *     O_new = e^(m_old - m_new) O_old + e^(rowmax(S_i) - m_new) e^(S_i - rowmax(S_i)) V_i
 * with the output normalised once, O / l, after the last block (the page's own
 * code does this in its final normalisation loop, §三).
 *
 * Loop order: key/value blocks outside, query blocks inside, as the Ascend page
 * describes ("FlashAttention 在昇腾 NPU 上是怎么省显存的？", tiling section) and as the
 * MCU page's code loops.  The running state is kept per query row (m[N], l[N],
 * O[N][d]); e^(-inf - x) is 0; a row with no visible key in a block skips it.
 * Causal visibility is j <= i.  Query head h reads key/value head h / (Hq/Hkv).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>

int blocked_attention_fwd(const double *q, const double *k, const double *v,
                          double *o, double *lse,
                          int64_t B, int64_t Hq, int64_t Hkv, int64_t N, int64_t d,
                          int causal, double scale, int64_t Br, int64_t Bc)
{
    if (!q || !k || !v || !o || !lse)
        return -1;
    if (B < 1 || Hq < 1 || Hkv < 1 || N < 1 || d < 1 || Hq % Hkv != 0 || Br < 1 || Bc < 1)
        return -2;

    double *m = (double *)malloc((size_t)N * sizeof(double));
    double *l = (double *)malloc((size_t)N * sizeof(double));
    double *acc = (double *)malloc((size_t)(N * d) * sizeof(double));
    double *sblk = (double *)malloc((size_t)Bc * sizeof(double));
    double *pv = (double *)malloc((size_t)d * sizeof(double));
    if (!m || !l || !acc || !sblk || !pv) {
        free(m); free(l); free(acc); free(sblk); free(pv);
        return -3;
    }

    for (int64_t b = 0; b < B; ++b) {
        for (int64_t h = 0; h < Hq; ++h) {
            const int64_t hk = h / (Hq / Hkv);
            const double *Qh = q + (b * Hq + h) * N * d;
            const double *Kh = k + (b * Hkv + hk) * N * d;
            const double *Vh = v + (b * Hkv + hk) * N * d;

            for (int64_t i = 0; i < N; ++i) {
                m[i] = -INFINITY;
                l[i] = 0.0;
            }
            for (int64_t x = 0; x < N * d; ++x)
                acc[x] = 0.0;

            for (int64_t j0 = 0; j0 < N; j0 += Bc) {
                const int64_t j1 = (j0 + Bc < N) ? j0 + Bc : N;
                for (int64_t i0 = 0; i0 < N; i0 += Br) {
                    const int64_t i1 = (i0 + Br < N) ? i0 + Br : N;
                    for (int64_t i = i0; i < i1; ++i) {
                        const int64_t jv = causal ? ((i + 1 < j1) ? i + 1 : j1) : j1;
                        if (jv <= j0)
                            continue;               /* nothing visible in this block */

                        /* Block scores and their local maximum. */
                        double mt = -INFINITY;
                        for (int64_t j = j0; j < jv; ++j) {
                            double dot = 0.0;
                            for (int64_t t = 0; t < d; ++t)
                                dot += Qh[i * d + t] * Kh[j * d + t];
                            sblk[j - j0] = scale * dot;
                            if (sblk[j - j0] > mt)
                                mt = sblk[j - j0];
                        }
                        /* Local exponentials, their row sum and their product with V. */
                        double lt = 0.0;
                        for (int64_t t = 0; t < d; ++t)
                            pv[t] = 0.0;
                        for (int64_t j = j0; j < jv; ++j) {
                            const double p = exp(sblk[j - j0] - mt);
                            lt += p;
                            for (int64_t t = 0; t < d; ++t)
                                pv[t] += p * Vh[j * d + t];
                        }
                        /* Merge with the running state through the new maximum. */
                        const double mn = (m[i] > mt) ? m[i] : mt;
                        const double a_old = exp(m[i] - mn);
                        const double a_blk = exp(mt - mn);
                        l[i] = a_old * l[i] + a_blk * lt;
                        for (int64_t t = 0; t < d; ++t)
                            acc[i * d + t] = a_old * acc[i * d + t] + a_blk * pv[t];
                        m[i] = mn;
                    }
                }
            }

            double *Oh = o + (b * Hq + h) * N * d;
            double *Lh = lse + (b * Hq + h) * N;
            for (int64_t i = 0; i < N; ++i) {
                for (int64_t t = 0; t < d; ++t)
                    Oh[i * d + t] = acc[i * d + t] / l[i];
                Lh[i] = m[i] + log(l[i]);
            }
        }
    }
    free(m); free(l); free(acc); free(sblk); free(pv);
    return 0;
}
