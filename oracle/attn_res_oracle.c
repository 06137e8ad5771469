/*
 * Attention-residual mixing: plain fp64 CPU oracle.
 *
 * TEST INFRASTRUCTURE ONLY.  Like situ_oracle.c, this file only checks the
 * HIP library; the product path never loads it, and it shares no code,
 * header, constant or helper with the GPU library.
 *
 * What it computes (NeMo AutoModel page
 * "nemo_automodel.components.models.kimi_k3.situ", `_attn_res_core` and
 * `_apply_attn_res`; the Kimi-K3 "dense-kda-layers / store" page,
 * `_forward_attn_residual`):
 *
 *   values [T, NB, H]: the stored block sums [T, m, H] followed by the
 *     current prefix sum [T, H] along the block axis (NB = m + 1), or a
 *     ready-stacked tensor (NB = m, no prefix);
 *   for every token t and block b, RMSNorm over the hidden axis with weight
 *     w [H] and epsilon eps:
 *       r_tb = 1 / sqrt(mean_h values[t,b,h]^2 + eps)
 *       n_tbh = values[t,b,h] * r_tb * w_h
 *   a projection to one logit per block with weight p [H] (a Linear to one
 *     output, squeezed):  l_tb = sum_h n_tbh * p_h
 *   a softmax over the blocks:  P_tb = exp(l_tb) / sum_c exp(l_tc)
 *   and the weighted combine of the raw values (multiply and sum over the
 *     block axis):  out_th = sum_b P_tb * values[t,b,h].
 *
 * The softmax is evaluated with the largest logit subtracted (the same value,
 * without overflow).  Besides the output, it can return per token and block
 * the logit l, the probability P and a_tb = r_tb * sum_h |values w p| (the
 * magnitude the logit's sum is taken over), and per output element
 * S_th = sum_b P_tb |values[t,b,h]| (the combine's own magnitude): the tests
 * derive their tolerances from them.
 */
#include <math.h>
#include <stdint.h>

/* value [b][h] of token t */
static double val(const double *blocks, const double *prefix, int64_t m, int64_t H, int64_t t, int64_t b,
                  int64_t h)
{
    if (b < m)
        return blocks[(t * m + b) * H + h];
    return prefix[t * H + h];
}

void ares_oracle_forward(int64_t T, int64_t m, int has_prefix, int64_t H, const double *blocks,
                         const double *prefix, const double *norm_w, const double *proj_w, double eps,
                         double *out, double *logits, double *probs, double *absdot, double *scale)
{
    const int64_t nb = m + (has_prefix ? 1 : 0);
    double l[64], a[64], P[64];
    for (int64_t t = 0; t < T; ++t) {
        for (int64_t b = 0; b < nb; ++b) {
            double ss = 0.0;
            for (int64_t h = 0; h < H; ++h) {
                double x = val(blocks, prefix, m, H, t, b, h);
                ss += x * x;
            }
            double r = 1.0 / sqrt(ss / (double)H + eps);
            double dot = 0.0, ad = 0.0;
            for (int64_t h = 0; h < H; ++h) {
                double x = val(blocks, prefix, m, H, t, b, h);
                double n = x * r * norm_w[h];
                dot += n * proj_w[h];
                ad += fabs(n * proj_w[h]);
            }
            l[b] = dot;
            a[b] = ad;
        }
        double lmax = l[0];
        for (int64_t b = 1; b < nb; ++b)
            if (l[b] > lmax)
                lmax = l[b];
        double den = 0.0;
        for (int64_t b = 0; b < nb; ++b) {
            P[b] = exp(l[b] - lmax);
            den += P[b];
        }
        for (int64_t b = 0; b < nb; ++b)
            P[b] /= den;
        for (int64_t h = 0; h < H; ++h) {
            double o = 0.0, s = 0.0;
            for (int64_t b = 0; b < nb; ++b) {
                double x = val(blocks, prefix, m, H, t, b, h);
                o += P[b] * x;
                s += P[b] * fabs(x);
            }
            out[t * H + h] = o;
            if (scale)
                scale[t * H + h] = s;
        }
        for (int64_t b = 0; b < nb; ++b) {
            if (logits)
                logits[t * nb + b] = l[b];
            if (probs)
                probs[t * nb + b] = P[b];
            if (absdot)
                absdot[t * nb + b] = a[b];
        }
    }
}
