/*
 * Weighted SiTU-GLU: plain fp64 CPU oracle.
 *
 * TEST INFRASTRUCTURE ONLY.  This file exists to check the HIP library; it is
 * never part of the product path.  Only the test suite, the smoke check and
 * the CPU-baseline leg of the benchmark load it.  It shares no code, header,
 * constant or helper with the GPU library.
 *
 * What it computes (every step is the plain definition, evaluated in double
 * precision and rounded once at the very end by the caller's choice of
 * output format):
 *
 *   Megatron-LM PR "[Dev] Add SiTU-GLU through Transformer Engine",
 *   section "Activation" (Kimi K3 report Eq. 12 as restated there):
 *       T_g = beta1 * tanh(G / beta1) * sigmoid(G)
 *       T_u = beta2 * tanh(U / beta2)
 *       Y   = T_g * T_u
 *   NeMo AutoModel page "nemo_automodel.components.models.kimi_k3.situ",
 *   `_situ_fwd_core`: the chunk result is situ(g) * up(u0) * w, with w the
 *   routing weight broadcast over the row; `linear_beta` (the up-branch beta)
 *   is optional, and without it the up branch is U itself.
 *   Same page, `_WeightedSiTUFunction.forward`: gate in the first half of the
 *   last axis of gate_up, up in the second half.
 *   atlas_core kimi_k3 `mla.rs` page, `fn sigmoid`: sigmoid is the logistic
 *   function 1 / (1 + exp(-x)).
 *
 * The backward (same NeMo page, `_situ_bwd_core` and
 * `_WeightedSiTUFunction.backward`) is the analytic gradient of
 * L = sum_ij go_ij * Y_ij, by the product and chain rules:
 *       dT_g/dG = sigmoid(G) * sech^2(G/beta1)
 *                 + beta1 * tanh(G/beta1) * sigmoid(G) * sigmoid(-G)
 *       dT_u/dU = sech^2(U/beta2)            (1 when linear_beta is None)
 *       dG = go * r * T_u * dT_g/dG ,  dU = go * r * T_g * dT_u/dU
 *       dr_i = sum_j go_ij * T_g(G_ij) * T_u(U_ij)     (per row)
 *   and, when one routing weight is broadcast over all rows, dr is the sum of
 *   that quantity over every row (autograd's sum over broadcast dimensions).
 *
 * sech^2 is written as 1 / cosh^2, never as 1 - tanh^2, so that it keeps its
 * relative accuracy in the tails.
 */
#include <math.h>
#include <stdint.h>
#include <string.h>

/* logistic sigmoid; the x < 0 branch is the same value, e^x / (1 + e^x),
 * written so that exp never overflows. */
static double logistic(double x)
{
    if (x >= 0.0)
        return 1.0 / (1.0 + exp(-x));
    double e = exp(x);
    return e / (1.0 + e);
}

static double sech2(double x)
{
    double c = cosh(x);
    return 1.0 / (c * c);
}

/* T_g(G) = beta1 * tanh(G / beta1) * sigmoid(G) */
double situ_oracle_gate(double g, double beta1)
{
    return beta1 * tanh(g / beta1) * logistic(g);
}

/* dT_g/dG */
double situ_oracle_gate_grad(double g, double beta1)
{
    double s = logistic(g);
    double sm = logistic(-g);
    return s * sech2(g / beta1) + beta1 * tanh(g / beta1) * s * sm;
}

/* T_u(U) = beta2 * tanh(U / beta2), or U when there is no linear beta */
double situ_oracle_up(double u, int has_lb, double beta2)
{
    return has_lb ? beta2 * tanh(u / beta2) : u;
}

/* dT_u/dU */
double situ_oracle_up_grad(double u, int has_lb, double beta2)
{
    return has_lb ? sech2(u / beta2) : 1.0;
}

/*
 * Forward over rows [0, rows).  gate_up is row-major [rows, 2*inter]; rw has
 * rw_rows entries (rw_rows == rows: one weight per row; rw_rows == 1: one
 * weight for every row); y is row-major [rows, inter].
 */
void situ_oracle_forward(int64_t rows, int64_t inter, const double *gate_up,
                         const double *rw, int64_t rw_rows, double beta1,
                         int has_lb, double beta2, double *y)
{
    for (int64_t i = 0; i < rows; ++i) {
        double r = rw[rw_rows == 1 ? 0 : i];
        const double *gu = gate_up + i * 2 * inter;
        for (int64_t j = 0; j < inter; ++j) {
            double tg = situ_oracle_gate(gu[j], beta1);
            double tu = situ_oracle_up(gu[inter + j], has_lb, beta2);
            y[i * inter + j] = r * tg * tu;
        }
    }
}

/*
 * Backward over rows [0, rows).  go is [rows, inter]; d_gate_up is
 * [rows, 2*inter] (dG in the first half of each row, dU in the second).
 *
 * Optional outputs (pass NULL to skip):
 *   dr      : rw_rows == rows -> dr[i] = sum_j go*T_g*T_u for row i;
 *             rw_rows == 1    -> dr[0] = that sum over every row and column.
 *   dr_abs  : [rows] sum_j |go*T_g*T_u|, the condition scale of each row sum.
 *   dg_scale: [rows, inter] |go*r*T_u| * (|sigmoid*sech^2| +
 *             |beta1*tanh*sigmoid*sigmoid(-G)|), the size of the two terms of
 *             dG before they are added (they cancel where dT_g/dG = 0).
 */
void situ_oracle_backward(int64_t rows, int64_t inter, const double *gate_up,
                          const double *rw, int64_t rw_rows, double beta1,
                          int has_lb, double beta2, const double *go,
                          double *d_gate_up, double *dr, double *dr_abs,
                          double *dg_scale)
{
    if (dr && rw_rows == 1)
        dr[0] = 0.0;
    for (int64_t i = 0; i < rows; ++i) {
        double r = rw[rw_rows == 1 ? 0 : i];
        const double *gu = gate_up + i * 2 * inter;
        const double *gor = go + i * inter;
        double *dgu = d_gate_up + i * 2 * inter;
        double acc = 0.0, acc_abs = 0.0;
        for (int64_t j = 0; j < inter; ++j) {
            double g = gu[j], u = gu[inter + j], o = gor[j];
            double tg = situ_oracle_gate(g, beta1);
            double tu = situ_oracle_up(u, has_lb, beta2);
            double tgp = situ_oracle_gate_grad(g, beta1);
            double tup = situ_oracle_up_grad(u, has_lb, beta2);
            dgu[j] = o * r * tu * tgp;
            dgu[inter + j] = o * r * tg * tup;
            double p = o * tg * tu;
            acc += p;
            acc_abs += fabs(p);
            if (dg_scale) {
                double s = logistic(g), sm = logistic(-g);
                double t1 = s * sech2(g / beta1);
                double t2 = beta1 * tanh(g / beta1) * s * sm;
                dg_scale[i * inter + j] = fabs(o * r * tu) * (fabs(t1) + fabs(t2));
            }
        }
        if (dr) {
            if (rw_rows == 1)
                dr[0] += acc;
            else
                dr[i] = acc;
        }
        if (dr_abs)
            dr_abs[i] = acc_abs;
    }
}

/*
 * Round a double to bfloat16 (8 significant bits, fp32's exponent range,
 * gradual underflow), round-to-nearest-even, and return the 16 bit pattern.
 * Written from the definition: the result is the multiple of the local
 * quantum 2^(E-7) (E = the binade's exponent, never below -126) nearest to x,
 * ties to the even multiple.  Magnitudes that round past the largest finite
 * bfloat16 become infinity.
 */
uint16_t situ_oracle_bf16_bits(double x)
{
    uint16_t sign = signbit(x) ? 0x8000u : 0u;
    if (isnan(x))
        return (uint16_t)(sign | 0x7fc0u);
    double ax = fabs(x);
    if (isinf(ax))
        return (uint16_t)(sign | 0x7f80u);
    if (ax == 0.0)
        return sign;
    int e2;
    frexp(ax, &e2);            /* ax in [2^(e2-1), 2^e2) */
    int e = e2 - 1;
    if (e < -126)
        e = -126;              /* below the normal range the quantum stays 2^-133 */
    double quantum = ldexp(1.0, e - 7);
    double q = nearbyint(ax / quantum);   /* scaling by a power of two is exact */
    double rounded = q * quantum;
    const double max_bf16 = ldexp(255.0, 120);   /* (2 - 2^-7) * 2^127 */
    if (rounded > max_bf16)
        return (uint16_t)(sign | 0x7f80u);
    float f = (float)rounded;  /* exact: at most 8 significant bits */
    uint32_t b;
    memcpy(&b, &f, sizeof b);
    return (uint16_t)(sign | (uint16_t)((b >> 16) & 0x7fffu));
}

void situ_oracle_bf16_bits_array(int64_t n, const double *x, uint16_t *out)
{
    for (int64_t i = 0; i < n; ++i)
        out[i] = situ_oracle_bf16_bits(x[i]);
}

/* Round to fp32 by C's conversion (round-to-nearest-even in the default
 * floating-point environment). */
void situ_oracle_f32_array(int64_t n, const double *x, float *out)
{
    for (int64_t i = 0; i < n; ++i)
        out[i] = (float)x[i];
}
