/*
 * MXFP8 quantisation: plain fp64 CPU oracle.
 *
 * TEST INFRASTRUCTURE ONLY.  Like situ_oracle.c, this file only checks the
 * HIP library; the product path never loads it, and it shares no code,
 * header, constant or helper with the GPU library.
 *
 * Where the format comes from.  The Megatron-LM PR "[Dev] Add SiTU-GLU
 * through Transformer Engine" (section "Test results") runs the SiTU-GLU of
 * routed and shared experts under MXFP8 block scaling; the pages do not
 * define the format.  Its plain reading is the published OCP definition:
 *   - OCP 8-bit Floating Point Specification (OFP8): element formats
 *       E4M3: 1 sign, 4 exponent bits (bias 7), 3 mantissa bits; exponent 0
 *             is subnormal (2^-6 * m/8); no infinities; S.1111.111 is NaN;
 *             largest finite magnitude 1.75 * 2^8 = 448.
 *       E5M2: 1 sign, 5 exponent bits (bias 15), 2 mantissa bits; IEEE-like
 *             subnormals (2^-14 * m/4), infinities (S.11111.00) and NaNs;
 *             largest finite magnitude 1.75 * 2^15 = 57344.
 *   - OCP Microscaling Formats (MX) Specification v1.0: a block of 32
 *     consecutive values shares one E8M0 scale X = 2^s (code s + 127,
 *     s in [-127, 127], code 255 = NaN); the conversion of a block takes
 *     s = floor(log2(max |V_i|)) - emax_elem (emax_elem = 8 for E4M3, 15
 *     for E5M2) and stores each V_i / X rounded to the element format,
 *     magnitudes past the largest finite value clamped to it.
 *
 * Readings taken where the definitions leave a choice (each is a parameter
 * or a rule below, stated once):
 *   - rounding of V_i / X: to nearest, ties to the even code (the element's
 *     mantissa LSB is the code's bit 0);
 *   - scale mode 0 ("floor") is the MX rule above; scale mode 1 ("ceil")
 *     takes the smallest s with max |V_i| <= max_finite * 2^s, so that no
 *     element saturates (the rounding-up variant used by some libraries);
 *   - s is clamped to [-127, 127]; an all-zero block gets s = -127 (code 0);
 *   - a block holding a NaN or an infinity gets the NaN scale (code 255);
 *     its element codes carry no information (the MX definition makes every
 *     element of such a block NaN); this oracle writes the NaN code;
 *   - the last block of a row may be shorter than 32 (rows whose length is
 *     not a multiple of 32); it is converted the same way over its values.
 */
#include <math.h>
#include <stdint.h>

#define MX_BLOCK 32

/* Format parameters: mantissa bits, exponent bias, the largest finite code
 * (positive), the largest finite value and emax_elem. */
struct fp8_format {
    int mbits;
    int bias;
    int max_code;
    double max_finite;
    int emax;
};

static struct fp8_format fmt_of(int fmt)
{
    struct fp8_format f;
    if (fmt == 0) {
        f.mbits = 3; f.bias = 7; f.max_code = 0x7e; f.max_finite = 448.0; f.emax = 8;
    } else {
        f.mbits = 2; f.bias = 15; f.max_code = 0x7b; f.max_finite = 57344.0; f.emax = 15;
    }
    return f;
}

/* Value of a code: (-1)^S * 2^(E - bias) * (1 + M / 2^mbits) for E > 0,
 * (-1)^S * 2^(1 - bias) * (M / 2^mbits) for E = 0, plus the special codes. */
double mx_oracle_fp8_decode(uint8_t code, int fmt)
{
    struct fp8_format f = fmt_of(fmt);
    int sign = code >> 7;
    int ebits = 7 - f.mbits;
    int e = (code >> f.mbits) & ((1 << ebits) - 1);
    int m = code & ((1 << f.mbits) - 1);
    double v;
    if (fmt == 0 && e == 15 && m == 7)
        return NAN;
    if (fmt == 1 && e == 31)
        v = m == 0 ? INFINITY : NAN;
    else if (e == 0)
        v = ldexp((double)m, 1 - f.bias - f.mbits);
    else
        v = ldexp(1.0 + (double)m / (double)(1 << f.mbits), e - f.bias);
    if (isnan(v))
        return v;
    return sign ? -v : v;
}

/* Nearest code to x, ties to the even code; magnitudes beyond the largest
 * finite value (infinities included) become that value; NaN gives the NaN
 * code 0x7f.  Written as a search over the ordered list of the format's
 * non-negative finite values, not by bit manipulation. */
uint8_t mx_oracle_fp8_encode(double x, int fmt)
{
    struct fp8_format f = fmt_of(fmt);
    if (isnan(x))
        return 0x7f;
    uint8_t sign = signbit(x) ? 0x80 : 0x00;
    double a = fabs(x);
    if (a >= f.max_finite)
        return (uint8_t)(sign | f.max_code);
    /* codes 0 .. max_code are the non-negative finite values in increasing
     * order; bisect for lo with value(lo) <= a < value(lo + 1) */
    int lo = 0, hi = f.max_code;          /* value(lo) <= a < value(hi) */
    while (hi - lo > 1) {
        int mid = (lo + hi) / 2;
        if (mx_oracle_fp8_decode((uint8_t)mid, fmt) <= a)
            lo = mid;
        else
            hi = mid;
    }
    int pick = lo;
    if (lo < f.max_code) {
        double below = a - mx_oracle_fp8_decode((uint8_t)lo, fmt);
        double above = mx_oracle_fp8_decode((uint8_t)(lo + 1), fmt) - a;
        if (above < below || (above == below && ((lo + 1) & 1) == 0))
            pick = lo + 1;
    }
    return (uint8_t)(sign | pick);
}

/* E8M0 scale code of a block whose largest magnitude is amax. */
int mx_oracle_scale_code(double amax, int fmt, int mode)
{
    struct fp8_format f = fmt_of(fmt);
    if (isnan(amax) || isinf(amax))
        return 255;
    int s;
    if (amax == 0.0) {
        s = -127;
    } else if (mode == 0) {
        int e2;
        frexp(amax, &e2);                 /* amax in [2^(e2-1), 2^e2) */
        s = (e2 - 1) - f.emax;            /* floor(log2(amax)) - emax_elem */
    } else {
        /* smallest s with amax <= max_finite * 2^s */
        int e2;
        frexp(amax, &e2);
        s = (e2 - 1) - f.emax;
        while (amax > ldexp(f.max_finite, s))
            ++s;
        while (amax <= ldexp(f.max_finite, s - 1))
            --s;
    }
    if (s < -127)
        s = -127;
    if (s > 127)
        s = 127;
    return s + 127;
}

/* Quantise one block of n <= 32 values. */
void mx_oracle_quantize_block(const double *v, int n, int fmt, int mode, uint8_t *codes, uint8_t *scale)
{
    double amax = 0.0;
    int nonfinite = 0;
    for (int i = 0; i < n; ++i) {
        if (isnan(v[i]) || isinf(v[i]))
            nonfinite = 1;
        else if (fabs(v[i]) > amax)
            amax = fabs(v[i]);
    }
    int sc = nonfinite ? 255 : mx_oracle_scale_code(amax, fmt, mode);
    *scale = (uint8_t)sc;
    for (int i = 0; i < n; ++i)
        codes[i] = sc == 255 ? 0x7f : mx_oracle_fp8_encode(ldexp(v[i], -(sc - 127)), fmt);
}

/* Rows of `cols` values (row-major), blocks of 32 along each row, the last
 * block of a row possibly short.  codes: [rows, cols]; scales:
 * [rows, ceil(cols / 32)]. */
void mx_oracle_quantize_rows(int64_t rows, int64_t cols, const double *x, int fmt, int mode,
                             uint8_t *codes, uint8_t *scales)
{
    int64_t nblk = (cols + MX_BLOCK - 1) / MX_BLOCK;
    for (int64_t i = 0; i < rows; ++i)
        for (int64_t b = 0; b < nblk; ++b) {
            int64_t j0 = b * MX_BLOCK;
            int n = (int)(cols - j0 < MX_BLOCK ? cols - j0 : MX_BLOCK);
            mx_oracle_quantize_block(x + i * cols + j0, n, fmt, mode, codes + i * cols + j0,
                                     scales + i * nblk + b);
        }
}

/* Element-wise array forms of the functions above (used by the tests to
 * bound what a GPU code may be). */
void mx_oracle_fp8_encode_array(int64_t n, const double *x, int fmt, uint8_t *out)
{
    for (int64_t i = 0; i < n; ++i)
        out[i] = mx_oracle_fp8_encode(x[i], fmt);
}

void mx_oracle_fp8_decode_array(int64_t n, const uint8_t *codes, int fmt, double *out)
{
    for (int64_t i = 0; i < n; ++i)
        out[i] = mx_oracle_fp8_decode(codes[i], fmt);
}

void mx_oracle_scale_code_array(int64_t n, const double *amax, int fmt, int mode, uint8_t *out)
{
    for (int64_t i = 0; i < n; ++i)
        out[i] = (uint8_t)mx_oracle_scale_code(amax[i], fmt, mode);
}
