// C ABI of the weighted SiTU-GLU library: argument validation, per-beta
// constants, and dispatch to the HIP kernels.  Declarations and the contract
// of every entry point are in include/situ_glu.h.
#include "situ_glu.h"

#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <string>

#include "situ_glu_internal.h"

namespace {

thread_local std::string g_last_error;

int fail(int code, const char *fmt, ...)
{
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    g_last_error = buf;
    return code;
}

bool dtype_ok(int d) { return d == SITU_DTYPE_F32 || d == SITU_DTYPE_BF16; }
int64_t dtype_bytes(int d) { return d == SITU_DTYPE_F32 ? 4 : 2; }

struct Range {
    const char *name;
    uintptr_t lo, hi;  // [lo, hi)
};

Range range(const char *name, const void *p, int64_t bytes)
{
    uintptr_t lo = reinterpret_cast<uintptr_t>(p);
    return Range{name, lo, lo + static_cast<uintptr_t>(bytes)};
}

bool overlaps(const Range &a, const Range &b)
{
    if (a.lo == a.hi || b.lo == b.hi)
        return false;
    return a.lo < b.hi && b.lo < a.hi;
}

// Shared validation of the forward's inputs.  Fills the sizes used later.
int check_common(const void *gate_up, int io_dtype, int64_t rows, int64_t inter,
                 const void *rw, int rw_dtype, int64_t rw_rows, double beta,
                 const double *linear_beta)
{
    if (!dtype_ok(io_dtype))
        return fail(SITU_ERR_INVALID_ARG, "io_dtype %d is not SITU_DTYPE_F32 (0) or SITU_DTYPE_BF16 (1)", io_dtype);
    if (!dtype_ok(rw_dtype))
        return fail(SITU_ERR_INVALID_ARG, "rw_dtype %d is not SITU_DTYPE_F32 (0) or SITU_DTYPE_BF16 (1)", rw_dtype);
    if (!(std::isfinite(beta) && beta > 0.0))
        return fail(SITU_ERR_INVALID_ARG, "beta must be finite and > 0 (got %g)", beta);
    if (linear_beta && !(std::isfinite(*linear_beta) && *linear_beta > 0.0))
        return fail(SITU_ERR_INVALID_ARG, "linear_beta must be finite and > 0, or NULL for None (got %g)",
                    *linear_beta);
    if (rows < 0 || inter < 0)
        return fail(SITU_ERR_INVALID_ARG, "negative size (rows=%lld, intermediate=%lld)", (long long)rows,
                    (long long)inter);
    if (!(rw_rows == rows || rw_rows == 1))
        return fail(SITU_ERR_INVALID_ARG,
                    "rw_rows must equal rows (%lld) or be 1 (broadcast); got %lld", (long long)rows,
                    (long long)rw_rows);
    if (inter > (int64_t)0x3fffffff)
        return fail(SITU_ERR_UNSUPPORTED, "intermediate %lld exceeds 2^30 - 1", (long long)inter);
    if (rows > (int64_t)0x7fffffff)
        return fail(SITU_ERR_UNSUPPORTED, "rows %lld exceeds 2^31 - 1", (long long)rows);
    if (rows > 0 && inter > 0) {
        if (!gate_up)
            return fail(SITU_ERR_INVALID_ARG, "gate_up is NULL");
        if (!rw)
            return fail(SITU_ERR_INVALID_ARG, "routing_weights is NULL");
        if (reinterpret_cast<uintptr_t>(gate_up) % dtype_bytes(io_dtype))
            return fail(SITU_ERR_INVALID_ARG, "gate_up is not aligned to its element size");
        if (reinterpret_cast<uintptr_t>(rw) % dtype_bytes(rw_dtype))
            return fail(SITU_ERR_INVALID_ARG, "routing_weights is not aligned to its element size");
    }
    return SITU_OK;
}

bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
bool aligned_to(const void *p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

int check_mx(int fp8_format, int scale_mode)
{
    if (fp8_format != SITU_FP8_E4M3 && fp8_format != SITU_FP8_E5M2)
        return fail(SITU_ERR_INVALID_ARG, "fp8_format %d is not SITU_FP8_E4M3 (0) or SITU_FP8_E5M2 (1)",
                    fp8_format);
    if (scale_mode != SITU_MX_SCALE_FLOOR && scale_mode != SITU_MX_SCALE_CEIL)
        return fail(SITU_ERR_INVALID_ARG,
                    "scale_mode %d is not SITU_MX_SCALE_FLOOR (0) or SITU_MX_SCALE_CEIL (1)", scale_mode);
    return SITU_OK;
}

int64_t mx_blocks(int64_t cols) { return (cols + SITU_MX_BLOCK - 1) / SITU_MX_BLOCK; }

}  // namespace

// ------------------------------------------------------------------ beta constants
namespace situ {
namespace {

// Truncated Taylor series c[k] = f^(k)(x0)/k! in long double.
constexpr int kJ = 10;
struct Jet {
    long double c[kJ];
};

Jet jconst(long double v)
{
    Jet j{};
    j.c[0] = v;
    return j;
}
Jet jadd(const Jet &a, const Jet &b)
{
    Jet r;
    for (int k = 0; k < kJ; ++k)
        r.c[k] = a.c[k] + b.c[k];
    return r;
}
Jet jsub(const Jet &a, const Jet &b)
{
    Jet r;
    for (int k = 0; k < kJ; ++k)
        r.c[k] = a.c[k] - b.c[k];
    return r;
}
Jet jscale(const Jet &a, long double s)
{
    Jet r;
    for (int k = 0; k < kJ; ++k)
        r.c[k] = a.c[k] * s;
    return r;
}
Jet jmul(const Jet &a, const Jet &b)
{
    Jet r{};
    for (int k = 0; k < kJ; ++k)
        for (int i = 0; i <= k; ++i)
            r.c[k] += a.c[i] * b.c[k - i];
    return r;
}
Jet jdiv(const Jet &a, const Jet &b)
{
    Jet q{};
    for (int k = 0; k < kJ; ++k) {
        long double s = a.c[k];
        for (int i = 0; i < k; ++i)
            s -= q.c[i] * b.c[k - i];
        q.c[k] = s / b.c[0];
    }
    return q;
}
// exp(alpha * (x0 + d)) as a series in d
Jet jexp_lin(long double alpha, long double x0)
{
    Jet r;
    long double e = expl(alpha * x0), t = 1.0L;
    for (int k = 0; k < kJ; ++k) {
        r.c[k] = e * t;
        t *= alpha / (long double)(k + 1);
    }
    return r;
}

// dT_g/dG for G < 0 as a series around x0 < 0, with e1 = exp(2G/b1),
// e2 = exp(G) (so that for G < 0: sigmoid(G) = e2/(1+e2), tanh(G/b1) =
// -(1-e1)/(1+e1), sech^2(G/b1) = 4 e1/(1+e1)^2):
//   T_g' = e2 [4 e1 (1 + e2) - b1 (1 - e1^2)] / ((1 + e1)^2 (1 + e2)^2)
Jet gate_grad_series(long double b1, long double x0)
{
    const Jet e1 = jexp_lin(2.0L / b1, x0);
    const Jet e2 = jexp_lin(1.0L, x0);
    const Jet one = jconst(1.0L);
    const Jet A = jadd(one, e1), B = jadd(one, e2);
    const Jet br = jsub(jscale(jmul(e1, B), 4.0L), jscale(jsub(one, jmul(e1, e1)), b1));
    const Jet den = jmul(jmul(A, A), jmul(B, B));
    return jdiv(jmul(e2, br), den);
}

// dT_g/dG at G < 0 in long double, from the same closed form.
long double gate_grad_at(long double b1, long double x)
{
    const long double e1 = expl(2.0L * x / b1), e2 = expl(x);
    const long double A = 1.0L + e1, B = 1.0L + e2;
    return e2 * (4.0L * e1 * B - b1 * (1.0L - e1 * e1)) / (A * A * B * B);
}

// Round a finite float to the nearest bf16 value (ties to even).
float round_to_bf16(float f)
{
    uint32_t u;
    std::memcpy(&u, &f, 4);
    u = (u + 0x7fffu + ((u >> 16) & 1u)) & 0xffff0000u;
    std::memcpy(&f, &u, 4);
    return f;
}

// The bracket 4 e1 (1 + e2) - b1 (1 - e1^2) as a function of a = -G > 0:
// positive at a = 0 (value 8), tends to -b1; its zero is -G*.
long double bracket_at(long double b1, long double a)
{
    const long double e1 = expl(-2.0L * a / b1), e2 = expl(-a);
    return 4.0L * e1 * (1.0L + e2) - b1 * (1.0L - e1 * e1);
}

}  // namespace

GateK make_gate_consts(double beta1)
{
    const long double b1 = beta1;
    GateK k{};
    k.beta1 = (float)beta1;
    k.k1 = (float)(2.0L / b1 * 1.4426950408889634073599L);
    k.y1k = (float)(2.0L / b1);
    // root of the bracket by bisection (the bracket changes sign once)
    long double lo = 0.0L, hi = 1.0L;
    while (bracket_at(b1, hi) > 0.0L && hi < 1e6L)
        hi *= 2.0L;
    for (int it = 0; it < 200; ++it) {
        const long double mid = 0.5L * (lo + hi);
        if (mid == lo || mid == hi)
            break;
        if (bracket_at(b1, mid) > 0.0L)
            lo = mid;
        else
            hi = mid;
    }
    const long double gstar = -0.5L * (lo + hi);
    const float ghi = (float)gstar;
    const Jet s = gate_grad_series(b1, (long double)ghi);
    k.win_ghi = ghi;
    k.c0 = (float)s.c[0];
    k.c1 = (float)s.c[1];
    k.c2 = (float)s.c[2];
    k.c3 = (float)s.c[3];
    k.c4 = (float)s.c[4];
    k.c5 = (float)s.c[5];
    k.c6 = (float)s.c[6];
    k.c7 = (float)s.c[7];
    // Half width: at most 1/8 and |G*|/4 (so that G - G*_f32 is exact), and
    // small enough that the dropped eighth-order term stays below 3e-7 of the
    // linear one: |c8/c1| hw^7 <= 3e-7 (the higher terms add less than that).
    // Outside it the terms of the plain difference cancel by a factor of
    // about 16 or less, so its fp32 rounding stays near 5e-6.
    long double hw = 1.0L / 8.0L;
    const long double q = fabsl(s.c[8]) > 0 ? powl(3e-7L * fabsl(s.c[1] / s.c[8]), 1.0L / 7.0L) : hw;
    if (q < hw)
        hw = q;
    if (fabsl(gstar) / 4.0L < hw)
        hw = fabsl(gstar) / 4.0L;
    k.win_hw = (float)hw;
    // bf16 io: the bf16 value nearest G* and its exact dT_g/dG / 4
    k.gsub = round_to_bf16(ghi);
    k.tsub = (float)(gate_grad_at(b1, (long double)k.gsub) / 4.0L);
    return k;
}

UpK make_up_consts(double beta2)
{
    UpK k{};
    k.beta2 = (float)beta2;
    k.ku = (float)(2.0L / (long double)beta2 * 1.4426950408889634073599L);
    const long double b = beta2, ib = 1.0L / b, ib2 = ib * ib;
    const long double p[4] = {ib, -ib * ib2 / 3.0L, 2.0L * ib * ib2 * ib2 / 15.0L,
                              -17.0L * ib * ib2 * ib2 * ib2 / 315.0L};
    bool normal = true;
    for (long double c : p)
        normal = normal && std::isnormal((float)c);
    k.inv_b2 = (float)ib;
    k.p1 = (float)p[0];
    k.p3 = (float)p[1];
    k.p5 = (float)p[2];
    k.p7 = (float)p[3];
    k.small_max = normal ? (float)(0.25L * b) : -1.0f;
    return k;
}

}  // namespace situ

namespace {

// Rows per workgroup of the strip-layout kernels (the MXFP8 element paths,
// the MXFP8 backward and the stand-alone quantiser) when a row is one strip:
// 0 lets the launcher choose; the environment variable
// SITU_GLU_ROWS_PER_BLOCK (1..16) fixes it (tuning).
int rows_per_block_override()
{
    static const int v = [] {
        const char *e = std::getenv("SITU_GLU_ROWS_PER_BLOCK");
        const int x = e ? std::atoi(e) : 0;
        return (x >= 1 && x <= 16) ? x : 0;
    }();
    return v;
}

int env_override(const char *name, int lo, int hi)
{
    const char *e = std::getenv(name);
    const int x = e ? std::atoi(e) : 0;
    return (x >= lo && x <= hi) ? x : 0;
}

// Work split of the 128-bit path (chunks of 1 KiB of every stream; see
// situ::ChunkGeom).  Measured on MI355X with bf16 io: single-wavefront
// workgroups of one chunk each read and write at 6.5-6.8 TB/s, the copy
// ceiling of that pattern, the forward with a linear beta too (its up branch's
// arithmetic hidden by the other wavefronts on the SIMD); the backward with a
// linear beta needs two chunks per wavefront (the second one's loads in
// flight during the first one's math) and four wavefronts per workgroup.
// Longer chunk runs per wavefront and persistent grid-stride loops were
// slower.
// SITU_GLU_CHUNKS_PER_WAVE (1..8) and SITU_GLU_WAVES_PER_BLOCK (1..4) override
// the choice (tuning).
constexpr int kDrWavesPerBlock = 4;  // row mapping: target wavefronts per workgroup
constexpr int kMaxRowWaves = 16;     // row mapping: wavefronts per row at most

// group4: the MXFP8 forward, where a wavefront that takes a row's aligned
// group of four chunks writes their scale bytes with one store
int plan_split(int64_t rows, int64_t inter, int64_t es, bool bwd, bool lb, bool row_dr, situ::ChunkSplit &sp,
               bool group4 = false)
{
    static const int env_k = env_override("SITU_GLU_CHUNKS_PER_WAVE", 1, 8);
    static const int env_w = env_override("SITU_GLU_WAVES_PER_BLOCK", 1, 4);
    situ::ChunkGeom g{};
    const int64_t half = inter * es;
    const int64_t cpr = (half + 1023) / 1024;
    const int64_t total = rows * cpr;
    if (total >= ((int64_t)1 << 31))
        return fail(SITU_ERR_UNSUPPORTED, "%lld rows of %lld bytes each exceed 2^31 KiB per half",
                    (long long)rows, (long long)half);
    g.half = (uint32_t)half;
    g.cpr = (int)cpr;
    if (cpr > 1) {
        // chunk / cpr = floor(chunk * magic / 2^(31 + l)) for every chunk < 2^31
        int l = 0;
        while (((int64_t)1 << l) < cpr)
            ++l;
        g.magic = (uint32_t)((((uint64_t)1) << (31 + l)) / (uint64_t)cpr + 1);
        g.shift = l - 1;
    }
    // the MXFP8 forward (group4) keeps two chunks per wavefront with a linear
    // beta where a row's chunks do not come in groups of four: its quantiser
    // adds enough arithmetic that one chunk per wavefront is 5% slower
    int k = es == 2 ? (group4 ? (cpr % 4 == 0 ? 4 : lb ? 2 : 1) : bwd && lb ? 2 : 1) : 2;
    int wpb = es == 2 && bwd && lb ? 4 : 1;
    if (env_k)
        k = env_k;
    if (env_w)
        wpb = env_w;
    if (!row_dr) {
        const int64_t waves = (total + k - 1) / k;
        g.k = k;
        sp.grid = (unsigned)((waves + wpb - 1) / wpb);
        sp.block = 64 * wpb;
    } else {
        const int64_t kmin = (cpr + kMaxRowWaves - 1) / kMaxRowWaves;
        const int64_t kr = k < kmin ? kmin : k;
        const int wpr = (int)((cpr + kr - 1) / kr);
        int rpb = (env_w ? env_w : kDrWavesPerBlock) / wpr;
        if (rpb < 1)
            rpb = 1;
        g.k = (int)kr;
        g.wpr = wpr;
        g.wmagic = (uint32_t)((256 + wpr - 1) / wpr);
        sp.grid = (unsigned)((rows + rpb - 1) / rpb);
        sp.block = 64 * wpr * rpb;
    }
    sp.geom = g;
    sp.total = (uint32_t)total;
    return SITU_OK;
}

// The constants depend on beta alone; keep the last one per thread.
const situ::GateK &gate_consts(double beta)
{
    thread_local double cached_beta = -1.0;
    thread_local situ::GateK cached{};
    if (beta != cached_beta) {
        cached = situ::make_gate_consts(beta);
        cached_beta = beta;
    }
    return cached;
}

}  // namespace

// ------------------------------------------------------------------ C ABI

extern "C" {

int situ_glu_abi_version(void) { return SITU_GLU_ABI_VERSION; }

const char *situ_glu_last_error(void) { return g_last_error.c_str(); }

size_t situ_glu_bwd_workspace_bytes(int64_t rows, int64_t intermediate, int64_t rw_rows)
{
    if (rows < 0 || intermediate < 0 || rows > (int64_t)0x7fffffff)
        return 0;
    if (rw_rows == 1 && rows > 1)
        return (size_t)rows * sizeof(float);
    return 0;
}

// Exposed for tests: the root-window constants the kernels use for a beta:
// out[0] = G*_f32, out[1] = half width, out[2..9] = c0..c7,
// out[10] = the bf16 value nearest G*, out[11] = dT_g/dG there.
int situ_glu_gate_window(double beta, float *out)
{
    g_last_error.clear();
    if (!(std::isfinite(beta) && beta > 0.0))
        return fail(SITU_ERR_INVALID_ARG, "beta must be finite and > 0 (got %g)", beta);
    if (!out)
        return fail(SITU_ERR_INVALID_ARG, "out is NULL");
    const situ::GateK k = situ::make_gate_consts(beta);
    out[0] = k.win_ghi;
    out[1] = k.win_hw;
    out[2] = k.c0;
    out[3] = k.c1;
    out[4] = k.c2;
    out[5] = k.c3;
    out[6] = k.c4;
    out[7] = k.c5;
    out[8] = k.c6;
    out[9] = k.c7;
    out[10] = k.gsub;
    out[11] = 4.0f * k.tsub;
    return SITU_OK;
}

int situ_glu_split(int io_dtype, int64_t rows, int64_t intermediate, int linear_beta_given, int direction,
                   int64_t *out)
{
    g_last_error.clear();
    if (!dtype_ok(io_dtype))
        return fail(SITU_ERR_INVALID_ARG, "io_dtype %d is not SITU_DTYPE_F32 (0) or SITU_DTYPE_BF16 (1)", io_dtype);
    if (direction < 0 || direction > 3)
        return fail(SITU_ERR_INVALID_ARG, "direction %d is not 0, 1, 2 or 3", direction);
    if (!out)
        return fail(SITU_ERR_INVALID_ARG, "out is NULL");
    if (rows < 1 || rows > (int64_t)0x7fffffff || intermediate < 1 || intermediate > (int64_t)0x3fffffff)
        return fail(SITU_ERR_INVALID_ARG, "sizes out of range (rows=%lld, intermediate=%lld)", (long long)rows,
                    (long long)intermediate);
    const int64_t es = dtype_bytes(io_dtype);
    if ((intermediate * es) % 16 || intermediate * 2 * es >= ((int64_t)1 << 31))
        return fail(SITU_ERR_INVALID_ARG, "these sizes take the element path (no chunk split)");
    situ::ChunkSplit sp{};
    const int rc = plan_split(rows, intermediate, es, direction == 1 || direction == 2, linear_beta_given != 0,
                              direction == 2, sp, direction == 3);
    if (rc)
        return rc;
    out[0] = sp.geom.cpr;
    out[1] = sp.total;
    out[2] = sp.geom.k;
    out[3] = sp.geom.wpr;
    out[4] = sp.grid;
    out[5] = sp.block;
    out[6] = sp.geom.magic;
    out[7] = sp.geom.shift;
    out[8] = sp.geom.wmagic;
    out[9] = sp.geom.half;
    return SITU_OK;
}

int situ_glu_fwd(const void *gate_up, int io_dtype, int64_t rows, int64_t intermediate,
                 const void *routing_weights, int rw_dtype, int64_t rw_rows, double beta,
                 const double *linear_beta, void *out, void *stream)
{
    g_last_error.clear();
    int rc = check_common(gate_up, io_dtype, rows, intermediate, routing_weights, rw_dtype, rw_rows,
                          beta, linear_beta);
    if (rc)
        return rc;
    if (rows == 0 || intermediate == 0)
        return SITU_OK;
    const int64_t es = dtype_bytes(io_dtype);
    if (!out)
        return fail(SITU_ERR_INVALID_ARG, "out is NULL");
    if (reinterpret_cast<uintptr_t>(out) % es)
        return fail(SITU_ERR_INVALID_ARG, "out is not aligned to its element size");
    const Range r_out = range("out", out, rows * intermediate * es);
    const Range r_in = range("gate_up", gate_up, rows * intermediate * 2 * es);
    const Range r_rw = range("routing_weights", routing_weights, rw_rows * dtype_bytes(rw_dtype));
    if (overlaps(r_out, r_in) || overlaps(r_out, r_rw))
        return fail(SITU_ERR_INVALID_ARG, "out overlaps an input");

    situ::FwdLaunch L{};
    L.gate_up = gate_up;
    L.rw = routing_weights;
    L.rw_bf16 = rw_dtype == SITU_DTYPE_BF16;
    L.rw_stride = rw_rows == rows ? 1 : 0;
    L.out = out;
    L.rows = rows;
    L.inter = (int)intermediate;
    L.io = io_dtype == SITU_DTYPE_BF16 ? situ::IO_BF16 : situ::IO_F32;
    L.vec = aligned16(gate_up) && aligned16(out) && (intermediate * es) % 16 == 0 &&
            intermediate * 2 * es < ((int64_t)1 << 31);
    L.lb = linear_beta != nullptr;
    L.fast = beta == 4.0;
    if (L.vec && (rc = plan_split(rows, intermediate, es, false, L.lb, false, L.split)))
        return rc;
    L.gk = gate_consts(beta);
    L.uk = situ::make_up_consts(linear_beta ? *linear_beta : 1.0);
    const int err = situ::launch_fwd(L, stream);
    if (err)
        return fail(SITU_ERR_DEVICE, "forward launch failed: %s", situ::device_error_string(err));
    return SITU_OK;
}

}  // extern "C"

namespace {

// situ_glu_bwd, with the broadcast-dr workspace either the caller's or (own_scratch) the
// library's per-device scratch array.
int bwd_entry(const void *gate_up, int io_dtype, int64_t rows, int64_t intermediate, const void *routing_weights,
              int rw_dtype, int64_t rw_rows, double beta, const double *linear_beta, const void *grad_out,
              void *d_gate_up, void *d_routing_weights, void *workspace, size_t workspace_bytes, bool own_scratch,
              void *stream)
{
    g_last_error.clear();
    int rc = check_common(gate_up, io_dtype, rows, intermediate, routing_weights, rw_dtype, rw_rows,
                          beta, linear_beta);
    if (rc)
        return rc;
    const int64_t es = dtype_bytes(io_dtype);
    const int64_t rs = dtype_bytes(rw_dtype);
    if (d_routing_weights && reinterpret_cast<uintptr_t>(d_routing_weights) % rs)
        return fail(SITU_ERR_INVALID_ARG, "d_routing_weights is not aligned to its element size");
    if (rows == 0 || intermediate == 0) {
        if (d_routing_weights && rw_rows > 0) {
            // an empty sum: the gradient of every routing weight is zero
            const int err = situ::launch_zero(d_routing_weights, rw_rows * rs, stream);
            if (err)
                return fail(SITU_ERR_DEVICE, "zero fill failed: %s", situ::device_error_string(err));
        }
        return SITU_OK;
    }
    if (!grad_out)
        return fail(SITU_ERR_INVALID_ARG, "grad_out is NULL");
    if (!d_gate_up)
        return fail(SITU_ERR_INVALID_ARG, "d_gate_up is NULL");
    if (reinterpret_cast<uintptr_t>(grad_out) % es)
        return fail(SITU_ERR_INVALID_ARG, "grad_out is not aligned to its element size");
    if (reinterpret_cast<uintptr_t>(d_gate_up) % es)
        return fail(SITU_ERR_INVALID_ARG, "d_gate_up is not aligned to its element size");
    const bool broadcast_dr = d_routing_weights && rw_rows == 1 && rows > 1;
    const size_t need = broadcast_dr ? (size_t)rows * sizeof(float) : 0;
    if (need && own_scratch) {
        if (rows > SITU_NOALLOC_MAX_ROWS)
            return fail(SITU_ERR_UNSUPPORTED,
                        "one broadcast routing weight with its gradient needs %lld rows of scratch; the "
                        "library's scratch holds %d (SITU_NOALLOC_MAX_ROWS)", (long long)rows,
                        (int)SITU_NOALLOC_MAX_ROWS);
        int err = 0;
        workspace = situ::device_scratch(&err);
        if (!workspace)
            return fail(SITU_ERR_DEVICE, "scratch address lookup failed: %s", situ::device_error_string(err));
        workspace_bytes = (size_t)SITU_NOALLOC_MAX_ROWS * sizeof(float);
    } else if (need) {
        if (!workspace)
            return fail(SITU_ERR_INVALID_ARG, "workspace is NULL but %zu bytes are needed", need);
        if (workspace_bytes < need)
            return fail(SITU_ERR_INVALID_ARG, "workspace has %zu bytes, %zu needed", workspace_bytes, need);
        if (reinterpret_cast<uintptr_t>(workspace) % sizeof(float))
            return fail(SITU_ERR_INVALID_ARG, "workspace is not 4-byte aligned");
    }
    const Range in_gu = range("gate_up", gate_up, rows * intermediate * 2 * es);
    const Range in_rw = range("routing_weights", routing_weights, rw_rows * rs);
    const Range in_go = range("grad_out", grad_out, rows * intermediate * es);
    const Range o_dgu = range("d_gate_up", d_gate_up, rows * intermediate * 2 * es);
    const Range o_drw = range("d_routing_weights", d_routing_weights, d_routing_weights ? rw_rows * rs : 0);
    // the library's own scratch is a separate allocation: it overlaps no caller buffer
    const Range o_ws = range("workspace", workspace, own_scratch ? 0 : (int64_t)need);
    const Range ins[] = {in_gu, in_rw, in_go};
    const Range outs[] = {o_dgu, o_drw, o_ws};
    for (const Range &o : outs)
        for (const Range &i : ins)
            if (overlaps(o, i))
                return fail(SITU_ERR_INVALID_ARG, "%s overlaps input %s", o.name, i.name);
    if (overlaps(o_dgu, o_drw) || overlaps(o_dgu, o_ws) || overlaps(o_drw, o_ws))
        return fail(SITU_ERR_INVALID_ARG, "output buffers overlap each other");

    situ::BwdLaunch L{};
    L.gate_up = gate_up;
    L.rw = routing_weights;
    L.rw_bf16 = rw_dtype == SITU_DTYPE_BF16;
    L.rw_stride = rw_rows == rows ? 1 : 0;
    L.grad_out = grad_out;
    L.d_gate_up = d_gate_up;
    L.d_rw = d_routing_weights;
    L.row_partials = static_cast<float *>(need ? workspace : nullptr);
    L.rows = rows;
    L.inter = (int)intermediate;
    L.io = io_dtype == SITU_DTYPE_BF16 ? situ::IO_BF16 : situ::IO_F32;
    L.vec = aligned16(gate_up) && aligned16(grad_out) && aligned16(d_gate_up) &&
            (intermediate * es) % 16 == 0 && intermediate * 2 * es < ((int64_t)1 << 31);
    L.lb = linear_beta != nullptr;
    L.fast = beta == 4.0;
    if (L.vec && (rc = plan_split(rows, intermediate, es, true, L.lb, d_routing_weights != nullptr, L.split)))
        return rc;
    L.gk = gate_consts(beta);
    L.uk = situ::make_up_consts(linear_beta ? *linear_beta : 1.0);
    const int err = situ::launch_bwd(L, stream);
    if (err)
        return fail(SITU_ERR_DEVICE, "backward launch failed: %s", situ::device_error_string(err));
    return SITU_OK;
}

}  // namespace

extern "C" {

int situ_glu_bwd(const void *gate_up, int io_dtype, int64_t rows, int64_t intermediate,
                 const void *routing_weights, int rw_dtype, int64_t rw_rows, double beta,
                 const double *linear_beta, const void *grad_out, void *d_gate_up,
                 void *d_routing_weights, void *workspace, size_t workspace_bytes, void *stream)
{
    return bwd_entry(gate_up, io_dtype, rows, intermediate, routing_weights, rw_dtype, rw_rows, beta, linear_beta,
                     grad_out, d_gate_up, d_routing_weights, workspace, workspace_bytes, false, stream);
}

int situ_glu_bwd_noalloc(const void *gate_up, int io_dtype, int64_t rows, int64_t intermediate,
                         const void *routing_weights, int rw_dtype, int64_t rw_rows, double beta,
                         const double *linear_beta, const void *grad_out, void *d_gate_up,
                         void *d_routing_weights, void *stream)
{
    return bwd_entry(gate_up, io_dtype, rows, intermediate, routing_weights, rw_dtype, rw_rows, beta, linear_beta,
                     grad_out, d_gate_up, d_routing_weights, nullptr, 0, true, stream);
}

int situ_glu_fwd_mxfp8(const void *gate_up, int io_dtype, int64_t rows, int64_t intermediate,
                       const void *routing_weights, int rw_dtype, int64_t rw_rows, double beta,
                       const double *linear_beta, int fp8_format, int scale_mode, void *codes, void *scales,
                       void *stream)
{
    g_last_error.clear();
    int rc = check_common(gate_up, io_dtype, rows, intermediate, routing_weights, rw_dtype, rw_rows,
                          beta, linear_beta);
    if (rc)
        return rc;
    if ((rc = check_mx(fp8_format, scale_mode)))
        return rc;
    if (rows == 0 || intermediate == 0)
        return SITU_OK;
    if (!codes)
        return fail(SITU_ERR_INVALID_ARG, "codes is NULL");
    if (!scales)
        return fail(SITU_ERR_INVALID_ARG, "scales is NULL");
    const int64_t es = dtype_bytes(io_dtype);
    const Range o_codes = range("codes", codes, rows * intermediate);
    const Range o_scales = range("scales", scales, rows * mx_blocks(intermediate));
    const Range ins[] = {range("gate_up", gate_up, rows * intermediate * 2 * es),
                         range("routing_weights", routing_weights, rw_rows * dtype_bytes(rw_dtype))};
    for (const Range &i : ins)
        if (overlaps(o_codes, i) || overlaps(o_scales, i))
            return fail(SITU_ERR_INVALID_ARG, "an output overlaps input %s", i.name);
    if (overlaps(o_codes, o_scales))
        return fail(SITU_ERR_INVALID_ARG, "codes and scales overlap");

    situ::FwdMxLaunch L{};
    L.gate_up = gate_up;
    L.rw = routing_weights;
    L.rw_bf16 = rw_dtype == SITU_DTYPE_BF16;
    L.rw_stride = rw_rows == rows ? 1 : 0;
    L.codes = codes;
    L.scales = scales;
    L.rows = rows;
    L.inter = (int)intermediate;
    L.io = io_dtype == SITU_DTYPE_BF16 ? situ::IO_BF16 : situ::IO_F32;
    L.vec = aligned16(gate_up) && (intermediate * es) % 16 == 0 && intermediate * 2 * es < ((int64_t)1 << 31) &&
            aligned_to(codes, io_dtype == SITU_DTYPE_BF16 ? 8 : 4);
    L.lb = linear_beta != nullptr;
    L.fast = beta == 4.0;
    L.fmt = fp8_format == SITU_FP8_E5M2 ? situ::FP8_E5M2 : situ::FP8_E4M3;
    L.ceil_mode = scale_mode == SITU_MX_SCALE_CEIL;
    L.rows_per_block = rows_per_block_override();
    if (L.vec && (rc = plan_split(rows, intermediate, es, false, L.lb, false, L.split, true)))
        return rc;
    L.gk = gate_consts(beta);
    L.uk = situ::make_up_consts(linear_beta ? *linear_beta : 1.0);
    const int err = situ::launch_fwd_mx(L, stream);
    if (err)
        return fail(SITU_ERR_DEVICE, "MXFP8 forward launch failed: %s", situ::device_error_string(err));
    return SITU_OK;
}

int situ_glu_bwd_mxfp8(const void *gate_up, int io_dtype, int64_t rows, int64_t intermediate,
                       const void *routing_weights, int rw_dtype, int64_t rw_rows, double beta,
                       const double *linear_beta, const void *grad_out, int fp8_format, int scale_mode,
                       void *d_codes, void *d_scales, void *d_routing_weights, void *workspace,
                       size_t workspace_bytes, void *stream)
{
    g_last_error.clear();
    int rc = check_common(gate_up, io_dtype, rows, intermediate, routing_weights, rw_dtype, rw_rows,
                          beta, linear_beta);
    if (rc)
        return rc;
    if ((rc = check_mx(fp8_format, scale_mode)))
        return rc;
    const int64_t es = dtype_bytes(io_dtype);
    const int64_t rs = dtype_bytes(rw_dtype);
    if (d_routing_weights && reinterpret_cast<uintptr_t>(d_routing_weights) % rs)
        return fail(SITU_ERR_INVALID_ARG, "d_routing_weights is not aligned to its element size");
    if (rows == 0 || intermediate == 0) {
        if (d_routing_weights && rw_rows > 0) {
            const int err = situ::launch_zero(d_routing_weights, rw_rows * rs, stream);
            if (err)
                return fail(SITU_ERR_DEVICE, "zero fill failed: %s", situ::device_error_string(err));
        }
        return SITU_OK;
    }
    if (!grad_out)
        return fail(SITU_ERR_INVALID_ARG, "grad_out is NULL");
    if (!d_codes || !d_scales)
        return fail(SITU_ERR_INVALID_ARG, "d_codes or d_scales is NULL");
    if (reinterpret_cast<uintptr_t>(grad_out) % es)
        return fail(SITU_ERR_INVALID_ARG, "grad_out is not aligned to its element size");
    const bool broadcast_dr = d_routing_weights && rw_rows == 1 && rows > 1;
    const size_t need = broadcast_dr ? (size_t)rows * sizeof(float) : 0;
    if (need) {
        if (!workspace)
            return fail(SITU_ERR_INVALID_ARG, "workspace is NULL but %zu bytes are needed", need);
        if (workspace_bytes < need)
            return fail(SITU_ERR_INVALID_ARG, "workspace has %zu bytes, %zu needed", workspace_bytes, need);
        if (reinterpret_cast<uintptr_t>(workspace) % sizeof(float))
            return fail(SITU_ERR_INVALID_ARG, "workspace is not 4-byte aligned");
    }
    const Range ins[] = {range("gate_up", gate_up, rows * intermediate * 2 * es),
                         range("routing_weights", routing_weights, rw_rows * rs),
                         range("grad_out", grad_out, rows * intermediate * es)};
    const Range outs[] = {range("d_codes", d_codes, rows * intermediate * 2),
                          range("d_scales", d_scales, rows * 2 * mx_blocks(intermediate)),
                          range("d_routing_weights", d_routing_weights, d_routing_weights ? rw_rows * rs : 0),
                          range("workspace", workspace, (int64_t)need)};
    for (const Range &o : outs)
        for (const Range &i : ins)
            if (overlaps(o, i))
                return fail(SITU_ERR_INVALID_ARG, "%s overlaps input %s", o.name, i.name);
    for (int a = 0; a < 4; ++a)
        for (int b = a + 1; b < 4; ++b)
            if (overlaps(outs[a], outs[b]))
                return fail(SITU_ERR_INVALID_ARG, "%s overlaps %s", outs[a].name, outs[b].name);

    situ::BwdMxLaunch L{};
    L.gate_up = gate_up;
    L.rw = routing_weights;
    L.rw_bf16 = rw_dtype == SITU_DTYPE_BF16;
    L.rw_stride = rw_rows == rows ? 1 : 0;
    L.grad_out = grad_out;
    L.codes = d_codes;
    L.scales = d_scales;
    L.d_rw = d_routing_weights;
    L.row_partials = static_cast<float *>(need ? workspace : nullptr);
    L.rows = rows;
    L.inter = (int)intermediate;
    L.io = io_dtype == SITU_DTYPE_BF16 ? situ::IO_BF16 : situ::IO_F32;
    L.vec = aligned16(gate_up) && aligned16(grad_out) && (intermediate * es) % 16 == 0 &&
            intermediate * 2 * es < ((int64_t)1 << 31) && aligned_to(d_codes, io_dtype == SITU_DTYPE_BF16 ? 8 : 4);
    L.lb = linear_beta != nullptr;
    L.fast = beta == 4.0;
    L.fmt = fp8_format == SITU_FP8_E5M2 ? situ::FP8_E5M2 : situ::FP8_E4M3;
    L.ceil_mode = scale_mode == SITU_MX_SCALE_CEIL;
    L.rows_per_block = rows_per_block_override();
    L.gk = gate_consts(beta);
    L.uk = situ::make_up_consts(linear_beta ? *linear_beta : 1.0);
    const int err = situ::launch_bwd_mx(L, stream);
    if (err)
        return fail(SITU_ERR_DEVICE, "MXFP8 backward launch failed: %s", situ::device_error_string(err));
    return SITU_OK;
}

int situ_glu_mx_quantize(const void *x, int io_dtype, int64_t rows, int64_t cols, int fp8_format,
                         int scale_mode, void *codes, void *scales, void *stream)
{
    g_last_error.clear();
    if (!dtype_ok(io_dtype))
        return fail(SITU_ERR_INVALID_ARG, "io_dtype %d is not SITU_DTYPE_F32 (0) or SITU_DTYPE_BF16 (1)", io_dtype);
    int rc = check_mx(fp8_format, scale_mode);
    if (rc)
        return rc;
    if (rows < 0 || cols < 0)
        return fail(SITU_ERR_INVALID_ARG, "negative size (rows=%lld, cols=%lld)", (long long)rows,
                    (long long)cols);
    if (cols > (int64_t)0x3fffffff)
        return fail(SITU_ERR_UNSUPPORTED, "cols %lld exceeds 2^30 - 1", (long long)cols);
    if (rows > (int64_t)0x7fffffff)
        return fail(SITU_ERR_UNSUPPORTED, "rows %lld exceeds 2^31 - 1", (long long)rows);
    if (rows == 0 || cols == 0)
        return SITU_OK;
    const int64_t es = dtype_bytes(io_dtype);
    if (!x)
        return fail(SITU_ERR_INVALID_ARG, "x is NULL");
    if (!aligned_to(x, (uintptr_t)es))
        return fail(SITU_ERR_INVALID_ARG, "x is not aligned to its element size");
    if (!codes)
        return fail(SITU_ERR_INVALID_ARG, "codes is NULL");
    if (!scales)
        return fail(SITU_ERR_INVALID_ARG, "scales is NULL");
    const Range in_x = range("x", x, rows * cols * es);
    const Range o_codes = range("codes", codes, rows * cols);
    const Range o_scales = range("scales", scales, rows * mx_blocks(cols));
    if (overlaps(o_codes, in_x) || overlaps(o_scales, in_x))
        return fail(SITU_ERR_INVALID_ARG, "an output overlaps input x");
    if (overlaps(o_codes, o_scales))
        return fail(SITU_ERR_INVALID_ARG, "codes and scales overlap");

    situ::MxQuantLaunch L{};
    L.x = x;
    L.codes = codes;
    L.scales = scales;
    L.rows = rows;
    L.cols = (int)cols;
    L.io = io_dtype == SITU_DTYPE_BF16 ? situ::IO_BF16 : situ::IO_F32;
    L.vec = aligned16(x) && (cols * es) % 16 == 0 && cols * es < ((int64_t)1 << 31) &&
            aligned_to(codes, io_dtype == SITU_DTYPE_BF16 ? 8 : 4);
    L.fmt = fp8_format == SITU_FP8_E5M2 ? situ::FP8_E5M2 : situ::FP8_E4M3;
    L.ceil_mode = scale_mode == SITU_MX_SCALE_CEIL;
    L.rows_per_block = rows_per_block_override();
    const int err = situ::launch_mx_quant(L, stream);
    if (err)
        return fail(SITU_ERR_DEVICE, "MXFP8 quantiser launch failed: %s", situ::device_error_string(err));
    return SITU_OK;
}

int situ_glu_attn_res_fwd(const void *blocks, int64_t tokens, int64_t nblocks, int64_t hidden, const void *prefix,
                          int io_dtype, const void *norm_weight, const void *proj_weight, int w_dtype, double eps,
                          void *out, int out_dtype, void *stream)
{
    g_last_error.clear();
    if (!dtype_ok(io_dtype) || !dtype_ok(w_dtype) || !dtype_ok(out_dtype))
        return fail(SITU_ERR_INVALID_ARG, "dtypes must be SITU_DTYPE_F32 (0) or SITU_DTYPE_BF16 (1) (io %d, w %d, out %d)",
                    io_dtype, w_dtype, out_dtype);
    if (!(std::isfinite(eps) && eps >= 0.0))
        return fail(SITU_ERR_INVALID_ARG, "eps must be finite and >= 0 (got %g)", eps);
    if (tokens < 0 || nblocks < 0 || hidden < 0)
        return fail(SITU_ERR_INVALID_ARG, "negative size (tokens=%lld, nblocks=%lld, hidden=%lld)", (long long)tokens,
                    (long long)nblocks, (long long)hidden);
    if (hidden > (int64_t)0x3fffffff)
        return fail(SITU_ERR_UNSUPPORTED, "hidden %lld exceeds 2^30 - 1", (long long)hidden);
    if (tokens > (int64_t)0x7fffffff)
        return fail(SITU_ERR_UNSUPPORTED, "tokens %lld exceeds 2^31 - 1", (long long)tokens);
    if (tokens == 0 || hidden == 0)
        return SITU_OK;
    const int64_t nb = nblocks + (prefix ? 1 : 0);
    if (nb < 1 || nb > 16)
        return fail(SITU_ERR_INVALID_ARG, "the values must hold 1 to 16 blocks (got %lld)", (long long)nb);
    if (nblocks > 0 && !blocks)
        return fail(SITU_ERR_INVALID_ARG, "blocks is NULL");
    if (!norm_weight || !proj_weight)
        return fail(SITU_ERR_INVALID_ARG, "norm_weight or proj_weight is NULL");
    if (!out)
        return fail(SITU_ERR_INVALID_ARG, "out is NULL");
    const int64_t es = dtype_bytes(io_dtype), ws = dtype_bytes(w_dtype), os = dtype_bytes(out_dtype);
    if ((blocks && !aligned_to(blocks, es)) || (prefix && !aligned_to(prefix, es)))
        return fail(SITU_ERR_INVALID_ARG, "blocks or prefix is not aligned to its element size");
    if (!aligned_to(norm_weight, ws) || !aligned_to(proj_weight, ws))
        return fail(SITU_ERR_INVALID_ARG, "a weight is not aligned to its element size");
    if (!aligned_to(out, os))
        return fail(SITU_ERR_INVALID_ARG, "out is not aligned to its element size");
    const Range o = range("out", out, tokens * hidden * os);
    const Range ins[] = {range("blocks", blocks, nblocks ? tokens * nblocks * hidden * es : 0),
                         range("prefix", prefix, prefix ? tokens * hidden * es : 0),
                         range("norm_weight", norm_weight, hidden * ws), range("proj_weight", proj_weight, hidden * ws)};
    for (const Range &i : ins)
        if (overlaps(o, i))
            return fail(SITU_ERR_INVALID_ARG, "out overlaps input %s", i.name);

    situ::AresLaunch L{};
    L.blocks = blocks;
    L.prefix = prefix;
    L.tokens = tokens;
    L.m = (int)nblocks;
    L.nb = (int)nb;
    L.hidden = (int)hidden;
    L.norm_w = norm_weight;
    L.proj_w = proj_weight;
    L.w_bf16 = w_dtype == SITU_DTYPE_BF16;
    L.eps = (float)eps;
    L.out = out;
    L.io = io_dtype == SITU_DTYPE_BF16 ? situ::IO_BF16 : situ::IO_F32;
    L.out_io = out_dtype == SITU_DTYPE_BF16 ? situ::IO_BF16 : situ::IO_F32;
    L.vec = (!blocks || aligned16(blocks)) && (!prefix || aligned16(prefix)) && aligned16(out) &&
            aligned16(norm_weight) && aligned16(proj_weight) && (hidden * es) % 16 == 0 &&
            hidden * 4 < ((int64_t)1 << 31);
    const int err = situ::launch_attn_res(L, stream);
    if (err)
        return fail(SITU_ERR_DEVICE, "attention-residual launch failed: %s", situ::device_error_string(err));
    return SITU_OK;
}

}  // extern "C"

namespace {

// Shared validation and launch of the fused grouped forward.  op 0: bf16 x
// and weight; 1 / 2: MX E4M3 / E5M2 codes with scale bytes (one per 32
// values along the hidden axis).
int grouped_fwd(int op, const void *x, const void *x_scales, int64_t rows, int64_t hidden, const void *weight,
                const void *w_scales, int64_t experts, int64_t intermediate, const int32_t *group_offsets,
                const void *routing_weights, int rw_dtype, int64_t rw_rows, double beta, const double *linear_beta,
                void *out, void *gate_up_out, void *workspace, size_t workspace_bytes, void *stream)
{
    const int64_t kstep = op ? 128 : 64;     // hidden elements of one pipeline stage
    const int64_t es = op ? 1 : 2;           // bytes per operand element
    int rc = check_common(x, SITU_DTYPE_BF16, rows, intermediate, routing_weights, rw_dtype, rw_rows, beta,
                          linear_beta);
    if (rc)
        return rc;
    if (hidden < 0 || experts < 0)
        return fail(SITU_ERR_INVALID_ARG, "negative size (hidden=%lld, experts=%lld)", (long long)hidden,
                    (long long)experts);
    if (rows == 0 || intermediate == 0)
        return SITU_OK;
    if (experts < 1 || experts > SITU_GROUPED_MAX_EXPERTS)
        return fail(SITU_ERR_INVALID_ARG, "experts must be 1 to %d (got %lld)", SITU_GROUPED_MAX_EXPERTS,
                    (long long)experts);
    if (hidden < kstep || hidden % kstep || hidden > SITU_GROUPED_MAX_HIDDEN)
        return fail(SITU_ERR_UNSUPPORTED, "hidden must be a positive multiple of %lld up to %d (got %lld)",
                    (long long)kstep, SITU_GROUPED_MAX_HIDDEN, (long long)hidden);
    if (intermediate % 128 || intermediate > SITU_GROUPED_MAX_INTERMEDIATE)
        return fail(SITU_ERR_UNSUPPORTED, "intermediate must be a multiple of 128 up to %d (got %lld)",
                    SITU_GROUPED_MAX_INTERMEDIATE, (long long)intermediate);
    if (situ::grouped_grid_blocks(rows, experts, intermediate) > (int64_t)0x7fffffff)
        return fail(SITU_ERR_UNSUPPORTED, "rows %lld, experts %lld and intermediate %lld need more than 2^31 - 1 "
                    "workgroups", (long long)rows, (long long)experts, (long long)intermediate);
    if (!weight || !group_offsets || !out)
        return fail(SITU_ERR_INVALID_ARG, "weight, group_offsets or out is NULL");
    const int64_t nk = hidden / 128, wrows = experts * 2 * intermediate;
    const int64_t xst = situ::grouped_mx_stage_stride(rows), wst = situ::grouped_mx_stage_stride(wrows);
    if (op && (xst * nk >= ((int64_t)1 << 30) || wst * nk >= ((int64_t)1 << 30)))
        return fail(SITU_ERR_UNSUPPORTED, "(rows + 64) * hidden / 128 and (experts * 2 * intermediate + 64) * "
                    "hidden / 128 must be below 2^30 on MXFP8 operands (got %lld and %lld)",
                    (long long)(xst * nk), (long long)(wst * nk));
    if (op && (!x_scales || !w_scales))
        return fail(SITU_ERR_INVALID_ARG, "x_scales or w_scales is NULL");
    const int64_t need = op ? situ::grouped_mx_scale_bytes(rows, hidden) + situ::grouped_mx_scale_bytes(wrows, hidden)
                            : 0;
    if (op && (!workspace || workspace_bytes < (size_t)need))
        return fail(SITU_ERR_INVALID_ARG, "workspace of %zu bytes at %p, %lld bytes needed", workspace_bytes,
                    workspace, (long long)need);
    if (op && !aligned16(workspace))
        return fail(SITU_ERR_INVALID_ARG, "workspace must be 16-byte aligned");
    if (!aligned16(x) || !aligned16(weight) || !aligned16(out) || (gate_up_out && !aligned16(gate_up_out)))
        return fail(SITU_ERR_INVALID_ARG, "x, weight, out and gate_up_out must be 16-byte aligned");
    if (op && (!aligned_to(x_scales, 4) || !aligned_to(w_scales, 4)))
        return fail(SITU_ERR_INVALID_ARG, "x_scales and w_scales must be 4-byte aligned");
    if (!aligned_to(group_offsets, 4))
        return fail(SITU_ERR_INVALID_ARG, "group_offsets is not 4-byte aligned");
    const int64_t sb = hidden / 32;
    const Range outs[] = {range("out", out, rows * intermediate * 2),
                          range("gate_up_out", gate_up_out, gate_up_out ? rows * intermediate * 4 : 0),
                          range("workspace", workspace, need)};
    const Range ins[] = {range("x", x, rows * hidden * es),
                         range("weight", weight, experts * 2 * intermediate * hidden * es),
                         range("x_scales", x_scales, op ? rows * sb : 0),
                         range("w_scales", w_scales, op ? experts * 2 * intermediate * sb : 0),
                         range("group_offsets", group_offsets, (experts + 1) * 4),
                         range("routing_weights", routing_weights, rw_rows * dtype_bytes(rw_dtype))};
    for (const Range &o : outs)
        for (const Range &i : ins)
            if (overlaps(o, i))
                return fail(SITU_ERR_INVALID_ARG, "%s overlaps input %s", o.name, i.name);
    for (int a = 0; a < 3; ++a)
        for (int b = a + 1; b < 3; ++b)
            if (overlaps(outs[a], outs[b]))
                return fail(SITU_ERR_INVALID_ARG, "%s overlaps %s", outs[a].name, outs[b].name);

    situ::GroupedLaunch L{};
    L.op = op;
    L.x = x;
    L.w = weight;
    L.x_scales = x_scales;
    L.w_scales = w_scales;
    L.offsets = group_offsets;
    L.rows = rows;
    L.hidden = (int)hidden;
    L.experts = (int)experts;
    L.inter = (int)intermediate;
    L.rw = routing_weights;
    L.rw_bf16 = rw_dtype == SITU_DTYPE_BF16;
    L.rw_stride = rw_rows == rows ? 1 : 0;
    L.out = out;
    L.gate_up = gate_up_out;
    L.lb = linear_beta != nullptr;
    L.fast = beta == 4.0;
    L.gk = gate_consts(beta);
    L.uk = situ::make_up_consts(linear_beta ? *linear_beta : 1.0);
    L.workspace = op ? workspace : nullptr;
    const int err = situ::launch_grouped_fwd(L, stream);
    if (err)
        return fail(SITU_ERR_DEVICE, "grouped GEMM launch failed: %s", situ::device_error_string(err));
    return SITU_OK;
}

}  // namespace

extern "C" {

int situ_glu_grouped_fwd(const void *x, int io_dtype, int64_t rows, int64_t hidden, const void *weight,
                         int64_t experts, int64_t intermediate, const int32_t *group_offsets,
                         const void *routing_weights, int rw_dtype, int64_t rw_rows, double beta,
                         const double *linear_beta, void *out, void *gate_up_out, void *stream)
{
    g_last_error.clear();
    if (io_dtype != SITU_DTYPE_BF16)
        return fail(SITU_ERR_UNSUPPORTED, "the grouped GEMM takes bf16 x and weight only (io_dtype %d)", io_dtype);
    return grouped_fwd(0, x, nullptr, rows, hidden, weight, nullptr, experts, intermediate, group_offsets,
                       routing_weights, rw_dtype, rw_rows, beta, linear_beta, out, gate_up_out, nullptr, 0, stream);
}

size_t situ_glu_grouped_fwd_mxfp8_workspace_bytes(int64_t rows, int64_t hidden, int64_t experts,
                                                  int64_t intermediate)
{
    if (rows < 0 || hidden < 0 || experts < 0 || intermediate < 0 || hidden > SITU_GROUPED_MAX_HIDDEN ||
        experts > SITU_GROUPED_MAX_EXPERTS || intermediate > SITU_GROUPED_MAX_INTERMEDIATE ||
        rows > (int64_t)0x7fffffff)
        return 0;
    return (size_t)(situ::grouped_mx_scale_bytes(rows, hidden) +
                    situ::grouped_mx_scale_bytes(experts * 2 * intermediate, hidden));
}

int situ_glu_grouped_fwd_mxfp8(const void *x_codes, const void *x_scales, int64_t rows, int64_t hidden,
                               const void *w_codes, const void *w_scales, int64_t experts, int64_t intermediate,
                               int fp8_format, const int32_t *group_offsets, const void *routing_weights,
                               int rw_dtype, int64_t rw_rows, double beta, const double *linear_beta, void *out,
                               void *gate_up_out, void *workspace, size_t workspace_bytes, void *stream)
{
    g_last_error.clear();
    if (fp8_format != SITU_FP8_E4M3 && fp8_format != SITU_FP8_E5M2)
        return fail(SITU_ERR_INVALID_ARG, "fp8_format %d is not SITU_FP8_E4M3 (0) or SITU_FP8_E5M2 (1)",
                    fp8_format);
    return grouped_fwd(fp8_format == SITU_FP8_E4M3 ? 1 : 2, x_codes, x_scales, rows, hidden, w_codes, w_scales,
                       experts, intermediate, group_offsets, routing_weights, rw_dtype, rw_rows, beta, linear_beta,
                       out, gate_up_out, workspace, workspace_bytes, stream);
}

}  // extern "C"
