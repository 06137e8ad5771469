// Device-side building blocks shared by the HIP kernels of the library:
// buffer-descriptor io, bf16 / fp32 unpacking, the per-element SiTU-GLU math
// and wavefront reductions.  Included by the .hip sources only.
//
// Math of the element functions (Megatron-LM PR "[Dev] Add SiTU-GLU through
// Transformer Engine", section "Activation"; NeMo AutoModel "kimi_k3.situ"
// page, `_situ_fwd_core` and `_situ_bwd_core`), with a = |G|,
// e1 = exp(-2a/b1), e2 = exp(-a), nt = 1 - e1, A = 1 + e1, B = 1 + e2:
//   tanh(a/b1) = nt / A,  sech^2(G/b1) = 4 e1 / A^2,
//   sigmoid(G) = sn / B,  sigmoid(-G) = snc / B,
//     with (sn, snc) = (1, e2) for G >= 0 and (e2, 1) for G < 0,
//   T_g   = b1 sgn(G) nt sn / (A B)
//   T_g'  = 4 sn [e1 B + (b1/4) sgn(G) (1 - e1^2) snc] / (A B)^2
// and for the up branch v = exp(-2|U|/b2), C = 1 + v, nu = 1 - v:
//   T_u = b2 sgn(U) nu / C,  T_u' = 4 v / C^2.
// One reciprocal of A B C serves every quotient of an element.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "situ_glu_internal.h"

namespace situ {
namespace {

constexpr int kMaxWaves = 16;           // wavefronts per workgroup
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.69314718055994531f;

__device__ __forceinline__ float ex2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float rcp(float x) { return __builtin_amdgcn_rcpf(x); }

// ---------------------------------------------------------------- buffer io
// The 128-bit path addresses each half row through a buffer descriptor (base
// = the half row, size = its bytes).  The hardware range check returns zeros
// for loads past the end and drops stores past it, so a wavefront runs its
// unrolled strip without per-vector guards.  Every access carries the
// non-temporal hint: each byte is touched exactly once.
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
using rsrc_t = __amdgpu_buffer_rsrc_t;
constexpr int kRsrcWord3 = 0x00020000;  // raw (untyped) buffer, 32-bit data format
constexpr int kStreaming = 2;           // cache policy operand: nt

__device__ __forceinline__ rsrc_t make_rsrc(const void *p, uint32_t bytes)
{
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(p), (short)0, (int)bytes, kRsrcWord3);
}
__device__ __forceinline__ uint4 bload(rsrc_t r, uint32_t off)
{
    const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, kStreaming);
    return make_uint4(v.x, v.y, v.z, v.w);
}
__device__ __forceinline__ void bstore(rsrc_t r, uint32_t off, const uint4 &x)
{
    const u32x4 v = {x.x, x.y, x.z, x.w};
    __builtin_amdgcn_raw_buffer_store_b128(v, r, (int)off, 0, kStreaming);
}

// ---------------------------------------------------------------- bf16 / f32 io
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ float bf_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }
__device__ __forceinline__ uint32_t pack_bf16(float lo, float hi)
{
    bf16x2 v = {(__bf16)lo, (__bf16)hi};   // round to nearest even
    return __builtin_bit_cast(uint32_t, v);
}
__device__ __forceinline__ float bf16_to_f32(uint16_t h) { return __uint_as_float((uint32_t)h << 16); }
__device__ __forceinline__ uint16_t f32_to_bf16(float f)
{
    __bf16 b = (__bf16)f;
    return __builtin_bit_cast(uint16_t, b);
}

template <int IO> struct Io;
template <> struct Io<IO_BF16> {
    static constexpr int kPerVec = 8;
    static constexpr int kBytes = 2;
    __device__ static void unpack(const uint4 &w, float *x)
    {
        const uint32_t a[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            x[2 * i] = bf_lo(a[i]);
            x[2 * i + 1] = bf_hi(a[i]);
        }
    }
    __device__ static uint4 pack(const float *x)
    {
        return make_uint4(pack_bf16(x[0], x[1]), pack_bf16(x[2], x[3]),
                          pack_bf16(x[4], x[5]), pack_bf16(x[6], x[7]));
    }
    __device__ static float load1(const void *p, int64_t i)
    {
        return bf16_to_f32(static_cast<const uint16_t *>(p)[i]);
    }
    __device__ static void store1(void *p, int64_t i, float v)
    {
        static_cast<uint16_t *>(p)[i] = f32_to_bf16(v);
    }
};
template <> struct Io<IO_F32> {
    static constexpr int kPerVec = 4;
    static constexpr int kBytes = 4;
    __device__ static void unpack(const uint4 &w, float *x)
    {
        x[0] = __uint_as_float(w.x);
        x[1] = __uint_as_float(w.y);
        x[2] = __uint_as_float(w.z);
        x[3] = __uint_as_float(w.w);
    }
    __device__ static uint4 pack(const float *x)
    {
        return make_uint4(__float_as_uint(x[0]), __float_as_uint(x[1]),
                          __float_as_uint(x[2]), __float_as_uint(x[3]));
    }
    __device__ static float load1(const void *p, int64_t i) { return static_cast<const float *>(p)[i]; }
    __device__ static void store1(void *p, int64_t i, float v) { static_cast<float *>(p)[i] = v; }
};

__device__ __forceinline__ float load_rw(const void *rw, int rw_bf16, int64_t i)
{
    return rw_bf16 ? bf16_to_f32(static_cast<const uint16_t *>(rw)[i])
                   : static_cast<const float *>(rw)[i];
}

// ---------------------------------------------------------------- element math

// s * (1 - exp(-y)) for y = zk z ln2 >= 0, given e = exp(-y) as rounded by the
// exponential (zk is 1 or 2, a compile-time constant).  For small y the
// subtraction 1 - e loses relative accuracy (v_exp_f32 is within 0.77 ulp, so
// the error is ~5e-8/y); there the Taylor series of 1 - exp(-y) is used
// instead.  PRECISE (fp32 io) keeps five terms below y = 1/16 (truncation
// < 2e-9 relative, subtraction error above < 1e-6); otherwise the first term
// below y = 2^-11 (truncation y/2 <= 2.4e-4, subtraction error above
// <= 1e-4), both well inside half a bf16 ulp (2^-9).  The scale s rides on
// both branches: s (1 - e) = fma(-e, s, s).
template <bool PRECISE, int ZK>
__device__ __forceinline__ float scaled_one_minus_exp2_neg(float z, float e, float s)
{
    if (PRECISE) {
        const float y = z * (ZK * kLn2);
        const float p = y * (1.0f - y * (0.5f - y * (1.0f / 6.0f - y * (1.0f / 24.0f - y * (1.0f / 120.0f)))));
        return y < 0.0625f ? s * p : fmaf(-e, s, s);
    } else {
        const float p = z * ((ZK * kLn2) * s);
        return z < (0.00048828125f / (ZK * kLn2)) ? p : fmaf(-e, s, s);
    }
}

struct Gate {
    float e1, e2, nt;
    float h;      // exp(-|G| / 2): e2 = h * h
    float sn_s;   // sgn(G) * sigmoid numerator: G < 0 ? -e2 : 1
    float snc_s;  // sgn(G) * sigmoid(-G) numerator: G < 0 ? -1 : e2
};

// Gate-branch pieces; nt is scaled by ntscale.
template <bool FAST, bool PRECISE>
__device__ __forceinline__ Gate gate_parts(float g, float ntscale, const GateK &k)
{
    Gate o;
    const float a = fabsf(g);
    const float z = a * (FAST ? 0.5f * kLog2e : k.k1);  // e1 = 2^-z = exp(-2a/b1)
    o.e1 = ex2(-z);
    if (FAST) {
        o.h = o.e1;
        o.e2 = o.e1 * o.e1;
    } else {
        // exp(-a) as the square of exp(-a/2): keeps gradual underflow to a ~ 174
        o.h = ex2(a * (-0.5f * kLog2e));
        o.e2 = o.h * o.h;
    }
    o.nt = scaled_one_minus_exp2_neg<PRECISE, 1>(z, o.e1, ntscale);
    const bool neg = g < 0.0f;
    o.sn_s = neg ? -o.e2 : 1.0f;
    o.snc_s = neg ? -1.0f : o.e2;
    return o;
}

// fp32 io, G < 0 with e2 = exp(G) below fp32's normal range: Y = -(nt h)
// (rest) h, the sigmoid numerator's two factors h multiplied into the
// already scaled product one at a time, so that Y is rounded once in the
// subnormal range rather than e2 first and that error then scaled.
template <bool PRECISE>
__device__ __forceinline__ float gate_times(const Gate &t, float g, float rest)
{
    const float y = (t.nt * t.sn_s) * rest;
    if (!PRECISE)
        return y;
    const float ys = -(((t.nt * t.h) * rest) * t.h);
    return g < 0.0f && t.e2 < 1.17549435e-38f ? ys : y;
}

// Y = r T_g T_u: rscale = r b1 b2 (r b1 without linear beta) rides on nt.
template <bool LB, bool FAST, bool PRECISE>
__device__ __forceinline__ float fwd_elem(float g, float u, float rscale, const GateK &gk, const UpK &uk)
{
    const Gate t = gate_parts<FAST, PRECISE>(g, rscale, gk);
    const float a = 1.0f + t.e1;
    const float m = fmaf(t.e2, a, a);  // (1 + e1)(1 + e2)
    if (LB) {
        const float z = fabsf(u) * uk.ku;  // v = 2^-z = exp(-2|U|/b2)
        const float v = ex2(-z);
        const float nu = copysignf(scaled_one_minus_exp2_neg<PRECISE, 1>(z, v, 1.0f), u);
        const float q = rcp(fmaf(m, v, m));  // 1 / ((1 + e1)(1 + e2)(1 + v))
        return gate_times<PRECISE>(t, g, nu * q);
    } else {
        const float q = rcp(m);
        return gate_times<PRECISE>(t, g, u * q);
    }
}

// tanh(U / b2) for |U| <= b2 / 4 as U P(U^2), the powers of 1/b2 folded
// into P (UpK): the odd Taylor series of tanh through x^5 (DEG 5: the first
// dropped term, 17 x^7 / 315, stays below 1.4e-5 of tanh there) or through
// x^7 (DEG 7: below 3.3e-7).  No exponential, no reciprocal and no
// cancellation for small U.
template <int DEG>
__device__ __forceinline__ float tanh_up(float u, const UpK &k)
{
    static_assert(DEG == 5 || DEG == 7, "degree 5 or 7");
    const float w = u * u;
    float p = DEG == 7 ? fmaf(k.p7, w, k.p5) : k.p5;
    p = fmaf(p, w, k.p3);
    p = fmaf(p, w, k.p1);
    return u * p;
}

// tanh(x) for |x| <= 1/4: the odd Taylor polynomial through x^9 (tanh's
// series x - x^3/3 + 2x^5/15 - 17x^7/315 + 62x^9/2835 - ...; the first term
// dropped is below 1e-8 of tanh there; fp32 evaluation adds ~3 ulp).  The
// backward's form (x = U / b2): measured faster there than tanh_up.
__device__ __forceinline__ float tanh_small(float x)
{
    const float x2 = x * x;
    const float p = fmaf(fmaf(fmaf(62.0f / 2835.0f, x2, -17.0f / 315.0f), x2, 2.0f / 15.0f), x2, -1.0f / 3.0f);
    return fmaf(x * x2, p, x);
}

// Forward with the up branch as tanh_up (bf16 io, |U| <= b2 / 4): one
// reciprocal of (1 + e1)(1 + e2) only.  Degree 5 is ample for a bf16 result
// (its ulp is 2^-8 relative); an fp32 Y that is quantised further (MXFP8)
// takes degree 7, inside the fp32 chain's 1e-5.
template <bool FAST, int DEG = 5>
__device__ __forceinline__ float fwd_elem_small_u(float g, float u, float rscale, const GateK &gk, const UpK &uk)
{
    const Gate t = gate_parts<FAST, false>(g, rscale, gk);
    const float a = 1.0f + t.e1;
    const float q = rcp(fmaf(t.e2, a, a));  // 1 / ((1 + e1)(1 + e2))
    return (t.nt * t.sn_s) * (tanh_up<DEG>(u, uk) * q);
}

// dT_g/dG / 4 near its root, where its two terms cancel.  fp32 io: the
// degree-7 Taylor polynomial in d = G - G*_f32 inside the window.  bf16 io: G
// is a bf16 value, and
// only the one nearest the root loses more than ~3e-5 to the cancellation;
// that value gets its exact dT_g/dG / 4.  `plain` elsewhere.
template <bool PRECISE>
__device__ __forceinline__ float gate_grad4_window(float g, float plain, const GateK &k)
{
    if (PRECISE) {
        const float d = g - k.win_ghi;  // exact (Sterbenz) inside the window
        float p = 0.25f * k.c7;
        p = fmaf(p, d, 0.25f * k.c6);
        p = fmaf(p, d, 0.25f * k.c5);
        p = fmaf(p, d, 0.25f * k.c4);
        p = fmaf(p, d, 0.25f * k.c3);
        p = fmaf(p, d, 0.25f * k.c2);
        p = fmaf(p, d, 0.25f * k.c1);
        p = fmaf(p, d, 0.25f * k.c0);
        return fabsf(d) <= k.win_hw ? p : plain;
    } else {
        return g == k.gsub ? k.tsub : plain;
    }
}

struct BwdOut {
    float dg, du, p;  // p = go T_g T_u / (b1 b2) (/ b1 without linear beta)
};

// cG = 4 r b2 (4 r without linear beta), cU = 4 r b1 (r b1 without).
// With m = (1 + e1)(1 + e2) = A B, q = 1 / (m C), a1 = nt sn and X = go q:
//   T_g / b1 = a1 q C,  T_u / b2 = nu q m,  T_u' / 4 = v (q m)^2,
// and since q m C = 1:
//   go T_g T_u / (b1 b2) = X a1 nu,  dU = X a1 v (q m) cU,
//   dG = go nu (q m) (T_g' / 4) cG,  T_g' / 4 = |sn| br (q C)^2.
// FOLD (no routing-weight gradient, so p is not needed): cU rides on nt and
// cG on nu (linear beta), one multiply fewer per gradient.
template <bool LB, bool FAST, bool PRECISE, bool FOLD = false>
__device__ __forceinline__ BwdOut bwd_elem(float g, float u, float go, float cG, float cU,
                                           const GateK &gk, const UpK &uk)
{
    BwdOut o;
    const Gate t = gate_parts<FAST, PRECISE>(g, FOLD ? cU : 1.0f, gk);
    // T_g' / (4 sn) * (A B)^2 = e1 B + (b1/4) sgn(G) (1 - e1^2) snc, e1 B = e1 + e1 e2
    const float om = FAST ? 1.0f - t.e2 : (0.25f * gk.beta1) * fmaf(-t.e1, t.e1, 1.0f);
    const float e1B = fmaf(t.e1, t.e2, t.e1);
    const float br = fmaf(om, t.snc_s, e1B);
    const float sbr = fabsf(t.sn_s) * br;
    const float m = (1.0f + t.e2) + e1B;
    const float a1 = t.nt * t.sn_s;
    if (LB) {
        // exp(-2|U|/b2) as the square of exp(-|U|/b2): gradual underflow of T_u'
        const float z = fabsf(u) * (0.5f * uk.ku);
        const float h = ex2(-z);
        const float v = h * h;
        const float nu = copysignf(scaled_one_minus_exp2_neg<PRECISE, 2>(z, v, FOLD ? cG : 1.0f), u);
        const float C = 1.0f + v;
        const float q = rcp(m * C);
        const float iab = q * C;                 // 1 / (A B)
        const float ic = q * m;                  // 1 / C
        const float tgp = gate_grad4_window<PRECISE>(g, sbr * (iab * iab), gk);  // T_g' / 4
        const float xa1 = (go * q) * a1;
        o.p = xa1 * nu;
        o.du = FOLD ? xa1 * v * ic : xa1 * v * ic * cU;
        o.dg = FOLD ? go * nu * ic * tgp : go * nu * ic * tgp * cG;
    } else {
        const float q = rcp(m);
        const float tgp = gate_grad4_window<PRECISE>(g, sbr * (q * q), gk);
        const float z1 = go * (a1 * q);          // go T_g / b1
        o.p = z1 * u;
        o.du = FOLD ? z1 : z1 * cU;
        o.dg = go * u * tgp * cG;
    }
    return o;
}

// Backward with the up branch as t = tanh_small(U / b2) (bf16 io,
// |U| <= b2 / 4): T_u = b2 t, T_u' = 1 - t^2, and with q = 1 / ((1 + e1)(1 + e2)):
//   go T_g T_u / (b1 b2) = go a1 q t,  dU = go a1 q (1 - t^2) cU / 4,
//   dG = go t (T_g' / 4) cG,  T_g' / 4 = |sn| br q^2.
// FOLD: cU / 4 rides on nt (no routing-weight gradient).
template <bool FAST, bool FOLD>
__device__ __forceinline__ BwdOut bwd_elem_small_u(float g, float u, float go, float cG, float cU4, const GateK &gk,
                                                   const UpK &uk)
{
    BwdOut o;
    const Gate t = gate_parts<FAST, false>(g, FOLD ? cU4 : 1.0f, gk);
    const float om = FAST ? 1.0f - t.e2 : (0.25f * gk.beta1) * fmaf(-t.e1, t.e1, 1.0f);
    const float e1B = fmaf(t.e1, t.e2, t.e1);
    const float br = fmaf(om, t.snc_s, e1B);
    const float sbr = fabsf(t.sn_s) * br;
    const float q = rcp((1.0f + t.e2) + e1B);
    const float tgp = gate_grad4_window<false>(g, sbr * (q * q), gk);
    const float tu = tanh_small(u * uk.inv_b2);
    const float s2 = fmaf(-tu, tu, 1.0f);
    const float gqa = (go * q) * (t.nt * t.sn_s);
    o.p = gqa * tu;
    o.du = FOLD ? gqa * s2 : gqa * s2 * cU4;
    o.dg = go * tu * tgp * cG;
    return o;
}

// True on every lane when no |U| of the wavefront's values exceeds the
// polynomial's range (NaN counts as in range: it propagates either way).
template <int E>
__device__ __forceinline__ bool wave_up_small(const float *u, const UpK &uk)
{
    float m = fabsf(u[0]);
#pragma unroll
    for (int e = 1; e < E; ++e)
        m = fmaxf(m, fabsf(u[e]));
    return __builtin_amdgcn_ballot_w64(!(m <= uk.small_max) && m == m) == 0;
}

// ---------------------------------------------------------------- reductions

template <int CTRL>
__device__ __forceinline__ float dpp_f(float x)
{
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xf, 0xf, false));
}

// Sum over the 64 lanes of a wavefront in a fixed order: DPP butterflies
// inside each row of 16 lanes (xor 1, xor 2, half-row mirror, row mirror),
// then the four row sums added in lane order.  Every lane of a row holds the
// same value after each step because IEEE addition commutes.
__device__ __forceinline__ float wave_sum(float x)
{
    x += dpp_f<0xB1>(x);   // quad_perm [1,0,3,2]
    x += dpp_f<0x4E>(x);   // quad_perm [2,3,0,1]
    x += dpp_f<0x141>(x);  // row_half_mirror
    x += dpp_f<0x140>(x);  // row_mirror
    const float r0 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), 0));
    const float r1 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), 16));
    const float r2 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), 32));
    const float r3 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), 48));
    return (r0 + r1) + (r2 + r3);
}

// Writes one row's d_routing_weights (one weight per row) or its fp32
// partial (one broadcast weight: a second launch adds the partials).
__device__ __forceinline__ void write_row_dr(float s, int64_t row, int64_t rw_stride, int rw_bf16, void *d_rw,
                                             float *row_partials)
{
    if (rw_stride == 0)
        row_partials[row] = s;
    else if (rw_bf16)
        static_cast<uint16_t *>(d_rw)[row] = f32_to_bf16(s);
    else
        static_cast<float *>(d_rw)[row] = s;
}

// ---------------------------------------------------------------- kernels
//
// 128-bit path.  blockDim.x = 64 * rows_per_block * waves_per_row; wavefront
// w of the block works on row blockIdx.x * rows_per_block + w / waves_per_row
// and takes strips w % waves_per_row, + waves_per_row, ... of it.

struct Place {
    int64_t row;
    int strip0;  // first strip of this wavefront
    int wpr;     // wavefronts per row (strip stride)
    int slot;    // wavefront index inside the block
};

__device__ __forceinline__ Place place(int waves_per_row)
{
    Place p;
    p.slot = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int rows_per_block = (int)(blockDim.x >> 6) / waves_per_row;
    p.row = (int64_t)blockIdx.x * rows_per_block + p.slot / waves_per_row;
    p.strip0 = p.slot % waves_per_row;
    p.wpr = waves_per_row;
    return p;
}

// ---------------------------------------------------------------- launch shape

// Launch shape.  128-bit path: a row of `spr` strips gets min(spr, 16)
// wavefronts; rows of one strip are packed rows_per_block to a workgroup.
// Element path: one wavefront per row, four rows per workgroup.
struct Shape {
    dim3 grid, block;
    int waves_per_row;
};

[[maybe_unused]] Shape shape(int64_t rows, int inter, int io, int vec, int rows_per_block, int unroll)
{
    const int kStrip = 64 * unroll;
    Shape s;
    if (!vec) {
        s.waves_per_row = 1;
        s.block = dim3(256);
        s.grid = dim3((unsigned)((rows + 3) / 4));
        return s;
    }
    const int64_t nv = inter / (io == IO_BF16 ? 8 : 4);
    const int64_t spr = (nv + kStrip - 1) / kStrip;
    const int wpr = (int)(spr < kMaxWaves ? spr : kMaxWaves);
    int rpb = wpr == 1 ? (rows_per_block > 0 ? rows_per_block : 1) : 1;
    if (rpb * wpr > kMaxWaves)
        rpb = kMaxWaves / wpr;
    s.waves_per_row = wpr;
    s.block = dim3((unsigned)(64 * wpr * rpb));
    s.grid = dim3((unsigned)((rows + rpb - 1) / rpb));
    return s;
}

}  // namespace
}  // namespace situ
