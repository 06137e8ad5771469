// Weighted SiTU-GLU forward / backward kernels for CDNA4 (gfx950).
//
// Operation (Megatron-LM PR "[Dev] Add SiTU-GLU through Transformer Engine",
// section "Activation"; NeMo AutoModel "kimi_k3.situ" page, `_situ_fwd_core`
// and `_situ_bwd_core`):
//   T_g = b1 tanh(G/b1) sigmoid(G),  T_u = b2 tanh(U/b2) (or U),  Y = r T_g T_u
// Backward recomputes everything from the saved inputs (the page's autograd
// Function keeps only the low-precision inputs) and returns dG, dU and the
// per-row reduction dr = sum_j go T_g T_u.
//
// Memory-bound elementwise work, no contraction, so no MFMA.  Layout of the
// work: one workgroup per group of rows; a row is cut into strips of
// 64 lanes x kUnroll 128-bit vectors of each half row, and each wavefront
// owns one strip at a time (long rows get several wavefronts, whose dr
// partials meet in LDS).  Loads and stores go through buffer descriptors
// with the non-temporal hint.
//
// Math, with a = |G|, e1 = exp(-2a/b1), e2 = exp(-a), nt = 1 - e1,
// A = 1 + e1, B = 1 + e2 (all cancellation free except nt, see below):
//   tanh(a/b1) = nt / A,  sech^2(G/b1) = 4 e1 / A^2,
//   sigmoid(G) = sn / B,  sigmoid(-G) = snc / B,
//     with (sn, snc) = (1, e2) for G >= 0 and (e2, 1) for G < 0,
//   T_g   = b1 sgn(G) nt sn / (A B)
//   T_g'  = 4 sn [e1 B + (b1/4) sgn(G) (1 - e1^2) snc] / (A B)^2
// and for the up branch v = exp(-2|U|/b2), C = 1 + v, nu = 1 - v:
//   T_u = b2 sgn(U) nu / C,  T_u' = 4 v / C^2.
// One reciprocal of A B C serves every quotient of an element.
// For b1 = 4, e1 = exp(-a/2) and e2 = e1^2: one exponential for the gate.
// nt = 1 - exp(-y) cancels for small y; there its Taylor series is used.
// T_g' cancels near its root G* < 0; there a polynomial in G - G* (built on
// the host for the given b1) replaces it.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "situ_glu_internal.h"

namespace situ {
namespace {

// 128-bit vectors in flight per lane and input stream; a wavefront's strip
// is 64 lanes x unroll vectors of each half row.  Measured on MI355X: 4 for
// the forward (2 input streams) and 2 for the backward (3 input streams,
// which then fits in 64 VGPRs: 8 wavefronts per SIMD).
#ifndef SITU_UNROLL_FWD
#define SITU_UNROLL_FWD 4
#endif
#ifndef SITU_UNROLL_BWD
#define SITU_UNROLL_BWD 2
#endif
constexpr int kUnrollFwd = SITU_UNROLL_FWD;
constexpr int kUnrollBwd = SITU_UNROLL_BWD;
constexpr int kMaxWaves = 16;           // wavefronts per workgroup
#ifndef SITU_BWD_MIN_WAVES
#define SITU_BWD_MIN_WAVES 8  // wavefronts per SIMD the backward must fit (<= 64 VGPRs)
#endif
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
        o.e2 = o.e1 * o.e1;
    } else {
        // exp(-a) as the square of exp(-a/2): keeps gradual underflow to a ~ 174
        const float h = ex2(a * (-0.5f * kLog2e));
        o.e2 = h * h;
    }
    o.nt = scaled_one_minus_exp2_neg<PRECISE, 1>(z, o.e1, ntscale);
    const bool neg = g < 0.0f;
    o.sn_s = neg ? -o.e2 : 1.0f;
    o.snc_s = neg ? -1.0f : o.e2;
    return o;
}

// Y = r T_g T_u: rscale = r b1 b2 (r b1 without linear beta) rides on nt.
template <bool LB, bool FAST, bool PRECISE>
__device__ __forceinline__ float fwd_elem(float g, float u, float rscale, const GateK &gk, const UpK &uk)
{
    const Gate t = gate_parts<FAST, PRECISE>(g, rscale, gk);
    const float m = (1.0f + t.e2) + fmaf(t.e1, t.e2, t.e1);  // (1 + e1)(1 + e2)
    if (LB) {
        const float z = fabsf(u) * uk.ku;  // v = 2^-z = exp(-2|U|/b2)
        const float v = ex2(-z);
        const float nu = copysignf(scaled_one_minus_exp2_neg<PRECISE, 1>(z, v, 1.0f), u);
        const float q = rcp(m * (1.0f + v));
        return (t.nt * t.sn_s) * (nu * q);
    } else {
        const float q = rcp(m);
        return (t.nt * t.sn_s) * (u * q);
    }
}

// dT_g/dG / 4 near its root: polynomial in d = G - G*_f32 inside the window
// (cubic for fp32 io, quadratic for bf16 io); `plain` elsewhere.
template <bool PRECISE>
__device__ __forceinline__ float gate_grad4_window(float g, float plain, const GateK &k)
{
    const float d = g - k.win_ghi;  // exact (Sterbenz) inside the window
    if (PRECISE) {
        const float p = fmaf(fmaf(fmaf(0.25f * k.c3, d, 0.25f * k.c2), d, 0.25f * k.c1), d, 0.25f * k.c0);
        return fabsf(d) <= k.win_hw ? p : plain;
    } else {
        const float p = fmaf(fmaf(0.25f * k.c2, d, 0.25f * k.c1), d, 0.25f * k.c0);
        return fabsf(d) <= k.win_hw2 ? p : plain;
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
template <bool LB, bool FAST, bool PRECISE>
__device__ __forceinline__ BwdOut bwd_elem(float g, float u, float go, float cG, float cU,
                                           const GateK &gk, const UpK &uk)
{
    BwdOut o;
    const Gate t = gate_parts<FAST, PRECISE>(g, 1.0f, gk);
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
        const float nu = copysignf(scaled_one_minus_exp2_neg<PRECISE, 2>(z, v, 1.0f), u);
        const float C = 1.0f + v;
        const float q = rcp(m * C);
        const float iab = q * C;                 // 1 / (A B)
        const float ic = q * m;                  // 1 / C
        const float tgp = gate_grad4_window<PRECISE>(g, sbr * (iab * iab), gk);  // T_g' / 4
        const float xa1 = (go * q) * a1;
        o.p = xa1 * nu;
        o.du = xa1 * v * ic * cU;
        o.dg = go * nu * ic * tgp * cG;
    } else {
        const float q = rcp(m);
        const float tgp = gate_grad4_window<PRECISE>(g, sbr * (q * q), gk);
        const float z1 = go * (a1 * q);          // go T_g / b1
        o.p = z1 * u;
        o.du = z1 * cU;
        o.dg = go * u * tgp * cG;
    }
    return o;
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

template <int IO, bool LB, bool FAST>
__global__ void __launch_bounds__(64 * kMaxWaves)
situ_glu_fwd_vec_kernel(const void *__restrict__ gate_up, const void *__restrict__ rw, int rw_bf16,
                        int64_t rw_stride, void *__restrict__ out, int64_t rows, int inter, int waves_per_row,
                        GateK gk, UpK uk)
{
    constexpr bool PRECISE = IO == IO_F32;
    using T = Io<IO>;
    constexpr int E = T::kPerVec;
    constexpr int kUnroll = kUnrollFwd, kStrip = 64 * kUnroll;
    const int lane = threadIdx.x & 63;
    const Place pl = place(waves_per_row);
    if (pl.row >= rows)
        return;
    const int nv = inter / E;
    const uint32_t half = (uint32_t)nv * 16u;  // bytes of a half row = an output row
    const int spr = (nv + kStrip - 1) / kStrip;
    const char *row = static_cast<const char *>(gate_up) + pl.row * (int64_t)half * 2;
    const rsrc_t rg = make_rsrc(row, half), ru = make_rsrc(row + half, half);
    const rsrc_t ro = make_rsrc(static_cast<char *>(out) + pl.row * (int64_t)half, half);
    const float r = load_rw(rw, rw_bf16, pl.row * rw_stride);
    const float rscale = LB ? r * gk.beta1 * uk.beta2 : r * gk.beta1;
    for (int s = pl.strip0; s < spr; s += pl.wpr) {
        uint4 gv[kUnroll], uv[kUnroll];
#pragma unroll
        for (int k = 0; k < kUnroll; ++k) {
            const uint32_t off = (uint32_t)(s * kStrip + 64 * k + lane) * 16u;
            gv[k] = bload(rg, off);
            uv[k] = bload(ru, off);
        }
#pragma unroll
        for (int k = 0; k < kUnroll; ++k) {
            // past the row end the loads returned zeros and the store is dropped
            const uint32_t off = (uint32_t)(s * kStrip + 64 * k + lane) * 16u;
            float g[E], u[E], y[E];
            T::unpack(gv[k], g);
            T::unpack(uv[k], u);
#pragma unroll
            for (int e = 0; e < E; ++e)
                y[e] = fwd_elem<LB, FAST, PRECISE>(g[e], u[e], rscale, gk, uk);
            bstore(ro, off, T::pack(y));
        }
    }
}

template <int IO, bool LB, bool FAST, bool DR>
__global__ void __launch_bounds__(64 * kMaxWaves, SITU_BWD_MIN_WAVES)
situ_glu_bwd_vec_kernel(const void *__restrict__ gate_up, const void *__restrict__ rw, int rw_bf16,
                        int64_t rw_stride, const void *__restrict__ grad_out, void *__restrict__ d_gate_up,
                        void *__restrict__ d_rw, float *__restrict__ row_partials, int64_t rows, int inter,
                        int waves_per_row, GateK gk, UpK uk)
{
    constexpr bool PRECISE = IO == IO_F32;
    using T = Io<IO>;
    constexpr int E = T::kPerVec;
    constexpr int kUnroll = kUnrollBwd, kStrip = 64 * kUnroll;
    __shared__ float wave_part[kMaxWaves];
    const int lane = threadIdx.x & 63;
    const Place pl = place(waves_per_row);
    const bool live = pl.row < rows;
    float acc = 0.0f;
    if (live) {
        const int nv = inter / E;
        const uint32_t half = (uint32_t)nv * 16u;
        const int spr = (nv + kStrip - 1) / kStrip;
        const char *row = static_cast<const char *>(gate_up) + pl.row * (int64_t)half * 2;
        const rsrc_t rg = make_rsrc(row, half), ru = make_rsrc(row + half, half);
        const rsrc_t rgo = make_rsrc(static_cast<const char *>(grad_out) + pl.row * (int64_t)half, half);
        char *drow = static_cast<char *>(d_gate_up) + pl.row * (int64_t)half * 2;
        const rsrc_t rdg = make_rsrc(drow, half), rdu = make_rsrc(drow + half, half);
        const float r = load_rw(rw, rw_bf16, pl.row * rw_stride);
        const float cG = LB ? 4.0f * r * uk.beta2 : 4.0f * r;
        const float cU = LB ? 4.0f * r * gk.beta1 : r * gk.beta1;
        for (int s = pl.strip0; s < spr; s += pl.wpr) {
            uint4 gv[kUnroll], uv[kUnroll], ov[kUnroll];
#pragma unroll
            for (int k = 0; k < kUnroll; ++k) {
                const uint32_t off = (uint32_t)(s * kStrip + 64 * k + lane) * 16u;
                gv[k] = bload(rg, off);
                uv[k] = bload(ru, off);
                ov[k] = bload(rgo, off);
            }
    #pragma unroll
            for (int k = 0; k < kUnroll; ++k) {
                // past the row end all three loads returned zeros: every term
                // below is then an exact zero and the stores are dropped
                const uint32_t off = (uint32_t)(s * kStrip + 64 * k + lane) * 16u;
                float g[E], u[E], og[E], dg[E], du[E];
                T::unpack(gv[k], g);
                T::unpack(uv[k], u);
                T::unpack(ov[k], og);
#pragma unroll
                for (int e = 0; e < E; ++e) {
                    const BwdOut b = bwd_elem<LB, FAST, PRECISE>(g[e], u[e], og[e], cG, cU, gk, uk);
                    dg[e] = b.dg;
                    du[e] = b.du;
                    if (DR)
                        acc += b.p;
                }
                bstore(rdg, off, T::pack(dg));
                bstore(rdu, off, T::pack(du));
            }
        }
    }
    if (DR) {
        const float scale = LB ? gk.beta1 * uk.beta2 : gk.beta1;
        const float s = wave_sum(acc);
        if (pl.wpr == 1) {
            if (live && lane == 0)
                write_row_dr(s * scale, pl.row, rw_stride, rw_bf16, d_rw, row_partials);
        } else {
            // the row's wavefronts meet in LDS; the first one adds them in order
            if (lane == 0)
                wave_part[pl.slot] = s;
            __syncthreads();
            if (live && pl.strip0 == 0 && lane == 0) {
                float t = 0.0f;
                for (int w = 0; w < pl.wpr; ++w)
                    t += wave_part[pl.slot + w];
                write_row_dr(t * scale, pl.row, rw_stride, rw_bf16, d_rw, row_partials);
            }
        }
    }
}

// Element path (any alignment, any intermediate): one wavefront per row.
template <int IO, bool LB, bool FAST>
__global__ void __launch_bounds__(64 * kMaxWaves)
situ_glu_fwd_elem_kernel(const void *__restrict__ gate_up, const void *__restrict__ rw, int rw_bf16,
                         int64_t rw_stride, void *__restrict__ out, int64_t rows, int inter, int /*unused*/,
                         GateK gk, UpK uk)
{
    constexpr bool PRECISE = IO == IO_F32;
    using T = Io<IO>;
    const int lane = threadIdx.x & 63;
    const int64_t row = (int64_t)blockIdx.x * (blockDim.x >> 6) + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    if (row >= rows)
        return;
    const float r = load_rw(rw, rw_bf16, row * rw_stride);
    const float rscale = LB ? r * gk.beta1 * uk.beta2 : r * gk.beta1;
    const char *gu_row = static_cast<const char *>(gate_up) + row * (int64_t)inter * 2 * T::kBytes;
    char *out_row = static_cast<char *>(out) + row * (int64_t)inter * T::kBytes;
    for (int j = lane; j < inter; j += 64) {
        const float g = T::load1(gu_row, j);
        const float u = T::load1(gu_row, (int64_t)inter + j);
        T::store1(out_row, j, fwd_elem<LB, FAST, PRECISE>(g, u, rscale, gk, uk));
    }
}

template <int IO, bool LB, bool FAST, bool DR>
__global__ void __launch_bounds__(64 * kMaxWaves)
situ_glu_bwd_elem_kernel(const void *__restrict__ gate_up, const void *__restrict__ rw, int rw_bf16,
                         int64_t rw_stride, const void *__restrict__ grad_out, void *__restrict__ d_gate_up,
                         void *__restrict__ d_rw, float *__restrict__ row_partials, int64_t rows, int inter,
                         int /*unused*/, GateK gk, UpK uk)
{
    constexpr bool PRECISE = IO == IO_F32;
    using T = Io<IO>;
    const int lane = threadIdx.x & 63;
    const int64_t row = (int64_t)blockIdx.x * (blockDim.x >> 6) + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    if (row >= rows)
        return;
    const float r = load_rw(rw, rw_bf16, row * rw_stride);
    const float cG = LB ? 4.0f * r * uk.beta2 : 4.0f * r;
    const float cU = LB ? 4.0f * r * gk.beta1 : r * gk.beta1;
    const int64_t in_off = row * (int64_t)inter;
    const char *gu_row = static_cast<const char *>(gate_up) + 2 * in_off * T::kBytes;
    const char *go_row = static_cast<const char *>(grad_out) + in_off * T::kBytes;
    char *dgu_row = static_cast<char *>(d_gate_up) + 2 * in_off * T::kBytes;
    float acc = 0.0f;
    for (int j = lane; j < inter; j += 64) {
        const float g = T::load1(gu_row, j);
        const float u = T::load1(gu_row, (int64_t)inter + j);
        const float o = T::load1(go_row, j);
        const BwdOut b = bwd_elem<LB, FAST, PRECISE>(g, u, o, cG, cU, gk, uk);
        T::store1(dgu_row, j, b.dg);
        T::store1(dgu_row, (int64_t)inter + j, b.du);
        if (DR)
            acc += b.p;
    }
    if (DR) {
        const float s = wave_sum(acc);
        if (lane == 0)
            write_row_dr(s * (LB ? gk.beta1 * uk.beta2 : gk.beta1), row, rw_stride, rw_bf16, d_rw, row_partials);
    }
}

// One workgroup adds the per-row partials in a fixed order: each thread sums
// a strided set of rows in row order, then a fixed tree over the threads.
constexpr int kReduceBlock = 1024;

__global__ void __launch_bounds__(kReduceBlock)
situ_glu_dr_reduce_kernel(const float *__restrict__ row_partials, int64_t rows, void *__restrict__ d_rw,
                          int rw_bf16)
{
    __shared__ float part[kReduceBlock];
    float s = 0.0f;
    for (int64_t i = threadIdx.x; i < rows; i += kReduceBlock)
        s += row_partials[i];
    part[threadIdx.x] = s;
    __syncthreads();
    for (int w = kReduceBlock / 2; w > 0; w >>= 1) {
        if ((int)threadIdx.x < w)
            part[threadIdx.x] += part[threadIdx.x + w];
        __syncthreads();
    }
    if (threadIdx.x == 0) {
        if (rw_bf16)
            *static_cast<uint16_t *>(d_rw) = f32_to_bf16(part[0]);
        else
            *static_cast<float *>(d_rw) = part[0];
    }
}

__global__ void situ_glu_zero_kernel(unsigned char *__restrict__ p, int64_t n)
{
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x)
        p[i] = 0;
}

// ---------------------------------------------------------------- dispatch

using FwdFn = void (*)(const void *, const void *, int, int64_t, void *, int64_t, int, int, GateK, UpK);
using BwdFn = void (*)(const void *, const void *, int, int64_t, const void *, void *, void *, float *,
                       int64_t, int, int, GateK, UpK);

template <int IO, bool VEC, bool LB, bool FAST>
constexpr FwdFn fwd_fn()
{
    if constexpr (VEC)
        return situ_glu_fwd_vec_kernel<IO, LB, FAST>;
    else
        return situ_glu_fwd_elem_kernel<IO, LB, FAST>;
}
template <int IO, bool VEC, bool LB, bool FAST, bool DR>
constexpr BwdFn bwd_fn()
{
    if constexpr (VEC)
        return situ_glu_bwd_vec_kernel<IO, LB, FAST, DR>;
    else
        return situ_glu_bwd_elem_kernel<IO, LB, FAST, DR>;
}

#define SITU_FWD_ROW(IO, VEC)                                                                  \
    { fwd_fn<IO, VEC, false, false>(), fwd_fn<IO, VEC, false, true>(),                        \
      fwd_fn<IO, VEC, true, false>(), fwd_fn<IO, VEC, true, true>() }
// index: [io][vec][lb * 2 + fast]
const FwdFn kFwd[2][2][4] = {
    {SITU_FWD_ROW(IO_F32, false), SITU_FWD_ROW(IO_F32, true)},
    {SITU_FWD_ROW(IO_BF16, false), SITU_FWD_ROW(IO_BF16, true)},
};
#define SITU_BWD_ROW(IO, VEC, DR)                                                              \
    { bwd_fn<IO, VEC, false, false, DR>(), bwd_fn<IO, VEC, false, true, DR>(),                \
      bwd_fn<IO, VEC, true, false, DR>(), bwd_fn<IO, VEC, true, true, DR>() }
// index: [io][vec][dr][lb * 2 + fast]
const BwdFn kBwd[2][2][2][4] = {
    {{SITU_BWD_ROW(IO_F32, false, false), SITU_BWD_ROW(IO_F32, false, true)},
     {SITU_BWD_ROW(IO_F32, true, false), SITU_BWD_ROW(IO_F32, true, true)}},
    {{SITU_BWD_ROW(IO_BF16, false, false), SITU_BWD_ROW(IO_BF16, false, true)},
     {SITU_BWD_ROW(IO_BF16, true, false), SITU_BWD_ROW(IO_BF16, true, true)}},
};

// Launch shape.  128-bit path: a row of `spr` strips gets min(spr, 16)
// wavefronts; rows of one strip are packed rows_per_block to a workgroup.
// Element path: one wavefront per row, four rows per workgroup.
struct Shape {
    dim3 grid, block;
    int waves_per_row;
};

Shape shape(int64_t rows, int inter, int io, int vec, int rows_per_block, int unroll)
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

int launch_fwd(const FwdLaunch &L, void *stream)
{
    const Shape sh = shape(L.rows, L.inter, L.io, L.vec, L.rows_per_block, kUnrollFwd);
    const FwdFn fn = kFwd[L.io][L.vec][L.lb * 2 + L.fast];
    hipLaunchKernelGGL(fn, sh.grid, sh.block, 0, (hipStream_t)stream, L.gate_up, L.rw, L.rw_bf16,
                       L.rw_stride, L.out, L.rows, L.inter, sh.waves_per_row, L.gk, L.uk);
    return (int)hipGetLastError();
}

int launch_bwd(const BwdLaunch &L, void *stream)
{
    const Shape sh = shape(L.rows, L.inter, L.io, L.vec, L.rows_per_block, kUnrollBwd);
    const int dr = L.d_rw != nullptr;
    const BwdFn fn = kBwd[L.io][L.vec][dr][L.lb * 2 + L.fast];
    hipLaunchKernelGGL(fn, sh.grid, sh.block, 0, (hipStream_t)stream, L.gate_up, L.rw, L.rw_bf16,
                       L.rw_stride, L.grad_out, L.d_gate_up, L.d_rw, L.row_partials, L.rows, L.inter,
                       sh.waves_per_row, L.gk, L.uk);
    int err = (int)hipGetLastError();
    if (err == 0 && dr && L.rw_stride == 0) {
        hipLaunchKernelGGL(situ_glu_dr_reduce_kernel, dim3(1), dim3(kReduceBlock), 0, (hipStream_t)stream,
                           (const float *)L.row_partials, L.rows, L.d_rw, L.rw_bf16);
        err = (int)hipGetLastError();
    }
    return err;
}

int launch_zero(void *p, int64_t bytes, void *stream)
{
    const int64_t blocks = (bytes + 255) / 256;
    hipLaunchKernelGGL(situ_glu_zero_kernel, dim3((unsigned)(blocks < 1024 ? blocks : 1024)), dim3(256), 0,
                       (hipStream_t)stream, static_cast<unsigned char *>(p), bytes);
    return (int)hipGetLastError();
}

const char *device_error_string(int err) { return hipGetErrorString((hipError_t)err); }

}  // namespace situ
