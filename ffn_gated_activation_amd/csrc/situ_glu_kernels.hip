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
// Memory-bound elementwise work: one wavefront owns one row; every lane moves
// 128-bit vectors of the paired G / U halves (and grad_out), computes in fp32
// registers and writes 128-bit vectors.  No MFMA: there is no contraction.
//
// Math, with a = |G|, e1 = exp(-2a/b1), e2 = exp(-a), nt = 1 - e1,
// A = 1 + e1, B = 1 + e2 (all cancellation free except nt, see below):
//   tanh(a/b1) = nt / A,  sech^2(G/b1) = 4 e1 / A^2,
//   sigmoid(G) = sn / B,  sigmoid(-G) = snc / B,
//     with (sn, snc) = (1, e2) for G >= 0 and (e2, 1) for G < 0,
//   T_g   = b1 sgn(G) nt sn / (A B)
//   T_g'  = sn [4 e1 B + b1 sgn(G) nt A snc] / (A B)^2
// and for the up branch v = exp(-2|U|/b2), C = 1 + v, nu = 1 - v:
//   T_u = b2 sgn(U) nu / C,  T_u' = 4 v / C^2.
// One reciprocal of A B C serves every quotient of an element.
// For b1 = 4, e1 = exp(-a/2) and e2 = e1^2: one exponential for the gate.
// nt = 1 - exp(-y) cancels for small y; there it is replaced by its Taylor
// series.  T_g' cancels near its root G* < 0; there a cubic in G - G* (built on
// the host for the given b1) replaces it.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "situ_glu_internal.h"

namespace situ {
namespace {

constexpr int kWaves = 4;            // wavefronts (rows) per workgroup
constexpr int kBlock = 64 * kWaves;  // threads per workgroup
constexpr int kUnroll = 4;           // 128-bit vectors in flight per lane and input
constexpr float kLog2e = 1.4426950408889634f;

__device__ __forceinline__ float ex2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float rcp(float x) { return __builtin_amdgcn_rcpf(x); }

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

// 1 - exp(-y) for y >= 0, given e = exp(-y) as rounded by the exponential.
// For small y the subtraction loses relative accuracy (error ~ ulp(1) / y);
// there the Taylor series y - y^2/2 + ... is used instead.  PRECISE (fp32 io)
// keeps five terms below 1/16 (truncation < 2e-9 relative, subtraction error
// above < 2e-6); otherwise two terms below 1/64 (< 5e-5 and < 1e-5), far
// inside half a bf16 ulp (2^-9).
template <bool PRECISE>
__device__ __forceinline__ float one_minus_exp_neg(float y, float e)
{
    if (PRECISE) {
        float s = y * (1.0f - y * (0.5f - y * (1.0f / 6.0f - y * (1.0f / 24.0f - y * (1.0f / 120.0f)))));
        return y < 0.0625f ? s : 1.0f - e;
    } else {
        float s = y * fmaf(-0.5f, y, 1.0f);
        return y < 0.015625f ? s : 1.0f - e;
    }
}

struct Gate {
    float e1, nt, A, B;
    float sn_s;   // sgn(G) * sigmoid numerator: G < 0 ? -e2 : 1
    float sn;     // sigmoid numerator:          G < 0 ?  e2 : 1
    float snc_s;  // sgn(G) * sigmoid(-G) numerator: G < 0 ? -1 : e2
};

template <bool FAST, bool PRECISE>
__device__ __forceinline__ Gate gate_parts(float g, const GateK &k)
{
    Gate o;
    const float a = fabsf(g);
    float e2;
    if (FAST) {  // b1 = 4: e1 = exp(-a/2), e2 = e1^2
        o.e1 = ex2(a * (-0.5f * kLog2e));
        e2 = o.e1 * o.e1;
        o.nt = one_minus_exp_neg<PRECISE>(a * 0.5f, o.e1);
    } else {
        o.e1 = ex2(a * k.k1);
        // exp(-a) as the square of exp(-a/2): keeps gradual underflow to a ~ 174
        const float h = ex2(a * (-0.5f * kLog2e));
        e2 = h * h;
        o.nt = one_minus_exp_neg<PRECISE>(a * k.y1k, o.e1);
    }
    o.A = 1.0f + o.e1;
    o.B = 1.0f + e2;
    const bool neg = g < 0.0f;
    o.sn_s = neg ? -e2 : 1.0f;
    o.sn = neg ? e2 : 1.0f;
    o.snc_s = neg ? -1.0f : e2;
    return o;
}

struct Up {
    float v, nu_s, C;  // nu_s = sgn(U) (1 - v)
};

template <bool PRECISE>
__device__ __forceinline__ Up up_parts(float u, const UpK &k)
{
    Up o;
    const float a = fabsf(u);
    // exp(-2a/b2) as the square of exp(-a/b2): gradual underflow for large |U|
    const float h = ex2(a * (0.5f * k.ku));
    o.v = h * h;
    o.nu_s = copysignf(one_minus_exp_neg<PRECISE>(a * k.y2k, o.v), u);
    o.C = 1.0f + o.v;
    return o;
}

// dT_g/dG near its root: cubic in d = G - G*_f32 when |d| <= half width.
__device__ __forceinline__ float gate_grad_window(float g, float plain, const GateK &k)
{
    const float d = g - k.win_ghi;  // exact (Sterbenz) inside the window
    const float p = fmaf(fmaf(fmaf(k.c3, d, k.c2), d, k.c1), d, k.c0);
    return fabsf(d) <= k.win_hw ? p : plain;
}

// Y / r
template <bool LB, bool FAST, bool PRECISE>
__device__ __forceinline__ float fwd_elem(float g, float u, float rscale, const GateK &gk, const UpK &uk)
{
    const Gate t = gate_parts<FAST, PRECISE>(g, gk);
    if (LB) {
        const Up w = up_parts<PRECISE>(u, uk);
        const float q = rcp(t.A * t.B * w.C);
        return rscale * (t.nt * t.sn_s) * (w.nu_s * q);      // rscale = r b1 b2
    } else {
        const float q = rcp(t.A * t.B);
        return rscale * (t.nt * t.sn_s) * (u * q);           // rscale = r b1
    }
}

struct BwdOut {
    float dg, du, p;  // p = go T_g T_u / (b1 b2) (b1 only without linear beta)
};

template <bool LB, bool FAST, bool PRECISE>
__device__ __forceinline__ BwdOut bwd_elem(float g, float u, float go, float r_b2, float r_b1x4,
                                           const GateK &gk, const UpK &uk)
{
    BwdOut o;
    const Gate t = gate_parts<FAST, PRECISE>(g, gk);
    // bracket of T_g': 4 e1 B + b1 sgn(G) (1 - e1)(1 + e1) snc
    const float br = fmaf(gk.beta1 * (t.nt * t.A), t.snc_s, 4.0f * t.e1 * t.B);
    if (LB) {
        const Up w = up_parts<PRECISE>(u, uk);
        const float m = t.A * t.B;
        const float q = rcp(m * w.C);
        const float iab = q * w.C;               // 1 / (A B)
        const float ic = q * m;                  // 1 / C
        const float tg = t.nt * t.sn_s * iab;    // T_g / b1
        const float tu = w.nu_s * ic;            // T_u / b2
        const float tgp = gate_grad_window(g, t.sn * br * (iab * iab), gk);  // T_g'
        const float tup = w.v * (ic * ic);       // T_u' / 4
        o.dg = go * r_b2 * tu * tgp;             // r_b2 = r b2
        o.du = go * r_b1x4 * tg * tup;           // r_b1x4 = 4 r b1
        o.p = go * tg * tu;
    } else {
        const float q = rcp(t.A * t.B);
        const float tg = t.nt * t.sn_s * q;      // T_g / b1
        const float tgp = gate_grad_window(g, t.sn * br * (q * q), gk);
        o.dg = go * r_b2 * u * tgp;              // r_b2 = r
        o.du = go * r_b1x4 * tg;                 // r_b1x4 = r b1
        o.p = go * tg * u;
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

// ---------------------------------------------------------------- kernels

template <int IO, bool VEC, bool LB, bool FAST>
__global__ void __launch_bounds__(kBlock)
situ_glu_fwd_kernel(const void *__restrict__ gate_up, const void *__restrict__ rw, int rw_bf16,
                    int64_t rw_stride, void *__restrict__ out, int64_t rows, int inter,
                    GateK gk, UpK uk)
{
    constexpr bool PRECISE = IO == IO_F32;
    using T = Io<IO>;
    const int lane = threadIdx.x & 63;
    const int64_t row = (int64_t)blockIdx.x * kWaves + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    if (row >= rows)
        return;
    const float r = load_rw(rw, rw_bf16, row * rw_stride);
    const float rscale = LB ? r * gk.beta1 * uk.beta2 : r * gk.beta1;
    const char *gu_row = static_cast<const char *>(gate_up) + row * (int64_t)inter * 2 * T::kBytes;
    char *out_row = static_cast<char *>(out) + row * (int64_t)inter * T::kBytes;

    if (VEC) {
        constexpr int E = T::kPerVec;
        const int nv = inter / E;
        const uint4 *G = reinterpret_cast<const uint4 *>(gu_row);
        const uint4 *U = G + nv;
        uint4 *O = reinterpret_cast<uint4 *>(out_row);
        for (int base = lane; base < nv; base += 64 * kUnroll) {
            uint4 gv[kUnroll], uv[kUnroll];
#pragma unroll
            for (int k = 0; k < kUnroll; ++k) {
                const int v = base + 64 * k;
                if (v < nv) {
                    gv[k] = G[v];
                    uv[k] = U[v];
                }
            }
#pragma unroll
            for (int k = 0; k < kUnroll; ++k) {
                const int v = base + 64 * k;
                if (v < nv) {
                    float g[E], u[E], y[E];
                    T::unpack(gv[k], g);
                    T::unpack(uv[k], u);
#pragma unroll
                    for (int e = 0; e < E; ++e)
                        y[e] = fwd_elem<LB, FAST, PRECISE>(g[e], u[e], rscale, gk, uk);
                    O[v] = T::pack(y);
                }
            }
        }
    } else {
        for (int j = lane; j < inter; j += 64) {
            const float g = T::load1(gu_row, j);
            const float u = T::load1(gu_row, (int64_t)inter + j);
            T::store1(out_row, j, fwd_elem<LB, FAST, PRECISE>(g, u, rscale, gk, uk));
        }
    }
}

template <int IO, bool VEC, bool LB, bool FAST, bool DR>
__global__ void __launch_bounds__(kBlock)
situ_glu_bwd_kernel(const void *__restrict__ gate_up, const void *__restrict__ rw, int rw_bf16,
                    int64_t rw_stride, const void *__restrict__ grad_out, void *__restrict__ d_gate_up,
                    void *__restrict__ d_rw, float *__restrict__ row_partials, int64_t rows, int inter,
                    GateK gk, UpK uk)
{
    constexpr bool PRECISE = IO == IO_F32;
    using T = Io<IO>;
    const int lane = threadIdx.x & 63;
    const int64_t row = (int64_t)blockIdx.x * kWaves + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    if (row >= rows)
        return;
    const float r = load_rw(rw, rw_bf16, row * rw_stride);
    const float r_b2 = LB ? r * uk.beta2 : r;
    const float r_b1x4 = LB ? 4.0f * r * gk.beta1 : r * gk.beta1;
    const int64_t in_off = row * (int64_t)inter;
    const char *gu_row = static_cast<const char *>(gate_up) + 2 * in_off * T::kBytes;
    const char *go_row = static_cast<const char *>(grad_out) + in_off * T::kBytes;
    char *dgu_row = static_cast<char *>(d_gate_up) + 2 * in_off * T::kBytes;
    float acc = 0.0f;

    if (VEC) {
        constexpr int E = T::kPerVec;
        const int nv = inter / E;
        const uint4 *G = reinterpret_cast<const uint4 *>(gu_row);
        const uint4 *U = G + nv;
        const uint4 *GO = reinterpret_cast<const uint4 *>(go_row);
        uint4 *DG = reinterpret_cast<uint4 *>(dgu_row);
        uint4 *DU = DG + nv;
        for (int base = lane; base < nv; base += 64 * kUnroll) {
            uint4 gv[kUnroll], uv[kUnroll], ov[kUnroll];
#pragma unroll
            for (int k = 0; k < kUnroll; ++k) {
                const int v = base + 64 * k;
                if (v < nv) {
                    gv[k] = G[v];
                    uv[k] = U[v];
                    ov[k] = GO[v];
                }
            }
#pragma unroll
            for (int k = 0; k < kUnroll; ++k) {
                const int v = base + 64 * k;
                if (v < nv) {
                    float g[E], u[E], o[E], dg[E], du[E];
                    T::unpack(gv[k], g);
                    T::unpack(uv[k], u);
                    T::unpack(ov[k], o);
#pragma unroll
                    for (int e = 0; e < E; ++e) {
                        const BwdOut b = bwd_elem<LB, FAST, PRECISE>(g[e], u[e], o[e], r_b2, r_b1x4, gk, uk);
                        dg[e] = b.dg;
                        du[e] = b.du;
                        if (DR)
                            acc += b.p;
                    }
                    DG[v] = T::pack(dg);
                    DU[v] = T::pack(du);
                }
            }
        }
    } else {
        for (int j = lane; j < inter; j += 64) {
            const float g = T::load1(gu_row, j);
            const float u = T::load1(gu_row, (int64_t)inter + j);
            const float o = T::load1(go_row, j);
            const BwdOut b = bwd_elem<LB, FAST, PRECISE>(g, u, o, r_b2, r_b1x4, gk, uk);
            T::store1(dgu_row, j, b.dg);
            T::store1(dgu_row, (int64_t)inter + j, b.du);
            if (DR)
                acc += b.p;
        }
    }

    if (DR) {
        const float scale = LB ? gk.beta1 * uk.beta2 : gk.beta1;
        const float s = wave_sum(acc) * scale;
        if (lane == 0) {
            if (rw_stride == 0)
                row_partials[row] = s;
            else if (rw_bf16)
                static_cast<uint16_t *>(d_rw)[row] = f32_to_bf16(s);
            else
                static_cast<float *>(d_rw)[row] = s;
        }
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

using FwdFn = void (*)(const void *, const void *, int, int64_t, void *, int64_t, int, GateK, UpK);
using BwdFn = void (*)(const void *, const void *, int, int64_t, const void *, void *, void *, float *,
                       int64_t, int, GateK, UpK);

template <int IO, bool VEC, bool LB, bool FAST>
constexpr FwdFn fwd_fn() { return situ_glu_fwd_kernel<IO, VEC, LB, FAST>; }
template <int IO, bool VEC, bool LB, bool FAST, bool DR>
constexpr BwdFn bwd_fn() { return situ_glu_bwd_kernel<IO, VEC, LB, FAST, DR>; }

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

}  // namespace

int launch_fwd(const FwdLaunch &L, void *stream)
{
    const dim3 grid((unsigned)((L.rows + kWaves - 1) / kWaves));
    const FwdFn fn = kFwd[L.io][L.vec][L.lb * 2 + L.fast];
    hipLaunchKernelGGL(fn, grid, dim3(kBlock), 0, (hipStream_t)stream, L.gate_up, L.rw, L.rw_bf16,
                       L.rw_stride, L.out, L.rows, L.inter, L.gk, L.uk);
    return (int)hipGetLastError();
}

int launch_bwd(const BwdLaunch &L, void *stream)
{
    const dim3 grid((unsigned)((L.rows + kWaves - 1) / kWaves));
    const int dr = L.d_rw != nullptr;
    const BwdFn fn = kBwd[L.io][L.vec][dr][L.lb * 2 + L.fast];
    hipLaunchKernelGGL(fn, grid, dim3(kBlock), 0, (hipStream_t)stream, L.gate_up, L.rw, L.rw_bf16,
                       L.rw_stride, L.grad_out, L.d_gate_up, L.d_rw, L.row_partials, L.rows, L.inter,
                       L.gk, L.uk);
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
