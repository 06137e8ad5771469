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
// The per-element math (one reciprocal per element, Taylor replacements where
// a difference cancels) is in situ_glu_device.h.
// For b1 = 4, e1 = exp(-a/2) and e2 = e1^2: one exponential for the gate.
// nt = 1 - exp(-y) cancels for small y; there its Taylor series is used.
// T_g' cancels near its root G* < 0; there a polynomial in G - G* (built on
// the host for the given b1) replaces it.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "situ_glu_device.h"
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
#ifndef SITU_BWD_MIN_WAVES
#define SITU_BWD_MIN_WAVES 8  // wavefronts per SIMD the backward must fit (<= 64 VGPRs)
#endif

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
    if (err == 0 && dr && L.rw_stride == 0)
        err = launch_dr_reduce(L.row_partials, L.rows, L.d_rw, L.rw_bf16, stream);
    return err;
}

int launch_dr_reduce(const float *row_partials, int64_t rows, void *d_rw, int rw_bf16, void *stream)
{
    hipLaunchKernelGGL(situ_glu_dr_reduce_kernel, dim3(1), dim3(kReduceBlock), 0, (hipStream_t)stream,
                       row_partials, rows, d_rw, rw_bf16);
    return (int)hipGetLastError();
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
