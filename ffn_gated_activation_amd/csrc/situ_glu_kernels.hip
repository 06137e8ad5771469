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
// work (128-bit path): a row is cut into chunks of 64 lanes x one 16-byte
// vector of each stream (1 KiB of each half row); a wavefront takes k
// consecutive chunks, issuing the next chunk's loads before the current
// chunk's math, and ends.  Without a routing-weight gradient the chunks are
// numbered over the whole tensor (flat mapping, one-wavefront workgroups by
// default); with it a row's chunks go to the wavefronts of one workgroup,
// whose partial sums meet in LDS.  Loads and stores go through buffer
// descriptors with the non-temporal hint.
//
// The per-element math (one reciprocal per element, Taylor replacements where
// a difference cancels) is in situ_glu_device.h.
// For b1 = 4, e1 = exp(-a/2) and e2 = e1^2: one exponential for the gate.
// nt = 1 - exp(-y) cancels for small y; there its Taylor series is used.
// T_g' cancels near its root G* < 0; there a polynomial in G - G* (fp32 io)
// or the exact value at the one bf16 input nearest G* (bf16 io), both built
// on the host for the given b1, replace it.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <mutex>

#include "situ_glu.h"
#include "situ_glu_chunk.h"
#include "situ_glu_device.h"
#include "situ_glu_internal.h"

namespace situ {
namespace {

// Streams of chunk c of a row.  NIN = 2: gate_up halves; 3: plus grad_out.
// NOUT = 1: out [rows, I]; 2: d_gate_up halves.
template <int NIN, int NOUT>
__device__ __forceinline__ Chunk<NIN, NOUT> chunk_at(int64_t row, uint32_t c, bool live, const ChunkGeom &g,
                                                      const char *gu, const char *go, char *o, uint32_t rbits)
{
    Chunk<NIN, NOUT> k;
    const uint32_t off = c * kChunkBytes;
    const uint32_t left = g.half - off;
    const uint32_t n = live ? (left < kChunkBytes ? left : kChunkBytes) : 0u;
    row = live ? row : 0;
    const char *gr = gu + row * (int64_t)g.half * 2 + off;
    k.in[0] = make_rsrc(gr, n);
    k.in[1] = make_rsrc(gr + g.half, n);
    if constexpr (NIN == 3)
        k.in[2] = make_rsrc(go + row * (int64_t)g.half + off, n);
    if constexpr (NOUT == 1) {
        k.out[0] = make_rsrc(o + row * (int64_t)g.half + off, n);
    } else {
        char *orow = o + row * (int64_t)g.half * 2 + off;
        k.out[0] = make_rsrc(orow, n);
        k.out[1] = make_rsrc(orow + g.half, n);
    }
    k.rbits = rbits;
    return k;
}

template <int IO, bool LB, bool FAST, bool RWB>
__device__ __forceinline__ void fwd_chunk(const uint4 *v, const Chunk<2, 1> &k, uint32_t voff, const GateK &gk,
                                          const UpK &uk)
{
    using T = Io<IO>;
    constexpr int E = T::kPerVec;
    const float r = weight_of<RWB>(k.rbits);
    const float rscale = LB ? r * gk.beta1 * uk.beta2 : r * gk.beta1;
    float g[E], u[E], y[E];
    T::unpack(v[0], g);
    T::unpack(v[1], u);
    if (LB && IO == IO_BF16 && wave_up_small<E>(u, uk)) {
#pragma unroll
        for (int e = 0; e < E; ++e)
            y[e] = fwd_elem_small_u<FAST>(g[e], u[e], rscale, gk, uk);
    } else {
#pragma unroll
        for (int e = 0; e < E; ++e)
            y[e] = fwd_elem<LB, FAST, IO == IO_F32>(g[e], u[e], rscale, gk, uk);
    }
    bstore(k.out[0], voff, T::pack(y));
    order_fence();
}

// DR: accumulate go T_g T_u / (b1 b2) (/ b1 without linear beta) into acc;
// otherwise the row scales ride on the gradients' factors (FOLD).
template <int IO, bool LB, bool FAST, bool RWB, bool DR>
__device__ __forceinline__ void bwd_chunk(const uint4 *v, const Chunk<3, 2> &k, uint32_t voff, const GateK &gk,
                                          const UpK &uk, float &acc)
{
    using T = Io<IO>;
    constexpr int E = T::kPerVec;
    const float r = weight_of<RWB>(k.rbits);
    const float cG = LB ? 4.0f * r * uk.beta2 : 4.0f * r;
    const float cU = LB ? 4.0f * r * gk.beta1 : r * gk.beta1;
    float g[E], u[E], og[E], dg[E], du[E];
    T::unpack(v[0], g);
    T::unpack(v[1], u);
    T::unpack(v[2], og);
    // bf16 io with a linear beta: the polynomial up branch when the whole
    // wavefront's |U| allows it.  Two half vectors, each with its own branch,
    // keep the values live across a branch (and so the registers) halved.
    const bool poly = LB && IO == IO_BF16 && wave_up_small<E>(u, uk);
    const float cU4 = 0.25f * cU;
#pragma unroll
    for (int h = 0; h < E; h += E / 2) {
        if (poly) {
#pragma unroll
            for (int e = h; e < h + E / 2; ++e) {
                const BwdOut b = bwd_elem_small_u<FAST, !DR>(g[e], u[e], og[e], cG, cU4, gk, uk);
                dg[e] = b.dg;
                du[e] = b.du;
                if (DR)
                    acc += b.p;
            }
        } else {
#pragma unroll
            for (int e = h; e < h + E / 2; ++e) {
                const BwdOut b = bwd_elem<LB, FAST, IO == IO_F32, !DR>(g[e], u[e], og[e], cG, cU, gk, uk);
                dg[e] = b.dg;
                du[e] = b.du;
                if (DR)
                    acc += b.p;
            }
        }
    }
    bstore(k.out[0], voff, T::pack(dg));
    bstore(k.out[1], voff, T::pack(du));
    order_fence();
}

// Forward, flat mapping: wavefront w takes chunks w k .. w k + k - 1 of the
// `total` chunks of the tensor.
template <int IO, bool LB, bool FAST, bool RWB>
__global__ void __launch_bounds__(256)
situ_glu_fwd_kernel(const void *__restrict__ gate_up, const void *__restrict__ rw, int64_t rw_stride, void *__restrict__ out, uint32_t total, ChunkGeom g, GateK gk, UpK uk)
{
    const uint32_t voff = (threadIdx.x & 63) * 16u;
    const uint32_t gw = blockIdx.x * (blockDim.x >> 6) + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const uint32_t first = gw * (uint32_t)g.k;
    if (first >= total)
        return;
    const int n = total - first < (uint32_t)g.k ? (int)(total - first) : g.k;
    int64_t row;
    uint32_t c;
    locate(first, g, row, c);
    auto step = [&](int64_t &r_, uint32_t &c_) {
        if (++c_ == (uint32_t)g.cpr) {
            c_ = 0;
            ++r_;
        }
    };
    const char *gp = static_cast<const char *>(gate_up);
    const char *gop = nullptr;
    char *op = static_cast<char *>(out);
#define SITU_FWD_BODY(R, K) fwd_chunk<IO, LB, FAST, RWB>(R, K, voff, gk, uk)
#define SITU_MAKE(R, C, L) chunk_at<2, 1>(R, C, L, g, gp, gop, op, weight_bits<RWB>(rw, (R) * rw_stride))
    SITU_CHUNK_PIPELINE(2, 1, SITU_MAKE, SITU_FWD_BODY)
#undef SITU_MAKE
#undef SITU_FWD_BODY
}

// Wavefronts per SIMD the backward kernels are built for (register budget
// 512 / n): 8 for the plain math, 6 with a linear beta (the bf16 kernels
// then carry both up-branch forms) or a bf16 routing weight, 5 with a
// linear beta and a beta other than 4.
#define SITU_BWD_MINW(LB, FAST, RWB) ((LB) && !(FAST) ? 5 : (LB) || (RWB) ? 6 : 8)

// Backward without a routing-weight gradient, flat mapping.
template <int IO, bool LB, bool FAST, bool RWB>
__global__ void __launch_bounds__(256, SITU_BWD_MINW(LB, FAST, RWB))
situ_glu_bwd_kernel(const void *__restrict__ gate_up, const void *__restrict__ rw, int64_t rw_stride, const void *__restrict__ grad_out, void *__restrict__ d_gate_up,
                    uint32_t total, ChunkGeom g, GateK gk, UpK uk)
{
    const uint32_t voff = (threadIdx.x & 63) * 16u;
    const uint32_t gw = blockIdx.x * (blockDim.x >> 6) + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const uint32_t first = gw * (uint32_t)g.k;
    if (first >= total)
        return;
    const int n = total - first < (uint32_t)g.k ? (int)(total - first) : g.k;
    int64_t row;
    uint32_t c;
    locate(first, g, row, c);
    auto step = [&](int64_t &r_, uint32_t &c_) {
        if (++c_ == (uint32_t)g.cpr) {
            c_ = 0;
            ++r_;
        }
    };
    const char *gp = static_cast<const char *>(gate_up);
    const char *gop = static_cast<const char *>(grad_out);
    char *op = static_cast<char *>(d_gate_up);
    float acc = 0.0f;
#define SITU_BWD_BODY(R, K) bwd_chunk<IO, LB, FAST, RWB, false>(R, K, voff, gk, uk, acc)
#define SITU_MAKE(R, C, L) chunk_at<3, 2>(R, C, L, g, gp, gop, op, weight_bits<RWB>(rw, (R) * rw_stride))
    SITU_CHUNK_PIPELINE(3, 2, SITU_MAKE, SITU_BWD_BODY)
#undef SITU_MAKE
#undef SITU_BWD_BODY
}

// Backward with the routing-weight gradient, row mapping: workgroup b holds
// rows b rpb .. b rpb + rpb - 1, wpr wavefronts each; wavefront j of a row
// takes its chunks j k .. j k + k - 1.  The row's wavefronts add their
// partial sums in LDS in wavefront order (deterministic).  One weight per
// row: d_rw[row]; one weight for all rows: the row's partial goes to
// row_partials[row] for the fixed-order second pass.
template <int IO, bool LB, bool FAST, bool RWB>
__global__ void __launch_bounds__(1024, SITU_BWD_MINW(LB, FAST, RWB))
situ_glu_bwd_dr_kernel(const void *__restrict__ gate_up, const void *__restrict__ rw, int64_t rw_stride, const void *__restrict__ grad_out, void *__restrict__ d_gate_up,
                       void *__restrict__ d_rw, float *__restrict__ row_partials, int64_t rows, ChunkGeom g,
                       GateK gk, UpK uk)
{
    __shared__ float wave_part[kMaxWaves];
    const uint32_t voff = (threadIdx.x & 63) * 16u;
    const int lane = threadIdx.x & 63;
    const int slot = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int rpb = (int)(blockDim.x >> 6) / g.wpr;
    const int rib = (slot * (int)g.wmagic) >> 8;  // slot / wpr
    const int grp = slot - rib * g.wpr;
    int64_t row = (int64_t)blockIdx.x * rpb + rib;
    const bool live = row < rows;
    const uint32_t c0 = (uint32_t)grp * (uint32_t)g.k;
    float acc = 0.0f;
    if (live && c0 < (uint32_t)g.cpr) {
        const int n = (uint32_t)g.cpr - c0 < (uint32_t)g.k ? (int)((uint32_t)g.cpr - c0) : g.k;
        uint32_t c = c0;
        auto step = [&](int64_t &, uint32_t &c_) { ++c_; };
        const char *gp = static_cast<const char *>(gate_up);
        const char *gop = static_cast<const char *>(grad_out);
        char *op = static_cast<char *>(d_gate_up);
        const uint32_t rb = weight_bits<RWB>(rw, row * rw_stride);  // one row: one weight
#define SITU_BWD_BODY(R, K) bwd_chunk<IO, LB, FAST, RWB, true>(R, K, voff, gk, uk, acc)
#define SITU_MAKE(R, C, L) chunk_at<3, 2>(R, C, L, g, gp, gop, op, rb)
        SITU_CHUNK_PIPELINE(3, 2, SITU_MAKE, SITU_BWD_BODY)
#undef SITU_MAKE
#undef SITU_BWD_BODY
    }
    const float scale = LB ? gk.beta1 * uk.beta2 : gk.beta1;
    const float s = wave_sum(acc);
    if (g.wpr == 1) {
        if (live && lane == 0)
            write_row_dr(s * scale, row, rw_stride, RWB, d_rw, row_partials);
    } else {
        if (lane == 0)
            wave_part[slot] = s;
        __syncthreads();
        if (live && grp == 0 && lane == 0) {
            float t = 0.0f;
            for (int w = 0; w < g.wpr; ++w)
                t += wave_part[slot + w];
            write_row_dr(t * scale, row, rw_stride, RWB, d_rw, row_partials);
        }
    }
}

// Element path (any alignment, any intermediate): one wavefront per row.
template <int IO, bool LB, bool FAST>
__global__ void __launch_bounds__(256)
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
__global__ void __launch_bounds__(256)
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

using FwdFn = void (*)(const void *, const void *, int64_t, void *, uint32_t, ChunkGeom, GateK, UpK);
using BwdFn = void (*)(const void *, const void *, int64_t, const void *, void *, uint32_t, ChunkGeom, GateK, UpK);
using BwdDrFn = void (*)(const void *, const void *, int64_t, const void *, void *, void *, float *, int64_t,
                         ChunkGeom, GateK, UpK);
using FwdElemFn = void (*)(const void *, const void *, int, int64_t, void *, int64_t, int, int, GateK, UpK);
using BwdElemFn = void (*)(const void *, const void *, int, int64_t, const void *, void *, void *, float *,
                           int64_t, int, int, GateK, UpK);

// index: [io][rw bf16][lb * 2 + fast]
#define SITU_BY_LB_FAST(K, IO, RWB) {K<IO, false, false, RWB>, K<IO, false, true, RWB>, \
                                     K<IO, true, false, RWB>, K<IO, true, true, RWB>}
#define SITU_BY_IO_RW(K) {{SITU_BY_LB_FAST(K, IO_F32, false), SITU_BY_LB_FAST(K, IO_F32, true)}, \
                          {SITU_BY_LB_FAST(K, IO_BF16, false), SITU_BY_LB_FAST(K, IO_BF16, true)}}
const FwdFn kFwd[2][2][4] = SITU_BY_IO_RW(situ_glu_fwd_kernel);
const BwdFn kBwd[2][2][4] = SITU_BY_IO_RW(situ_glu_bwd_kernel);
const BwdDrFn kBwdDr[2][2][4] = SITU_BY_IO_RW(situ_glu_bwd_dr_kernel);
#define SITU_ELEM(K, IO, ...) {K<IO, false, false __VA_ARGS__>, K<IO, false, true __VA_ARGS__>, \
                               K<IO, true, false __VA_ARGS__>, K<IO, true, true __VA_ARGS__>}
// index: [io][lb * 2 + fast]
const FwdElemFn kFwdElem[2][4] = {SITU_ELEM(situ_glu_fwd_elem_kernel, IO_F32), SITU_ELEM(situ_glu_fwd_elem_kernel, IO_BF16)};
// index: [io][dr][lb * 2 + fast]
const BwdElemFn kBwdElem[2][2][4] = {
    {SITU_ELEM(situ_glu_bwd_elem_kernel, IO_F32, , false), SITU_ELEM(situ_glu_bwd_elem_kernel, IO_F32, , true)},
    {SITU_ELEM(situ_glu_bwd_elem_kernel, IO_BF16, , false), SITU_ELEM(situ_glu_bwd_elem_kernel, IO_BF16, , true)}};

// Element path: one wavefront per row, four rows per workgroup.
constexpr int kElemRowsPerBlock = 4;

}  // namespace

int launch_fwd(const FwdLaunch &L, void *stream)
{
    const int v = L.lb * 2 + L.fast;
    if (L.vec) {
        hipLaunchKernelGGL(kFwd[L.io][L.rw_bf16][v], dim3(L.split.grid), dim3(L.split.block), 0, (hipStream_t)stream,
                           L.gate_up, L.rw, L.rw_stride, L.out, L.split.total, L.split.geom, L.gk, L.uk);
    } else {
        const unsigned grid = (unsigned)((L.rows + kElemRowsPerBlock - 1) / kElemRowsPerBlock);
        hipLaunchKernelGGL(kFwdElem[L.io][v], dim3(grid), dim3(64 * kElemRowsPerBlock), 0, (hipStream_t)stream,
                           L.gate_up, L.rw, L.rw_bf16, L.rw_stride, L.out, L.rows, L.inter, 0, L.gk, L.uk);
    }
    return (int)hipGetLastError();
}

int launch_bwd(const BwdLaunch &L, void *stream)
{
    const int v = L.lb * 2 + L.fast;
    const int dr = L.d_rw != nullptr;
    if (L.vec && dr) {
        hipLaunchKernelGGL(kBwdDr[L.io][L.rw_bf16][v], dim3(L.split.grid), dim3(L.split.block), 0,
                           (hipStream_t)stream, L.gate_up, L.rw, L.rw_stride, L.grad_out, L.d_gate_up, L.d_rw,
                           L.row_partials, L.rows, L.split.geom, L.gk, L.uk);
    } else if (L.vec) {
        hipLaunchKernelGGL(kBwd[L.io][L.rw_bf16][v], dim3(L.split.grid), dim3(L.split.block), 0, (hipStream_t)stream,
                           L.gate_up, L.rw, L.rw_stride, L.grad_out, L.d_gate_up, L.split.total, L.split.geom, L.gk,
                           L.uk);
    } else {
        const unsigned grid = (unsigned)((L.rows + kElemRowsPerBlock - 1) / kElemRowsPerBlock);
        hipLaunchKernelGGL(kBwdElem[L.io][dr][v], dim3(grid), dim3(64 * kElemRowsPerBlock), 0, (hipStream_t)stream,
                           L.gate_up, L.rw, L.rw_bf16, L.rw_stride, L.grad_out, L.d_gate_up, L.d_rw, L.row_partials,
                           L.rows, L.inter, 0, L.gk, L.uk);
    }
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

// ---------------------------------------------------------------- scratch of the allocation-free backward
//
// Every device the library runs on holds one copy of this array until the
// process ends.  Host code never uses its name as an address: the name is a
// host-side stand-in.  Its device address on each device comes from
// hipGetSymbolAddress, taken once per device with that device current.
static __device__ __align__(256) float scratch[SITU_NOALLOC_MAX_ROWS];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mutex;
float *g_scratch_ptr[kMaxDevices];
}  // namespace

float *device_scratch(int *err)
{
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess || dev < 0 || dev >= kMaxDevices) {
        *err = e != hipSuccess ? (int)e : (int)hipErrorInvalidDevice;
        return nullptr;
    }
    std::lock_guard<std::mutex> lock(g_scratch_mutex);
    if (!g_scratch_ptr[dev]) {
        void *p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess || !p) {
            *err = e != hipSuccess ? (int)e : (int)hipErrorInvalidSymbol;
            return nullptr;
        }
        g_scratch_ptr[dev] = static_cast<float *>(p);
    }
    return g_scratch_ptr[dev];
}

}  // namespace situ
