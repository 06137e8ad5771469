// Attention-residual mixing for CDNA4 (gfx950).
//
// NeMo AutoModel page "nemo_automodel.components.models.kimi_k3.situ",
// `_attn_res_core` and `_apply_attn_res` (the Kimi-K3 "dense-kda-layers /
// store" page, `_forward_attn_residual`, shows the call sites): for every
// token, the values are the stored block sums followed by the current prefix
// sum; each value row is RMS-normalised (weight w, epsilon eps) and projected
// to one logit (weight p), the logits are soft-maxed over the blocks, and the
// output is the probability-weighted sum of the raw value rows:
//   r_b = 1/sqrt(mean_h x_bh^2 + eps),  l_b = r_b sum_h x_bh w_h p_h,
//   P = softmax(l),  out_h = sum_b P_b x_bh.
// The page computes this chain in fp32; so does this kernel, reading the
// values once.
//
// Work decomposition: one workgroup per token.  A lane owns VPL 128-bit
// vectors of the hidden axis and holds them for every block in registers
// (NB <= 16 blocks), so each value is read from HBM exactly once: first the
// per-block sums of x^2 and x w p (lane partials -> DPP butterflies -> one
// LDS slot per wavefront -> a fixed-order sum), then the softmax (computed
// on every lane, the probabilities kept in scalar registers), then the
// combine from the same value registers.
// The stored sums and the prefix come through separate pointers, so the
// caller never concatenates them.  The sums are taken in a fixed order:
// results are bitwise reproducible and independent of the other tokens.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "situ_glu_device.h"
#include "situ_glu_internal.h"

namespace situ {
namespace {

constexpr int kAresMaxBlocks = 16;

// fp32 value of weight i (bf16 or fp32)
__device__ __forceinline__ float load_w(const void *w, int w_bf16, int i)
{
    return w_bf16 ? bf16_to_f32(static_cast<const uint16_t *>(w)[i]) : static_cast<const float *>(w)[i];
}

// 128-bit load that stays in the caches (the weights are read by every token)
__device__ __forceinline__ uint4 bload_cached(rsrc_t r, uint32_t off)
{
    const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, 0);
    return make_uint4(v.x, v.y, v.z, v.w);
}

// The E weights of value vector j (E = 8 for bf16 values, 4 for fp32), from a
// buffer over the weight vector: one 128-bit load, two, or one 64-bit load.
template <bool WBF16, int E>
__device__ __forceinline__ void load_wvec(rsrc_t r, uint32_t j, float *w)
{
    if (WBF16 && E == 8) {
        Io<IO_BF16>::unpack(bload_cached(r, j * 16u), w);
    } else if (!WBF16 && E == 8) {
        Io<IO_F32>::unpack(bload_cached(r, j * 32u), w);
        Io<IO_F32>::unpack(bload_cached(r, j * 32u + 16u), w + 4);
    } else if (!WBF16 && E == 4) {
        Io<IO_F32>::unpack(bload_cached(r, j * 16u), w);
    } else {
        typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
        const u32x2 v = __builtin_amdgcn_raw_buffer_load_b64(r, (int)(j * 8u), 0, 0);
        w[0] = bf_lo(v.x);
        w[1] = bf_hi(v.x);
        w[2] = bf_lo(v.y);
        w[3] = bf_hi(v.y);
    }
}

// Two fp32 -> two bf16 (low, high half), round to nearest even on the bit
// patterns: (a + 0x7fff + lsb) >> 16 rounds every finite value as the
// hardware conversion does (overflow to infinity included) and keeps a
// quiet NaN a NaN.  Written out instead of the bf16 conversion because, with
// that conversion, the compiler spills the streaming kernel's registers.
__device__ __forceinline__ uint32_t pack_bf16_rne(float lo, float hi)
{
    const uint32_t a = __float_as_uint(lo), b = __float_as_uint(hi);
    const uint32_t ra = (a + 0x7fffu + ((a >> 16) & 1u)) >> 16;
    const uint32_t rb = (b + 0x7fffu + ((b >> 16) & 1u)) & 0xffff0000u;
    return ra | rb;
}

// Store the E outputs of value vector j in the output dtype.
template <int IO, int OUT>
__device__ __forceinline__ void store_out(rsrc_t r, uint32_t j, const float *acc)
{
    if (IO == OUT && OUT == IO_BF16) {  // 8 values -> 8 bf16
        bstore(r, j * 16u, make_uint4(pack_bf16_rne(acc[0], acc[1]), pack_bf16_rne(acc[2], acc[3]),
                                      pack_bf16_rne(acc[4], acc[5]), pack_bf16_rne(acc[6], acc[7])));
    } else if (IO == OUT) {             // 4 fp32 -> 4 fp32
        bstore(r, j * 16u, Io<OUT>::pack(acc));
    } else if (IO == IO_BF16) {         // 8 values -> 8 fp32
        bstore(r, j * 32u, Io<IO_F32>::pack(acc));
        bstore(r, j * 32u + 16u, Io<IO_F32>::pack(acc + 4));
    } else {                            // 4 values -> 4 bf16
        typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
        const u32x2 v = {pack_bf16_rne(acc[0], acc[1]), pack_bf16_rne(acc[2], acc[3])};
        __builtin_amdgcn_raw_buffer_store_b64(v, r, (int)(j * 8u), 0, kStreaming);
    }
}

// The values of a 128-bit vector again, for the combine.  For bf16 the
// halves are widened with byte permutes rather than the shifts of Io::unpack:
// the same bits, but the compiler cannot merge this with the unpack of the
// sums pass and keep every block's fp32 copy alive across the barrier (which
// would not fit in registers).
template <int IO>
__device__ __forceinline__ void unpack_again(const uint4 &w, float *x)
{
    if (IO == IO_BF16) {
        const uint32_t a[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            x[2 * i] = __uint_as_float(__builtin_amdgcn_perm(0u, a[i], 0x01000c0cu));      // low half << 16
            x[2 * i + 1] = __uint_as_float(__builtin_amdgcn_perm(0u, a[i], 0x03020c0cu));  // high half
        }
    } else {
        Io<IO>::unpack(w, x);
    }
}

// One block's lane partials (sum of x^2, sum of x w p) -> wavefront sums
// (fixed-order DPP butterflies) -> this wavefront's LDS slots for block b.
// `part` holds 2 * kAresMaxBlocks floats per wavefront: sums of squares in
// slots [0, 16), dot products in [16, 32).
__device__ __forceinline__ void block_partials(float ss, float d, int b, float *part)
{
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const float s = wave_sum(ss);
    const float t = wave_sum(d);
    if ((threadIdx.x & 63) == 0) {
        part[wave * 2 * kAresMaxBlocks + b] = s;
        part[wave * 2 * kAresMaxBlocks + kAresMaxBlocks + b] = t;
    }
}

// After a barrier: the token's totals (wavefront slots added in wavefront
// order), logits l_b = d_b / sqrt(ss_b / H + eps), and the softmax over the
// blocks.  P[b] ends in scalar registers (the same on every lane).
template <int MAXNB>
__device__ __forceinline__ void block_probs(const float *part, int nwaves, int nb, float inv_h, float eps, float *P)
{
    const int lane = threadIdx.x & 63;
    float tot = 0.0f;
    if (lane < 2 * kAresMaxBlocks)
        for (int w = 0; w < nwaves; ++w)
            tot += part[w * 2 * kAresMaxBlocks + lane];
    float l[MAXNB];
    float lmax = -__builtin_inff();
#pragma unroll
    for (int b = 0; b < MAXNB; ++b) {
        if (b < nb) {
            const float ss = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(tot), b));
            const float dd = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(tot), kAresMaxBlocks + b));
            l[b] = dd * __builtin_amdgcn_rsqf(fmaf(ss, inv_h, eps));
            lmax = fmaxf(lmax, l[b]);
        }
    }
    float den = 0.0f;
#pragma unroll
    for (int b = 0; b < MAXNB; ++b) {
        if (b < nb) {
            l[b] = __builtin_amdgcn_exp2f((l[b] - lmax) * kLog2e);
            den += l[b];
        }
    }
    const float inv = 1.0f / den;
#pragma unroll
    for (int b = 0; b < MAXNB; ++b)
        P[b] = b < nb ? __int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(l[b] * inv))) : 0.0f;
}

// 128-bit path: one token per workgroup, VPL vectors per lane, up to MAXNB
// blocks held in registers (VPL * MAXNB <= 16 keeps them within the 128
// VGPRs a 1024-thread workgroup allows).
template <int IO, int OUT, bool WBF16, int VPL, int MAXNB>
__global__ void __launch_bounds__(64 * kMaxWaves)
situ_glu_attn_res_vec_kernel(const void *__restrict__ blocks, const void *__restrict__ prefix, int m, int nb,
                             int hidden, const void *__restrict__ norm_w, const void *__restrict__ proj_w, int,
                             float eps, void *__restrict__ out)
{
    using T = Io<IO>;
    using O = Io<OUT>;
    constexpr int E = T::kPerVec;
    constexpr int WB = WBF16 ? 2 : 4;
    __shared__ float part[kMaxWaves * 2 * kAresMaxBlocks];
    const int64_t tok = blockIdx.x;
    const int nthreads = blockDim.x;
    const int nwaves = nthreads >> 6;
    const uint32_t rowb = (uint32_t)hidden * T::kBytes;
    const char *brow = static_cast<const char *>(blocks) + tok * (int64_t)m * rowb;
    const char *prow = prefix ? static_cast<const char *>(prefix) + tok * (int64_t)rowb : nullptr;

    // every block's vectors, kept in registers until the combine; past the
    // row end the loads return zeros (and the stores below are dropped)
    uint4 xv[MAXNB][VPL];
#pragma unroll
    for (int b = 0; b < MAXNB; ++b) {
        if (b < nb) {
            const rsrc_t r = make_rsrc(b < m ? brow + (int64_t)b * rowb : prow, rowb);
#pragma unroll
            for (int k = 0; k < VPL; ++k)
                xv[b][k] = bload(r, (uint32_t)(threadIdx.x + k * nthreads) * 16u);
        }
    }
    // c_h = w_h p_h for this lane's values (zeros past the end)
    const rsrc_t rw = make_rsrc(norm_w, (uint32_t)hidden * WB), rp = make_rsrc(proj_w, (uint32_t)hidden * WB);
    float c[VPL][E];
#pragma unroll
    for (int k = 0; k < VPL; ++k) {
        float w[E], p[E];
        load_wvec<WBF16, E>(rw, threadIdx.x + k * nthreads, w);
        load_wvec<WBF16, E>(rp, threadIdx.x + k * nthreads, p);
#pragma unroll
        for (int e = 0; e < E; ++e)
            c[k][e] = w[e] * p[e];
    }
#pragma unroll
    for (int b = 0; b < MAXNB; ++b) {
        if (b < nb) {
            float ss = 0.0f, d = 0.0f;
#pragma unroll
            for (int k = 0; k < VPL; ++k) {
                float x[E];
                T::unpack(xv[b][k], x);
#pragma unroll
                for (int e = 0; e < E; ++e) {
                    ss = fmaf(x[e], x[e], ss);
                    d = fmaf(x[e], c[k][e], d);
                }
            }
            block_partials(ss, d, b, part);
        }
    }
    __syncthreads();
    float P[MAXNB];
    block_probs<MAXNB>(part, nwaves, nb, 1.0f / (float)hidden, eps, P);
    const rsrc_t ro = make_rsrc(static_cast<char *>(out) + tok * (int64_t)hidden * O::kBytes,
                                (uint32_t)hidden * O::kBytes);
#pragma unroll
    for (int k = 0; k < VPL; ++k) {
        float acc[E];
#pragma unroll
        for (int e = 0; e < E; ++e)
            acc[e] = 0.0f;
#pragma unroll
        for (int b = 0; b < MAXNB; ++b) {
            if (b < nb) {
                float x[E];
                unpack_again<IO>(xv[b][k], x);
#pragma unroll
                for (int e = 0; e < E; ++e)
                    acc[e] = fmaf(P[b], x[e], acc[e]);
            }
        }
        store_out<IO, OUT>(ro, threadIdx.x + k * nthreads, acc);
    }
}

// Row-partial form of the reductions (the streaming kernel): each block's
// two lane sums are reduced inside every row of 16 lanes only (four DPP
// butterfly steps; every lane of a row then holds the row's sum), and the
// first lane of each row writes it to its slot: value v (sums of squares of
// block v for v < 16, dot products of block v - 16 above) of row q of
// wavefront w at part[v * kRowStride + 4 w + q].  The cross-row and
// cross-wavefront sums are left to the softmax step, which reads each
// value's 4 * nwaves partials as 16-byte vectors, two lanes per value (the
// stride is padded by 16 bytes against bank conflicts).  Compared with full
// wavefront sums this saves four lane reads and three adds per sum.
constexpr int kRowStride = 4 * kMaxWaves + 4;
constexpr int kRowPartFloats = 2 * kAresMaxBlocks * kRowStride;

__device__ __forceinline__ float row_sum(float x)
{
    x += dpp_f<0xB1>(x);   // quad_perm [1,0,3,2]
    x += dpp_f<0x4E>(x);   // quad_perm [2,3,0,1]
    x += dpp_f<0x141>(x);  // row_half_mirror
    x += dpp_f<0x140>(x);  // row_mirror
    return x;
}

__device__ __forceinline__ void block_row_partials(float ss, float d, int b, float *part)
{
    const float s = row_sum(ss);
    const float t = row_sum(d);
    if ((threadIdx.x & 15) == 0) {
        const int slot = (int)(threadIdx.x >> 4);  // 4 * wavefront + row
        part[b * kRowStride + slot] = s;
        part[(kAresMaxBlocks + b) * kRowStride + slot] = t;
    }
}

// Softmax over MAXNB blocks of which the first nb are real (blocks past nb
// get probability 0), from the row partials, spread over the wavefront
// instead of repeated per block in every lane: block b owns lanes 4b..4b+3.
// Lanes 4b and 4b+1 add the first and the second half of the wavefronts'
// partials of the block's sum of squares, lanes 4b+2 and 4b+3 those of its
// dot product (fixed order: four running sums, then pairwise); a quad
// exchange puts both sums on every lane of the quad, so each quad holds its
// block's logit.  Largest logit and denominator: two DPP steps inside each
// 16-lane row (4 blocks), then the rows' values in row order.  P ends in
// scalar registers.
template <int MAXNB>
__device__ __forceinline__ void block_probs_quads(const float *part, int nwaves, int nb, float inv_h, float eps,
                                                  float *P)
{
    static_assert(4 * MAXNB <= 64, "one quad of lanes per block");
    constexpr int kRows = (MAXNB + 3) / 4;
    const int lane = threadIdx.x & 63;
    const int b = lane >> 2, h = lane & 3;
    const int half = (nwaves + 1) >> 1;
    float tot = 0.0f;
    if (b < MAXNB) {
        const float4 *pv = reinterpret_cast<const float4 *>(part + ((h >> 1) * kAresMaxBlocks + b) * kRowStride);
        const int w1 = (h & 1) ? nwaves : half;
        float a0 = 0.0f, a1 = 0.0f, a2 = 0.0f, a3 = 0.0f;
        for (int w = (h & 1) ? half : 0; w < w1; ++w) {
            const float4 v = pv[w];
            a0 += v.x;
            a1 += v.y;
            a2 += v.z;
            a3 += v.w;
        }
        tot = (a0 + a1) + (a2 + a3);
    }
    tot += dpp_f<0xB1>(tot);              // quad_perm [1,0,3,2]: the two halves
    const float ss = dpp_f<0x00>(tot);    // quad_perm [0,0,0,0]: sum of squares
    const float dd = dpp_f<0xAA>(tot);    // quad_perm [2,2,2,2]: dot product
    const float l = b < nb ? dd * __builtin_amdgcn_rsqf(fmaf(ss, inv_h, eps)) : -__builtin_inff();
    float m = fmaxf(l, dpp_f<0x141>(l));  // row_half_mirror: quads 0 <-> 1, 2 <-> 3
    m = fmaxf(m, dpp_f<0x140>(m));        // row_mirror: the two half rows
    float lmax = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(m), 0));
#pragma unroll
    for (int q = 1; q < kRows; ++q)
        lmax = fmaxf(lmax, __int_as_float(__builtin_amdgcn_readlane(__float_as_int(m), 16 * q)));
    const float e = __builtin_amdgcn_exp2f((l - lmax) * kLog2e);
    float t = e + dpp_f<0x141>(e);
    t += dpp_f<0x140>(t);
    float den = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(t), 0));
#pragma unroll
    for (int q = 1; q < kRows; ++q)
        den += __int_as_float(__builtin_amdgcn_readlane(__float_as_int(t), 16 * q));
    const float pe = e * (1.0f / den);
#pragma unroll
    for (int k = 0; k < MAXNB; ++k)
        P[k] = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(pe), 4 * k));
}

// Streaming variant of the 128-bit path for up to MAXNB blocks: one
// workgroup per CU walks the tokens blockIdx.x, + gridDim.x, ...; while a
// token is reduced and combined, the next token's values are already in
// flight into a second register set, and the weights are read once.  The
// two register sets swap roles every token (the loop body is written twice),
// and the LDS slots alternate by token parity, so one barrier per token
// suffices: a wavefront can only write slots of parity q again after the
// barrier of the next token, which every wavefront reaches only once done
// reading parity q.
#ifndef SITU_ARES_STREAM
#define SITU_ARES_STREAM 1
#endif

// The loads are unconditional (blocks past nb get a buffer of size 0: no
// memory access, zeros), so the code stays straight-line and the compiler's
// wait counters can tell this token's loads from the next token's.
template <int IO, int MAXNB>
__device__ __forceinline__ void ares_load_token(uint4 *xv, const char *blocks, const char *prefix, int m, int nb,
                                                uint32_t rowb, int64_t tok)
{
#pragma unroll
    for (int b = 0; b < MAXNB; ++b) {
        const char *row = b < m ? blocks + (tok * m + b) * (int64_t)rowb : prefix + tok * (int64_t)rowb;
        xv[b] = bload(make_rsrc(row, b < nb ? rowb : 0u), (uint32_t)threadIdx.x * 16u);
    }
}

// One token: sums, barrier, softmax, combine, store.  Blocks past nb were
// loaded as zeros, so every loop below runs MAXNB times without branches.
template <int IO, int OUT, int MAXNB>
__device__ __forceinline__ void ares_mix_token(const uint4 *xv, const float *c, int nb, int hidden, float eps,
                                               float *part, int nwaves, void *out, int64_t tok)
{
    using T = Io<IO>;
    using O = Io<OUT>;
    constexpr int E = T::kPerVec;
#pragma unroll
    for (int b = 0; b < MAXNB; ++b) {
        float x[E];
        T::unpack(xv[b], x);
        float ss = 0.0f, d = 0.0f;
#pragma unroll
        for (int e = 0; e < E; ++e) {
            ss = fmaf(x[e], x[e], ss);
            d = fmaf(x[e], c[e], d);
        }
        block_row_partials(ss, d, b, part);
        // one block's reduction at a time: interleaving all of them would
        // need more registers than the two tokens leave
        __builtin_amdgcn_sched_barrier(0);
    }
    __syncthreads();
    // keep the combine's widening of the values below this point: hoisted
    // above the barrier, every block's fp32 copy would be live at once
    __builtin_amdgcn_sched_barrier(0);
    float P[MAXNB];
    block_probs_quads<MAXNB>(part, nwaves, nb, 1.0f / (float)hidden, eps, P);
    float acc[E];
#pragma unroll
    for (int e = 0; e < E; ++e)
        acc[e] = 0.0f;
#pragma unroll
    for (int b = 0; b < MAXNB; ++b) {
        float x[E];
        unpack_again<IO>(xv[b], x);
#pragma unroll
        for (int e = 0; e < E; ++e)
            acc[e] = fmaf(P[b], x[e], acc[e]);
    }
    const rsrc_t ro = make_rsrc(static_cast<char *>(out) + tok * (int64_t)hidden * O::kBytes,
                                (uint32_t)hidden * O::kBytes);
    store_out<IO, OUT>(ro, threadIdx.x, acc);
}

template <int IO, int OUT, bool WBF16, int MAXNB>
__global__ void __launch_bounds__(64 * kMaxWaves)
situ_glu_attn_res_stream_kernel(const void *__restrict__ blocks, const void *__restrict__ prefix, int m, int nb,
                                int hidden, const void *__restrict__ norm_w, const void *__restrict__ proj_w,
                                int64_t tokens, float eps, void *__restrict__ out)
{
    using T = Io<IO>;
    constexpr int E = T::kPerVec;
    constexpr int WB = WBF16 ? 2 : 4;
    __shared__ __attribute__((aligned(16))) float part[2][kRowPartFloats];
    const int nwaves = blockDim.x >> 6;
    const uint32_t rowb = (uint32_t)hidden * T::kBytes;
    const char *bl = static_cast<const char *>(blocks);
    const char *pf = static_cast<const char *>(prefix);
    int64_t tok = blockIdx.x;
    if (tok >= tokens)
        return;
    float c[E];
    {
        const rsrc_t rw = make_rsrc(norm_w, (uint32_t)hidden * WB), rp = make_rsrc(proj_w, (uint32_t)hidden * WB);
        float w[E], p[E];
        load_wvec<WBF16, E>(rw, threadIdx.x, w);
        load_wvec<WBF16, E>(rp, threadIdx.x, p);
#pragma unroll
        for (int e = 0; e < E; ++e)
            c[e] = w[e] * p[e];
    }
    uint4 xa[MAXNB], xb[MAXNB];
    ares_load_token<IO, MAXNB>(xa, bl, pf, m, nb, rowb, tok);
    for (;;) {
        int64_t next = tok + gridDim.x;
        if (next < tokens)
            ares_load_token<IO, MAXNB>(xb, bl, pf, m, nb, rowb, next);
        ares_mix_token<IO, OUT, MAXNB>(xa, c, nb, hidden, eps, part[0], nwaves, out, tok);
        if (next >= tokens)
            break;
        tok = next;
        next = tok + gridDim.x;
        if (next < tokens)
            ares_load_token<IO, MAXNB>(xa, bl, pf, m, nb, rowb, next);
        ares_mix_token<IO, OUT, MAXNB>(xb, c, nb, hidden, eps, part[1], nwaves, out, tok);
        if (next >= tokens)
            break;
        tok = next;
    }
}

// Element path (any alignment, any hidden size): one workgroup per token,
// two passes over the values (sums, then the combine).
template <int IO, int OUT>
__global__ void __launch_bounds__(256)
situ_glu_attn_res_elem_kernel(const void *__restrict__ blocks, const void *__restrict__ prefix, int m, int nb,
                              int hidden, const void *__restrict__ norm_w, const void *__restrict__ proj_w,
                              int w_bf16, float eps, void *__restrict__ out)
{
    using T = Io<IO>;
    using O = Io<OUT>;
    __shared__ float part[4 * 2 * kAresMaxBlocks];
    const int64_t tok = blockIdx.x;
    const char *brow = static_cast<const char *>(blocks) + tok * (int64_t)m * hidden * T::kBytes;
    const char *prow = prefix ? static_cast<const char *>(prefix) + tok * (int64_t)hidden * T::kBytes : nullptr;
    // pass 1: per block, the sums over the token's hidden values
#pragma unroll
    for (int b = 0; b < kAresMaxBlocks; ++b) {
        if (b < nb) {
            float ss = 0.0f, d = 0.0f;
            for (int h = threadIdx.x; h < hidden; h += blockDim.x) {
                const float x = b < m ? T::load1(brow, (int64_t)b * hidden + h) : T::load1(prow, h);
                ss = fmaf(x, x, ss);
                d = fmaf(x, load_w(norm_w, w_bf16, h) * load_w(proj_w, w_bf16, h), d);
            }
            block_partials(ss, d, b, part);
        }
    }
    __syncthreads();
    float P[kAresMaxBlocks];
    block_probs<kAresMaxBlocks>(part, blockDim.x >> 6, nb, 1.0f / (float)hidden, eps, P);
    char *orow = static_cast<char *>(out) + tok * (int64_t)hidden * O::kBytes;
    for (int h = threadIdx.x; h < hidden; h += blockDim.x) {
        float acc = 0.0f;
#pragma unroll
        for (int b = 0; b < kAresMaxBlocks; ++b) {
            if (b < nb) {
                const float x = b < m ? T::load1(brow, (int64_t)b * hidden + h) : T::load1(prow, h);
                acc = fmaf(P[b], x, acc);
            }
        }
        O::store1(orow, h, acc);
    }
}

using AresFn = void (*)(const void *, const void *, int, int, int, const void *, const void *, int, float, void *);
using AresStreamFn = void (*)(const void *, const void *, int, int, int, const void *, const void *, int64_t, float,
                              void *);

// The streaming kernel for each block count 1..10 (the loops run exactly nb
// times: no all-zero blocks).
constexpr int kAresStreamMaxBlocks = 10;
#define SITU_ARES_SN(IO, OUT, W) \
    {situ_glu_attn_res_stream_kernel<IO, OUT, W, 1>, situ_glu_attn_res_stream_kernel<IO, OUT, W, 2>, \
     situ_glu_attn_res_stream_kernel<IO, OUT, W, 3>, situ_glu_attn_res_stream_kernel<IO, OUT, W, 4>, \
     situ_glu_attn_res_stream_kernel<IO, OUT, W, 5>, situ_glu_attn_res_stream_kernel<IO, OUT, W, 6>, \
     situ_glu_attn_res_stream_kernel<IO, OUT, W, 7>, situ_glu_attn_res_stream_kernel<IO, OUT, W, 8>, \
     situ_glu_attn_res_stream_kernel<IO, OUT, W, 9>, situ_glu_attn_res_stream_kernel<IO, OUT, W, 10>}
#define SITU_ARES_S(IO, OUT) {SITU_ARES_SN(IO, OUT, false), SITU_ARES_SN(IO, OUT, true)}
// index: [io][out][w_bf16][nb - 1]
const AresStreamFn kAresStream[2][2][2][kAresStreamMaxBlocks] = {
    {SITU_ARES_S(IO_F32, IO_F32), SITU_ARES_S(IO_F32, IO_BF16)},
    {SITU_ARES_S(IO_BF16, IO_F32), SITU_ARES_S(IO_BF16, IO_BF16)},
};

// Compute units of the current device (cached per device).
int cu_count()
{
    static int cached[64] = {0};
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64)
        return 256;
    if (!cached[dev]) {
        int n = 0;
        if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
            n = 256;
        cached[dev] = n;
    }
    return cached[dev];
}

// path: 0 = element path; 1 = one vector per lane, <= 12 blocks (<= 72
// VGPRs: two 14-wavefront workgroups per CU); 2 = two vectors per lane,
// <= 8 blocks; 3 = one vector per lane, <= 16 blocks (one workgroup per CU);
// 4 = the streaming kernel, one vector per lane, <= 10 blocks
template <int IO, int OUT, bool WBF16, int PATH>
constexpr AresFn ares_fn()
{
    if constexpr (PATH == 0)
        return situ_glu_attn_res_elem_kernel<IO, OUT>;
    else if constexpr (PATH == 1)
        return situ_glu_attn_res_vec_kernel<IO, OUT, WBF16, 1, 12>;
    else if constexpr (PATH == 2)
        return situ_glu_attn_res_vec_kernel<IO, OUT, WBF16, 2, 8>;
    else
        return situ_glu_attn_res_vec_kernel<IO, OUT, WBF16, 1, 16>;
}
#define SITU_ARES_P(IO, OUT, W) \
    {ares_fn<IO, OUT, W, 0>(), ares_fn<IO, OUT, W, 1>(), ares_fn<IO, OUT, W, 2>(), ares_fn<IO, OUT, W, 3>()}
#define SITU_ARES_W(IO, OUT) {SITU_ARES_P(IO, OUT, false), SITU_ARES_P(IO, OUT, true)}
// index: [io][out][w_bf16][path]
const AresFn kAres[2][2][2][4] = {
    {SITU_ARES_W(IO_F32, IO_F32), SITU_ARES_W(IO_F32, IO_BF16)},
    {SITU_ARES_W(IO_BF16, IO_F32), SITU_ARES_W(IO_BF16, IO_BF16)},
};

}  // namespace

int attn_res_path(int io, int hidden, int nb, int vec_ok)
{
    if (!vec_ok)
        return 0;
    const int nv = hidden / (io == IO_BF16 ? 8 : 4);
    if (SITU_ARES_STREAM && nv <= 64 * kMaxWaves && nb <= kAresStreamMaxBlocks)
        return 4;
    if (nv <= 64 * kMaxWaves && nb <= 12)
        return 1;
    if (nv <= 64 * kMaxWaves && nb <= 16)
        return 3;
    if (nv <= 2 * 64 * kMaxWaves && nb <= 8)
        return 2;
    return 0;
}

int launch_attn_res(const AresLaunch &L, void *stream)
{
    const int path = attn_res_path(L.io, L.hidden, L.nb, L.vec);
    if (path == 4) {
        const int nv = L.hidden / (L.io == IO_BF16 ? 8 : 4);
        const int threads = ((nv + 63) / 64) * 64;
        const int64_t grid = L.tokens < cu_count() ? L.tokens : cu_count();
        hipLaunchKernelGGL(kAresStream[L.io][L.out_io][L.w_bf16][L.nb - 1], dim3((unsigned)grid), dim3((unsigned)threads), 0,
                           (hipStream_t)stream, L.blocks, L.prefix, L.m, L.nb, L.hidden, L.norm_w, L.proj_w, L.tokens,
                           L.eps, L.out);
        return (int)hipGetLastError();
    }
    int threads = 256;
    if (path) {
        const int nv = L.hidden / (L.io == IO_BF16 ? 8 : 4);
        const int vpl = path == 2 ? 2 : 1;
        const int lanes = (nv + vpl - 1) / vpl;
        threads = ((lanes + 63) / 64) * 64;
    }
    const AresFn fn = kAres[L.io][L.out_io][L.w_bf16][path];
    hipLaunchKernelGGL(fn, dim3((unsigned)L.tokens), dim3((unsigned)threads), 0, (hipStream_t)stream, L.blocks,
                       L.prefix, L.m, L.nb, L.hidden, L.norm_w, L.proj_w, L.w_bf16, L.eps, L.out);
    return (int)hipGetLastError();
}

}  // namespace situ
