// MXFP8 output of the weighted SiTU-GLU forward and of its backward's
// d_gate_up for CDNA4 (gfx950), and the same block quantiser on its own.
//
// The Megatron-LM PR "[Dev] Add SiTU-GLU through Transformer Engine" (section
// "Test results") runs the activation of routed and shared experts under MXFP8
// block scaling: the activation's output is consumed as MXFP8 by the next
// projection.  Here the forward writes that form directly, so Y never exists
// in 16 or 32 bits in HBM.  Format (OCP Microscaling Formats (MX) v1.0 with
// the OCP 8-bit floating point element formats):
//   - each row is cut into blocks of 32 consecutive values (the last block of
//     a row may be shorter); each block has one E8M0 scale X = 2^s, stored as
//     the byte s + 127 (255 = NaN);
//   - scale mode floor: s = floor(log2(amax)) - emax_elem (8 for E4M3, 15 for
//     E5M2), the MX definition; mode ceil: the smallest s with
//     amax <= max_finite * 2^s, so that no element saturates; s is clamped to
//     [-127, 127] (an all-zero block gets s = -127);
//   - element i is Y_i / X rounded to nearest even in E4M3 or E5M2, with
//     magnitudes past the largest finite value clamped to it;
//   - a block holding a NaN or an infinity gets the NaN scale (the element
//     bytes of such a block carry no value).
//
// Layout: codes [rows, cols] bytes (row major, one byte per value), scales
// [rows, ceil(cols / 32)] bytes.
//
// Work decomposition: the forward takes the bf16 forward's chunk layout (a
// chunk is 64 lanes x one 128-bit vector of each half row, k consecutive
// chunks per wavefront, the next chunk's loads issued before the current
// chunk's math); the backward and the stand-alone quantiser strips of 64
// lanes x 2 or 4 vectors per wavefront.  A lane holds 8 (bf16) or 4 (fp32) consecutive
// values of a vector, so a block of 32 is 4 or 8 neighbouring lanes: their
// largest magnitude meets through DPP lane swaps, inside the quad (and the
// half row for 8 lanes).  Values are converted two at a time by gfx950's
// scaled fp32 -> fp8 conversion, which divides by the power of two in its
// scale operand's exponent field (the E8M0 byte itself, shifted into place)
// and rounds to nearest even; floor mode clamps to the largest finite
// value first.  Measured on MI355X, integer, compare and select
// instructions issue at about two thirds the rate of fp32 multiply-add, and
// the conversions at less than half: the instruction choices below follow
// those rates.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "situ_glu_chunk.h"
#include "situ_glu_device.h"
#include "situ_glu_internal.h"

namespace situ {
namespace {

constexpr int kMxBlock = 32;
constexpr int kUnrollMx = 4;   // 128-bit vectors in flight per lane and input stream

typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));

enum { MX_FLOOR = 0, MX_CEIL = 1 };

template <int FMT> struct Fp8;
template <> struct Fp8<FP8_E4M3> {
    static constexpr int kEmax = 8;         // largest finite value 1.75 * 2^8 = 448
    // (a, b) / 2^(exponent field of scale - 127), rounded to nearest even,
    // into bytes 0, 1 (lo) or 2, 3 (hi) of old; no saturation (E4M3
    // overflow gives NaN)
    __device__ static uint32_t lo(float a, float b, float scale, uint32_t old)
    {
        return bits(__builtin_amdgcn_cvt_scalef32_pk_fp8_f32(vec(old), a, b, scale, false));
    }
    __device__ static uint32_t hi(float a, float b, float scale, uint32_t old)
    {
        return bits(__builtin_amdgcn_cvt_scalef32_pk_fp8_f32(vec(old), a, b, scale, true));
    }
    typedef short v2i16 __attribute__((ext_vector_type(2)));
    __device__ static v2i16 vec(uint32_t x) { return __builtin_bit_cast(v2i16, x); }
    __device__ static uint32_t bits(v2i16 x) { return __builtin_bit_cast(uint32_t, x); }
};
template <> struct Fp8<FP8_E5M2> {
    static constexpr int kEmax = 15;        // largest finite value 1.75 * 2^15 = 57344
    typedef short v2i16 __attribute__((ext_vector_type(2)));
    __device__ static uint32_t lo(float a, float b, float scale, uint32_t old)
    {
        return bits(__builtin_amdgcn_cvt_scalef32_pk_bf8_f32(vec(old), a, b, scale, false));
    }
    __device__ static uint32_t hi(float a, float b, float scale, uint32_t old)
    {
        return bits(__builtin_amdgcn_cvt_scalef32_pk_bf8_f32(vec(old), a, b, scale, true));
    }
    __device__ static v2i16 vec(uint32_t x) { return __builtin_bit_cast(v2i16, x); }
    __device__ static uint32_t bits(v2i16 x) { return __builtin_bit_cast(uint32_t, x); }
};

// Bit pattern of the largest magnitude of E values.  With the sign cleared,
// the unsigned order of float bit patterns is the order of magnitudes, with
// infinity above every finite value and NaN above infinity: one integer max
// yields a pattern >= 0x7f800000 exactly when a value is infinite or NaN.
template <int E>
__device__ __forceinline__ uint32_t lane_amax_bits(const float *y)
{
    uint32_t m = 0;
#pragma unroll
    for (int e = 0; e < E; ++e)
        m = max(m, __float_as_uint(y[e]) & 0x7fffffffu);
    return m;
}

// E8M0 code of a block from the bit pattern of its largest magnitude (at or
// above 0x7f800000 for a block with a NaN or an infinity: NaN scale).  With
// amax = 1.f * 2^(eb - 127) (eb the biased exponent), floor gives
// s + 127 = eb - emax.  max_finite = 1.75 * 2^emax, so ceil adds one exactly
// when the fraction exceeds 0.75: adding 0x1fffff carries into the exponent
// field exactly then.  Zero and subnormal amax (eb = 0) fall below s = -127
// and clamp to code 0; finite codes stay <= 247.
template <int FMT, int MODE>
__device__ __forceinline__ uint32_t scale_code(uint32_t amax_bits)
{
    const uint32_t adj = MODE == MX_CEIL ? amax_bits + 0x1fffffu : amax_bits;
    const int c = (int)(adj >> 23) - Fp8<FMT>::kEmax;
    return amax_bits >= 0x7f800000u ? 255u : (uint32_t)max(c, 0);
}

// Four values -> four element codes (byte i = value i) under the block's
// scale code.  The conversion divides by 2^(code - 127), the exponent field
// of its scale operand, and rounds to nearest even.  Floor mode first clamps
// each value to +-max_finite * 2^(code - 127) (the saturation the format
// asks for; ceil mode never exceeds it).
template <int FMT, int MODE>
__device__ __forceinline__ uint32_t encode4(const float *y, uint32_t code)
{
    const float scale = __uint_as_float(code << 23);
    if (MODE == MX_FLOOR) {
        // 1.75 * 2^(code + emax - 127): exponent field code + emax, fraction 0.75
        const float lim = __uint_as_float(((code + Fp8<FMT>::kEmax) << 23) | 0x600000u);
        const float a = __builtin_amdgcn_fmed3f(y[0], -lim, lim);
        const float b = __builtin_amdgcn_fmed3f(y[1], -lim, lim);
        const float c = __builtin_amdgcn_fmed3f(y[2], -lim, lim);
        const float d = __builtin_amdgcn_fmed3f(y[3], -lim, lim);
        return Fp8<FMT>::hi(c, d, scale, Fp8<FMT>::lo(a, b, scale, 0u));
    }
    return Fp8<FMT>::hi(y[2], y[3], scale, Fp8<FMT>::lo(y[0], y[1], scale, 0u));
}

template <int CTRL>
__device__ __forceinline__ uint32_t dpp_u(uint32_t x)
{
    return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, CTRL, 0xf, 0xf, false);
}

// Largest value over aligned groups of LANES (4 or 8) lanes; every lane of
// the group ends with it.  All 64 lanes must be active.
template <int LANES>
__device__ __forceinline__ uint32_t group_max(uint32_t m)
{
    m = max(m, dpp_u<0xB1>(m));       // quad_perm [1,0,3,2]
    m = max(m, dpp_u<0x4E>(m));       // quad_perm [2,3,0,1]
    if (LANES == 8)
        m = max(m, dpp_u<0x141>(m));  // row_half_mirror: lane i <-> 7 - i of each 8
    return m;
}

// One lane's vector of E values (vector index v of its row): block maximum,
// scale code, element codes.  Codes go to byte offset v * E of the row's
// code buffer (stores past its end are dropped); the scale code is returned.
template <int FMT, int MODE, int E>
__device__ __forceinline__ uint32_t quantize_codes(const float *y, int v, rsrc_t rc)
{
    constexpr int kLanes = kMxBlock / E;
    const uint32_t m = group_max<kLanes>(lane_amax_bits<E>(y));
    const uint32_t code = scale_code<FMT, MODE>(m);
    if (E == 8) {
        const u32x2 w = {encode4<FMT, MODE>(y, code), encode4<FMT, MODE>(y + 4, code)};
        __builtin_amdgcn_raw_buffer_store_b64(w, rc, v * 8, 0, kStreaming);
    } else {
        __builtin_amdgcn_raw_buffer_store_b32(encode4<FMT, MODE>(y, code), rc, v * 4, 0, kStreaming);
    }
    return code;
}

// The same with the scale stored: from the first lane of the block to byte
// v / (32 / E) of the row's scale buffer (dropped past its end).  Every lane
// issues the scale store, the block's other lanes at an offset past any
// buffer's end: no lane mask to set up and restore around it (measured 3%
// faster for the fused forward than a store under `if (first lane)`).
template <int FMT, int MODE, int E>
__device__ __forceinline__ void quantize_vector(const float *y, int v, int lane, rsrc_t rc, rsrc_t rs)
{
    constexpr int kLanes = kMxBlock / E;
    const uint32_t code = quantize_codes<FMT, MODE, E>(y, v, rc);
    __builtin_amdgcn_raw_buffer_store_b8((unsigned char)code, rs,
                                         (lane & (kLanes - 1)) == 0 ? v / kLanes : 0x7fffffff, 0, kStreaming);
}

// One value (element paths): code of y under the block's scale code.
template <int FMT, int MODE>
__device__ __forceinline__ unsigned char encode1(float y, uint32_t code)
{
    const float z[4] = {y, 0.0f, 0.0f, 0.0f};
    return (unsigned char)(encode4<FMT, MODE>(z, code) & 0xffu);
}

// ---------------------------------------------------------------- kernels

// Streams of chunk c of a row for the fused forward: the gate and up halves
// in, the chunk's element codes (kChunkBytes / element size of them) and
// block scales out.
template <int IO>
__device__ __forceinline__ Chunk<2, 2> mx_chunk_at(int64_t row, uint32_t c, bool live, const ChunkGeom &g,
                                                   const char *gu, unsigned char *codes, unsigned char *scales,
                                                   uint32_t inter, uint32_t nblk, uint32_t rbits)
{
    constexpr uint32_t kVals = kChunkBytes / Io<IO>::kBytes, kBlocks = kVals / kMxBlock;
    Chunk<2, 2> k;
    const uint32_t off = c * kChunkBytes;
    const uint32_t left = g.half - off;
    const uint32_t n = live ? (left < kChunkBytes ? left : kChunkBytes) : 0u;
    const uint32_t v0 = c * kVals, b0 = c * kBlocks;
    const uint32_t nv = live ? (inter - v0 < kVals ? inter - v0 : kVals) : 0u;
    const uint32_t nb = live ? (nblk - b0 < kBlocks ? nblk - b0 : kBlocks) : 0u;
    row = live ? row : 0;
    const char *gr = gu + row * (int64_t)g.half * 2 + off;
    k.in[0] = make_rsrc(gr, n);
    k.in[1] = make_rsrc(gr + g.half, n);
    k.out[0] = make_rsrc(codes + row * (int64_t)inter + v0, nv);
    k.out[1] = make_rsrc(scales + row * (int64_t)nblk + b0, nb);
    k.rbits = rbits;
    return k;
}

// One chunk of the fused forward: Y in fp32, then its blocks quantised.  bf16
// io with a linear beta takes the polynomial up branch when the wavefront's
// |U| allow it (degree 7: the fp32 Y stays inside the chain's 1e-5).  Past
// the row end the loads returned zeros: Y = 0 there, which leaves every
// block maximum unchanged, and the stores are dropped.  KEEP: the block's
// scale code is returned instead of stored (the caller stores a group's).
template <int IO, bool LB, bool FAST, bool RWB, int FMT, int MODE, bool KEEP = false>
__device__ __forceinline__ uint32_t fwd_mx_chunk(const uint4 *v, const Chunk<2, 2> &k, int lane, const GateK &gk,
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
            y[e] = fwd_elem_small_u<FAST, 7>(g[e], u[e], rscale, gk, uk);
    } else {
#pragma unroll
        for (int e = 0; e < E; ++e)
            y[e] = fwd_elem<LB, FAST, IO == IO_F32>(g[e], u[e], rscale, gk, uk);
    }
    uint32_t code = 0;
    if (KEEP)
        code = quantize_codes<FMT, MODE, E>(y, lane, k.out[0]);
    else
        quantize_vector<FMT, MODE, E>(y, lane, lane, k.out[0], k.out[1]);
    order_fence();
    return code;
}

// Fused forward, 128-bit path: flat chunk mapping, wavefront w takes chunks
// w k .. w k + k - 1 of the `total` chunks.
template <int IO, bool LB, bool FAST, bool RWB, int FMT, int MODE>
__global__ void __launch_bounds__(256)
situ_glu_fwd_mx_kernel(const void *__restrict__ gate_up, const void *__restrict__ rw, int64_t rw_stride,
                       unsigned char *__restrict__ codes, unsigned char *__restrict__ scales, uint32_t inter,
                       uint32_t total, ChunkGeom g, GateK gk, UpK uk)
{
    const int lane = threadIdx.x & 63;
    const uint32_t voff = (uint32_t)lane * 16u;
    const uint32_t gw = blockIdx.x * (blockDim.x >> 6) + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const uint32_t first = gw * (uint32_t)g.k;
    if (first >= total)
        return;
    const int n = total - first < (uint32_t)g.k ? (int)(total - first) : g.k;
    const uint32_t nblk = (inter + kMxBlock - 1) / kMxBlock;
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
    if (IO == IO_BF16 && g.k == 4 && g.cpr % 4 == 0) {
        // the wavefront's four chunks are one aligned group of a row: lane
        // 4q + j keeps block q's scale code of chunk j, and one byte store
        // writes the group's 64 scale bytes (chunk j's block q at 16 j + q)
        const uint32_t j = lane & 3, q = lane >> 2;
        uint4 A[2], B[2];
        Chunk<2, 2> ka = mx_chunk_at<IO>(row, c, true, g, gp, codes, scales, inter, nblk,
                                         weight_bits<RWB>(rw, row * rw_stride));
        load_chunk(A, ka, voff);
        Chunk<2, 2> kb = mx_chunk_at<IO>(row, c + 1, true, g, gp, codes, scales, inter, nblk, ka.rbits);
        load_chunk(B, kb, voff);
        uint32_t sc = fwd_mx_chunk<IO, LB, FAST, RWB, FMT, MODE, true>(A, ka, lane, gk, uk);
        ka = mx_chunk_at<IO>(row, c + 2, true, g, gp, codes, scales, inter, nblk, kb.rbits);
        load_chunk(A, ka, voff);
        const uint32_t s1 = fwd_mx_chunk<IO, LB, FAST, RWB, FMT, MODE, true>(B, kb, lane, gk, uk);
        sc = j == 1 ? s1 : sc;
        kb = mx_chunk_at<IO>(row, c + 3, true, g, gp, codes, scales, inter, nblk, ka.rbits);
        load_chunk(B, kb, voff);
        const uint32_t s2 = fwd_mx_chunk<IO, LB, FAST, RWB, FMT, MODE, true>(A, ka, lane, gk, uk);
        sc = j == 2 ? s2 : sc;
        const uint32_t s3 = fwd_mx_chunk<IO, LB, FAST, RWB, FMT, MODE, true>(B, kb, lane, gk, uk);
        sc = j == 3 ? s3 : sc;
        // the row's blocks from the group's first on, at most 64: the last
        // chunk of a row may be partial, and bytes past the row are dropped
        const uint32_t b0 = c * (kChunkBytes / 2 / kMxBlock);
        const rsrc_t rs = make_rsrc(scales + row * (int64_t)nblk + b0, nblk - b0 < 64u ? nblk - b0 : 64u);
        __builtin_amdgcn_raw_buffer_store_b8((unsigned char)sc, rs, (int)(16 * j + q), 0, kStreaming);
        return;
    }
#define SITU_MX_BODY(R, K) fwd_mx_chunk<IO, LB, FAST, RWB, FMT, MODE>(R, K, lane, gk, uk)
#define SITU_MAKE(R, C, L) \
    mx_chunk_at<IO>(R, C, L, g, gp, codes, scales, inter, nblk, weight_bits<RWB>(rw, (R) * rw_stride))
    SITU_CHUNK_PIPELINE(2, 2, SITU_MAKE, SITU_MX_BODY)
#undef SITU_MAKE
#undef SITU_MX_BODY
}

// Largest value over each half wavefront (lanes 0-31, 32-63).
__device__ __forceinline__ uint32_t half_wave_max(uint32_t m)
{
#pragma unroll
    for (int o = 1; o < 32; o <<= 1)
        m = max(m, (uint32_t)__shfl_xor((int)m, o));
    return m;
}

// Fused forward, element path (any alignment, any intermediate): one
// wavefront per row, 64 values (two blocks) per step.
template <int IO, bool LB, bool FAST, int FMT, int MODE>
__global__ void __launch_bounds__(64 * kMaxWaves)
situ_glu_fwd_mx_elem_kernel(const void *__restrict__ gate_up, const void *__restrict__ rw, int rw_bf16,
                            int64_t rw_stride, unsigned char *__restrict__ codes,
                            unsigned char *__restrict__ scales, int64_t rows, int inter, int /*unused*/,
                            GateK gk, UpK uk)
{
    constexpr bool PRECISE = IO == IO_F32;
    using T = Io<IO>;
    const int lane = threadIdx.x & 63;
    const int64_t row = (int64_t)blockIdx.x * (blockDim.x >> 6) + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    if (row >= rows)
        return;
    const int nblk = (inter + kMxBlock - 1) / kMxBlock;
    const float r = load_rw(rw, rw_bf16, row * rw_stride);
    const float rscale = LB ? r * gk.beta1 * uk.beta2 : r * gk.beta1;
    const char *gu_row = static_cast<const char *>(gate_up) + row * (int64_t)inter * 2 * T::kBytes;
    unsigned char *c_row = codes + row * (int64_t)inter;
    unsigned char *s_row = scales + row * (int64_t)nblk;
    for (int j0 = 0; j0 < inter; j0 += 64) {
        const int j = j0 + lane;
        float y = 0.0f;
        if (j < inter)
            y = fwd_elem<LB, FAST, PRECISE>(T::load1(gu_row, j), T::load1(gu_row, (int64_t)inter + j), rscale,
                                            gk, uk);
        const uint32_t code = scale_code<FMT, MODE>(half_wave_max(__float_as_uint(y) & 0x7fffffffu));
        if (j < inter) {
            c_row[j] = encode1<FMT, MODE>(y, code);
            if ((lane & 31) == 0)
                s_row[j / kMxBlock] = (unsigned char)code;
        }
    }
}

// The block quantiser on its own: x [rows, cols] of the io dtype.
template <int IO, int FMT, int MODE>
__global__ void __launch_bounds__(64 * kMaxWaves)
situ_glu_mx_quant_vec_kernel(const void *__restrict__ x, unsigned char *__restrict__ codes,
                             unsigned char *__restrict__ scales, int64_t rows, int cols, int waves_per_row)
{
    using T = Io<IO>;
    constexpr int E = T::kPerVec;
    constexpr int kStrip = 64 * kUnrollMx;
    const int lane = threadIdx.x & 63;
    const Place pl = place(waves_per_row);
    if (pl.row >= rows)
        return;
    const int nv = cols / E;
    const uint32_t bytes = (uint32_t)nv * 16u;
    const int nblk = (cols + kMxBlock - 1) / kMxBlock;
    const int spr = (nv + kStrip - 1) / kStrip;
    const rsrc_t rx = make_rsrc(static_cast<const char *>(x) + pl.row * (int64_t)bytes, bytes);
    const rsrc_t rc = make_rsrc(codes + pl.row * (int64_t)cols, (uint32_t)cols);
    const rsrc_t rs = make_rsrc(scales + pl.row * (int64_t)nblk, (uint32_t)nblk);
    for (int s = pl.strip0; s < spr; s += pl.wpr) {
        uint4 xv[kUnrollMx];
#pragma unroll
        for (int k = 0; k < kUnrollMx; ++k)
            xv[k] = bload(rx, (uint32_t)(s * kStrip + 64 * k + lane) * 16u);
#pragma unroll
        for (int k = 0; k < kUnrollMx; ++k) {
            float y[E];
            T::unpack(xv[k], y);
            quantize_vector<FMT, MODE, E>(y, s * kStrip + 64 * k + lane, lane, rc, rs);
        }
    }
}

template <int IO, int FMT, int MODE>
__global__ void __launch_bounds__(64 * kMaxWaves)
situ_glu_mx_quant_elem_kernel(const void *__restrict__ x, unsigned char *__restrict__ codes,
                              unsigned char *__restrict__ scales, int64_t rows, int cols, int /*unused*/)
{
    using T = Io<IO>;
    const int lane = threadIdx.x & 63;
    const int64_t row = (int64_t)blockIdx.x * (blockDim.x >> 6) + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    if (row >= rows)
        return;
    const int nblk = (cols + kMxBlock - 1) / kMxBlock;
    const char *x_row = static_cast<const char *>(x) + row * (int64_t)cols * T::kBytes;
    unsigned char *c_row = codes + row * (int64_t)cols;
    unsigned char *s_row = scales + row * (int64_t)nblk;
    for (int j0 = 0; j0 < cols; j0 += 64) {
        const int j = j0 + lane;
        const float y = j < cols ? T::load1(x_row, j) : 0.0f;
        const uint32_t code = scale_code<FMT, MODE>(half_wave_max(__float_as_uint(y) & 0x7fffffffu));
        if (j < cols) {
            c_row[j] = encode1<FMT, MODE>(y, code);
            if ((lane & 31) == 0)
                s_row[j / kMxBlock] = (unsigned char)code;
        }
    }
}

// Backward with MXFP8 d_gate_up: dG and dU of a row are quantised as two
// rows of `inter` values (blocks never straddle them): codes [rows, 2 inter]
// (dG then dU), scales [rows, 2 ceil(inter / 32)] (dG's blocks, then dU's).
// dr as in the bf16 backward; `d_rw` NULL skips it.  128-bit path with the
// backward's placement and unroll.
#ifndef SITU_UNROLL_BWD_MX
#define SITU_UNROLL_BWD_MX 2
#endif
#ifndef SITU_BWD_MX_WAVES_PER_SIMD
#define SITU_BWD_MX_WAVES_PER_SIMD 1
#endif
constexpr int kUnrollBwdMx = SITU_UNROLL_BWD_MX;

template <int IO, bool LB, bool FAST, int FMT, int MODE>
__global__ void __launch_bounds__(64 * kMaxWaves, SITU_BWD_MX_WAVES_PER_SIMD)
situ_glu_bwd_mx_vec_kernel(const void *__restrict__ gate_up, const void *__restrict__ rw, int rw_bf16,
                           int64_t rw_stride, const void *__restrict__ grad_out, unsigned char *__restrict__ codes,
                           unsigned char *__restrict__ scales, void *__restrict__ d_rw,
                           float *__restrict__ row_partials, int64_t rows, int inter, int waves_per_row, GateK gk,
                           UpK uk)
{
    constexpr bool PRECISE = IO == IO_F32;
    using T = Io<IO>;
    constexpr int E = T::kPerVec;
    constexpr int kStrip = 64 * kUnrollBwdMx;
    __shared__ float wave_part[kMaxWaves];
    const int lane = threadIdx.x & 63;
    const Place pl = place(waves_per_row);
    const bool live = pl.row < rows;
    const bool dr = d_rw != nullptr;
    float acc = 0.0f;
    if (live) {
        const int nv = inter / E;
        const uint32_t half = (uint32_t)nv * 16u;
        const int spr = (nv + kStrip - 1) / kStrip;
        const int nblk = (inter + kMxBlock - 1) / kMxBlock;
        const char *row = static_cast<const char *>(gate_up) + pl.row * (int64_t)half * 2;
        const rsrc_t rg = make_rsrc(row, half), ru = make_rsrc(row + half, half);
        const rsrc_t rgo = make_rsrc(static_cast<const char *>(grad_out) + pl.row * (int64_t)half, half);
        unsigned char *crow = codes + pl.row * 2 * (int64_t)inter;
        unsigned char *srow = scales + pl.row * 2 * (int64_t)nblk;
        const rsrc_t rcg = make_rsrc(crow, (uint32_t)inter), rcu = make_rsrc(crow + inter, (uint32_t)inter);
        const rsrc_t rsg = make_rsrc(srow, (uint32_t)nblk), rsu = make_rsrc(srow + nblk, (uint32_t)nblk);
        const float r = load_rw(rw, rw_bf16, pl.row * rw_stride);
        const float cG = LB ? 4.0f * r * uk.beta2 : 4.0f * r;
        const float cU = LB ? 4.0f * r * gk.beta1 : r * gk.beta1;
        for (int s = pl.strip0; s < spr; s += pl.wpr) {
            uint4 gv[kUnrollBwdMx], uv[kUnrollBwdMx], ov[kUnrollBwdMx];
#pragma unroll
            for (int k = 0; k < kUnrollBwdMx; ++k) {
                const uint32_t off = (uint32_t)(s * kStrip + 64 * k + lane) * 16u;
                gv[k] = bload(rg, off);
                uv[k] = bload(ru, off);
                ov[k] = bload(rgo, off);
            }
#pragma unroll
            for (int k = 0; k < kUnrollBwdMx; ++k) {
                // past the row end the loads returned zeros: dG = dU = 0
                // there, which leaves every block maximum unchanged, and the
                // stores are dropped
                float g[E], u[E], og[E], dg[E], du[E];
                T::unpack(gv[k], g);
                T::unpack(uv[k], u);
                T::unpack(ov[k], og);
#pragma unroll
                for (int e = 0; e < E; ++e) {
                    const BwdOut b = bwd_elem<LB, FAST, PRECISE>(g[e], u[e], og[e], cG, cU, gk, uk);
                    dg[e] = b.dg;
                    du[e] = b.du;
                    acc += b.p;
                }
                const int v = s * kStrip + 64 * k + lane;
                quantize_vector<FMT, MODE, E>(dg, v, lane, rcg, rsg);
                quantize_vector<FMT, MODE, E>(du, v, lane, rcu, rsu);
            }
        }
    }
    if (dr) {
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

// Backward with MXFP8 d_gate_up, element path (any alignment, any
// intermediate): one wavefront per row, 64 values (two blocks) per step.
template <int IO, bool LB, bool FAST, int FMT, int MODE>
__global__ void __launch_bounds__(64 * kMaxWaves)
situ_glu_bwd_mx_elem_kernel(const void *__restrict__ gate_up, const void *__restrict__ rw, int rw_bf16,
                            int64_t rw_stride, const void *__restrict__ grad_out, unsigned char *__restrict__ codes,
                            unsigned char *__restrict__ scales, void *__restrict__ d_rw,
                            float *__restrict__ row_partials, int64_t rows, int inter, int /*unused*/, GateK gk,
                            UpK uk)
{
    constexpr bool PRECISE = IO == IO_F32;
    using T = Io<IO>;
    const int lane = threadIdx.x & 63;
    const int64_t row = (int64_t)blockIdx.x * (blockDim.x >> 6) + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    if (row >= rows)
        return;
    const int nblk = (inter + kMxBlock - 1) / kMxBlock;
    const float r = load_rw(rw, rw_bf16, row * rw_stride);
    const float cG = LB ? 4.0f * r * uk.beta2 : 4.0f * r;
    const float cU = LB ? 4.0f * r * gk.beta1 : r * gk.beta1;
    const char *gu_row = static_cast<const char *>(gate_up) + row * (int64_t)inter * 2 * T::kBytes;
    const char *go_row = static_cast<const char *>(grad_out) + row * (int64_t)inter * T::kBytes;
    unsigned char *cg_row = codes + row * 2 * (int64_t)inter, *cu_row = cg_row + inter;
    unsigned char *sg_row = scales + row * 2 * (int64_t)nblk, *su_row = sg_row + nblk;
    float acc = 0.0f;
    for (int j0 = 0; j0 < inter; j0 += 64) {
        const int j = j0 + lane;
        float dg = 0.0f, du = 0.0f;
        if (j < inter) {
            const BwdOut b = bwd_elem<LB, FAST, PRECISE>(T::load1(gu_row, j), T::load1(gu_row, (int64_t)inter + j),
                                                         T::load1(go_row, j), cG, cU, gk, uk);
            dg = b.dg;
            du = b.du;
            acc += b.p;
        }
        const uint32_t code_g = scale_code<FMT, MODE>(half_wave_max(__float_as_uint(dg) & 0x7fffffffu));
        const uint32_t code_u = scale_code<FMT, MODE>(half_wave_max(__float_as_uint(du) & 0x7fffffffu));
        if (j < inter) {
            cg_row[j] = encode1<FMT, MODE>(dg, code_g);
            cu_row[j] = encode1<FMT, MODE>(du, code_u);
            if ((lane & 31) == 0) {
                sg_row[j / kMxBlock] = (unsigned char)code_g;
                su_row[j / kMxBlock] = (unsigned char)code_u;
            }
        }
    }
    if (d_rw != nullptr) {
        const float s = wave_sum(acc);
        if (lane == 0)
            write_row_dr(s * (LB ? gk.beta1 * uk.beta2 : gk.beta1), row, rw_stride, rw_bf16, d_rw, row_partials);
    }
}

// ---------------------------------------------------------------- dispatch

using FwdMxFn = void (*)(const void *, const void *, int, int64_t, unsigned char *, unsigned char *, int64_t, int,
                         int, GateK, UpK);
using QuantFn = void (*)(const void *, unsigned char *, unsigned char *, int64_t, int, int);
using BwdMxFn = void (*)(const void *, const void *, int, int64_t, const void *, unsigned char *, unsigned char *,
                         void *, float *, int64_t, int, int, GateK, UpK);

template <int IO, bool VEC, int FMT, int MODE>
constexpr QuantFn quant_fn()
{
    if constexpr (VEC)
        return situ_glu_mx_quant_vec_kernel<IO, FMT, MODE>;
    else
        return situ_glu_mx_quant_elem_kernel<IO, FMT, MODE>;
}

// element path: index [io][lb * 2 + fast][fmt][mode]
#define SITU_MXE_FM(IO, LB, FAST, FMT)                                                                \
    {situ_glu_fwd_mx_elem_kernel<IO, LB, FAST, FMT, MX_FLOOR>, situ_glu_fwd_mx_elem_kernel<IO, LB, FAST, FMT, MX_CEIL>}
#define SITU_MXE_CASE(IO, LB, FAST) {SITU_MXE_FM(IO, LB, FAST, FP8_E4M3), SITU_MXE_FM(IO, LB, FAST, FP8_E5M2)}
#define SITU_MXE_ROW(IO)                                                                             \
    { SITU_MXE_CASE(IO, false, false), SITU_MXE_CASE(IO, false, true), SITU_MXE_CASE(IO, true, false), \
      SITU_MXE_CASE(IO, true, true) }
const FwdMxFn kFwdMxElem[2][4][2][2] = {SITU_MXE_ROW(IO_F32), SITU_MXE_ROW(IO_BF16)};
// 128-bit path: index [io][rw bf16][lb * 2 + fast][fmt][mode]
#define SITU_MXV_FM(IO, RWB, LB, FAST, FMT)                                                          \
    {situ_glu_fwd_mx_kernel<IO, LB, FAST, RWB, FMT, MX_FLOOR>, situ_glu_fwd_mx_kernel<IO, LB, FAST, RWB, FMT, MX_CEIL>}
#define SITU_MXV_CASE(IO, RWB, LB, FAST) {SITU_MXV_FM(IO, RWB, LB, FAST, FP8_E4M3), SITU_MXV_FM(IO, RWB, LB, FAST, FP8_E5M2)}
#define SITU_MXV_RW(IO, RWB)                                                                         \
    { SITU_MXV_CASE(IO, RWB, false, false), SITU_MXV_CASE(IO, RWB, false, true),                       \
      SITU_MXV_CASE(IO, RWB, true, false), SITU_MXV_CASE(IO, RWB, true, true) }
using FwdMxVecFn = void (*)(const void *, const void *, int64_t, unsigned char *, unsigned char *, uint32_t, uint32_t,
                            ChunkGeom, GateK, UpK);
const FwdMxVecFn kFwdMxVec[2][2][4][2][2] = {{SITU_MXV_RW(IO_F32, false), SITU_MXV_RW(IO_F32, true)},
                                             {SITU_MXV_RW(IO_BF16, false), SITU_MXV_RW(IO_BF16, true)}};
template <int IO, bool VEC, bool LB, bool FAST, int FMT, int MODE>
constexpr BwdMxFn bwd_mx_fn()
{
    if constexpr (VEC)
        return situ_glu_bwd_mx_vec_kernel<IO, LB, FAST, FMT, MODE>;
    else
        return situ_glu_bwd_mx_elem_kernel<IO, LB, FAST, FMT, MODE>;
}
#define SITU_BMX_FM(IO, VEC, LB, FAST, FMT) {bwd_mx_fn<IO, VEC, LB, FAST, FMT, MX_FLOOR>(), bwd_mx_fn<IO, VEC, LB, FAST, FMT, MX_CEIL>()}
#define SITU_BMX_CASE(IO, VEC, LB, FAST) {SITU_BMX_FM(IO, VEC, LB, FAST, FP8_E4M3), SITU_BMX_FM(IO, VEC, LB, FAST, FP8_E5M2)}
#define SITU_BMX_ROW(IO, VEC)                                                                        \
    { SITU_BMX_CASE(IO, VEC, false, false), SITU_BMX_CASE(IO, VEC, false, true),                    \
      SITU_BMX_CASE(IO, VEC, true, false), SITU_BMX_CASE(IO, VEC, true, true) }
// index: [io][vec][lb * 2 + fast][fmt][mode]
const BwdMxFn kBwdMx[2][2][4][2][2] = {
    {SITU_BMX_ROW(IO_F32, false), SITU_BMX_ROW(IO_F32, true)},
    {SITU_BMX_ROW(IO_BF16, false), SITU_BMX_ROW(IO_BF16, true)},
};
#define SITU_Q_FM(IO, VEC, FMT) {quant_fn<IO, VEC, FMT, MX_FLOOR>(), quant_fn<IO, VEC, FMT, MX_CEIL>()}
// index: [io][vec][fmt][mode]
const QuantFn kQuant[2][2][2][2] = {
    {{SITU_Q_FM(IO_F32, false, FP8_E4M3), SITU_Q_FM(IO_F32, false, FP8_E5M2)},
     {SITU_Q_FM(IO_F32, true, FP8_E4M3), SITU_Q_FM(IO_F32, true, FP8_E5M2)}},
    {{SITU_Q_FM(IO_BF16, false, FP8_E4M3), SITU_Q_FM(IO_BF16, false, FP8_E5M2)},
     {SITU_Q_FM(IO_BF16, true, FP8_E4M3), SITU_Q_FM(IO_BF16, true, FP8_E5M2)}},
};

}  // namespace

int launch_fwd_mx(const FwdMxLaunch &L, void *stream)
{
    const int v = L.lb * 2 + L.fast, mode = L.ceil_mode ? MX_CEIL : MX_FLOOR;
    if (L.vec) {
        hipLaunchKernelGGL(kFwdMxVec[L.io][L.rw_bf16][v][L.fmt][mode], dim3(L.split.grid), dim3(L.split.block), 0,
                           (hipStream_t)stream, L.gate_up, L.rw, L.rw_stride, static_cast<unsigned char *>(L.codes),
                           static_cast<unsigned char *>(L.scales), (uint32_t)L.inter, L.split.total, L.split.geom,
                           L.gk, L.uk);
    } else {
        const Shape sh = shape(L.rows, L.inter, L.io, 0, L.rows_per_block, kUnrollMx);
        hipLaunchKernelGGL(kFwdMxElem[L.io][v][L.fmt][mode], sh.grid, sh.block, 0, (hipStream_t)stream, L.gate_up,
                           L.rw, L.rw_bf16, L.rw_stride, static_cast<unsigned char *>(L.codes),
                           static_cast<unsigned char *>(L.scales), L.rows, L.inter, sh.waves_per_row, L.gk, L.uk);
    }
    return (int)hipGetLastError();
}

int launch_bwd_mx(const BwdMxLaunch &L, void *stream)
{
    const Shape sh = shape(L.rows, L.inter, L.io, L.vec, L.rows_per_block, kUnrollBwdMx);
    const BwdMxFn fn = kBwdMx[L.io][L.vec][L.lb * 2 + L.fast][L.fmt][L.ceil_mode ? MX_CEIL : MX_FLOOR];
    hipLaunchKernelGGL(fn, sh.grid, sh.block, 0, (hipStream_t)stream, L.gate_up, L.rw, L.rw_bf16, L.rw_stride,
                       L.grad_out, static_cast<unsigned char *>(L.codes), static_cast<unsigned char *>(L.scales),
                       L.d_rw, L.row_partials, L.rows, L.inter, sh.waves_per_row, L.gk, L.uk);
    int err = (int)hipGetLastError();
    if (err == 0 && L.d_rw && L.rw_stride == 0)
        err = launch_dr_reduce(L.row_partials, L.rows, L.d_rw, L.rw_bf16, stream);
    return err;
}

int launch_mx_quant(const MxQuantLaunch &L, void *stream)
{
    const Shape sh = shape(L.rows, L.cols, L.io, L.vec, L.rows_per_block, kUnrollMx);
    const QuantFn fn = kQuant[L.io][L.vec][L.fmt][L.ceil_mode ? MX_CEIL : MX_FLOOR];
    hipLaunchKernelGGL(fn, sh.grid, sh.block, 0, (hipStream_t)stream, L.x, static_cast<unsigned char *>(L.codes),
                       static_cast<unsigned char *>(L.scales), L.rows, L.cols, sh.waves_per_row);
    return (int)hipGetLastError();
}

}  // namespace situ
