// Fused FC1 of routed experts + weighted SiTU-GLU on the MFMA matrix cores.
//
// What it computes (Megatron-LM PR "[Dev] Add SiTU-GLU through Transformer
// Engine", section "Design": routed experts run FC1 as a grouped GEMM, and a
// SiTU-capable cuDNN frontend fuses that grouped GEMM with the scaled
// SiTU-GLU; the activation itself as in section "Activation" and NeMo
// AutoModel "kimi_k3.situ", `_situ_fwd_core`):
//   rows of x [M, K] are grouped by expert: expert e owns rows
//   offsets[e] .. offsets[e+1];  w [E, 2I, K] holds every expert's FC1
//   weight, gate rows first;  for a row m of expert e
//     G = x_m . w_e[j],  U = x_m . w_e[I + j]          (j < I)
//     Y[m, j] = r_m * T_g(G) * T_u(U)
//   with the projections kept in fp32 accumulators (never rounded to bf16
//   before the activation) and Y rounded once to bf16.  Optionally the
//   projections are also written, rounded to bf16, as gate_up [M, 2I] for a
//   later backward.
//
// Tiling (CDNA4, 64-wide wavefronts):
//   * a workgroup of 256 threads (4 wavefronts) computes a tile of kBM = 128
//     rows x kBN = 128 output columns, i.e. 128 gate and the 128 matching up
//     projection columns.  Wavefront (wm, wn) owns rows wm*64.. and output
//     columns wn*64..: 2 x 2 blocks of 32 x 32 for G and the same for U, 8
//     accumulators of v_mfma_f32_32x32x16_bf16.  G and U of one output
//     element sit in the same lane and register, so the activation is applied
//     on the accumulators directly.
//   * the hidden axis is consumed in stages of kBK = 64: x and w tiles are
//     loaded from global memory into registers one stage ahead and written to
//     one of two LDS buffers (rows padded to 144 bytes so that the 16-byte
//     fragment reads of 32 consecutive rows fall in distinct banks); one
//     barrier per stage.
//   * the epilogue stages the bf16 results in LDS and writes whole 16-byte
//     vectors of each row.
//
// Grouping on the device: the group offsets stay in device memory (a router
// produces them there).  Row tiles are numbered by slots: expert e's tiles
// occupy slots floor(offsets[e] / kBM) + e onwards, which never overlap the
// next expert's and need at most floor(M / kBM) + E slots in total; a slot
// past an expert's rows exits at once.  Each workgroup finds its expert with
// one parallel comparison over the offsets.
#include "situ_glu_device.h"

namespace situ {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kBM = 128;               // rows of a tile
constexpr int kBN = 128;               // output columns of a tile
constexpr int kBK = 64;                // hidden elements per stage
constexpr int kThreads = 256;
constexpr int kRowBytes = kBK * 2 + 16;             // padded LDS row: 144 bytes
constexpr int kARows = kBM, kBRows = 2 * kBN;       // x rows, then gate rows and up rows
constexpr int kStageBytes = (kARows + kBRows) * kRowBytes;  // 55296
constexpr int kYRowBytes = kBN * 2 + 16;            // epilogue staging row of Y (272 bytes)
constexpr int kGuRowBytes = 2 * kBN * 2 + 16;       // epilogue staging row of G|U (528 bytes)
static_assert(kBM * (kYRowBytes + kGuRowBytes) <= 2 * kStageBytes, "epilogue staging must fit");
#ifndef SITU_GEMM_GROUP_M
#define SITU_GEMM_GROUP_M 16
#endif
constexpr int kGroupM = SITU_GEMM_GROUP_M;          // row tiles of a super tile

__device__ __forceinline__ uint4 gload(rsrc_t r, uint32_t voff, uint32_t soff)
{
    // x and w are re-read by other workgroups: default cache policy
    const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(r, (int)voff, (int)soff, 0);
    return make_uint4(v.x, v.y, v.z, v.w);
}

// Tile (slot, column tile) of a linear workgroup index: super tiles of
// kGroupM row slots x all column tiles, row slots fastest inside, so that the
// workgroups in flight share x rows and one expert's weight.
__device__ __forceinline__ void tile_of(int L, int slots, int ntn, int &rt, int &ct)
{
    const int per = kGroupM * ntn;
    const int s = L / per, p = L - s * per;
    const int gm = min(kGroupM, slots - s * kGroupM);
    rt = s * kGroupM + p % gm;
    ct = p / gm;
}

__device__ __forceinline__ void st_bf16(char *p, float v)
{
    *reinterpret_cast<uint16_t *>(p) = f32_to_bf16(v);
}

template <bool LB, bool FAST, bool GU>
__global__ void __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(1, 1)))
situ_glu_grouped_fwd_kernel(const void *__restrict__ x, const void *__restrict__ w,
                            const int32_t *__restrict__ offsets, int64_t rows, int hidden, int experts,
                            int inter, int slots, const void *__restrict__ rw, int rw_bf16, int64_t rw_stride,
                            void *__restrict__ out, void *__restrict__ gate_up, GateK gk, UpK uk)
{
    __shared__ __attribute__((aligned(16))) char smem[2 * kStageBytes];
    __shared__ float s_rs[kBM];
    __shared__ int s_expert;

    const int t = threadIdx.x;
    const int ntn = inter / kBN;
    int rt, ct;
    tile_of(blockIdx.x, slots, ntn, rt, ct);

    // ---- which expert owns row slot rt (the largest match wins on malformed offsets)
    if (t == 0)
        s_expert = -1;
    __syncthreads();
    const int M = (int)rows;
    for (int e = t; e < experts; e += kThreads) {
        const int a = min(max(offsets[e], 0), M);
        const int b = min(max(offsets[e + 1], a), M);
        const int sa = a / kBM + e, sb = b / kBM + e + 1;
        if (rt >= sa && rt < sb && a + (rt - sa) * kBM < b)
            atomicMax(&s_expert, e);
    }
    __syncthreads();
    const int e = s_expert;
    if (e < 0)
        return;  // an unused slot
    const int ga = min(max(offsets[e], 0), M);
    const int gb = min(max(offsets[e + 1], ga), M);
    const int row0 = ga + (rt - (ga / kBM + e)) * kBM;
    const int nrows = min(kBM, gb - row0);
    const int n0 = ct * kBN;

    // ---- per-row scale r * b1 (* b2), zero past the tile's rows
    if (t < kBM) {
        float r = 0.0f;
        if (t < nrows)
            r = load_rw(rw, rw_bf16, (int64_t)(row0 + t) * rw_stride);
        s_rs[t] = LB ? r * gk.beta1 * uk.beta2 : r * gk.beta1;
    }

    // ---- operand descriptors: the tile's x rows, its gate rows and its up rows
    const uint32_t kbytes = (uint32_t)hidden * 2u;
    const char *xb = static_cast<const char *>(x) + (int64_t)row0 * kbytes;
    const char *wb = static_cast<const char *>(w) + ((int64_t)e * 2 * inter + n0) * kbytes;
    const rsrc_t ra = make_rsrc(xb, (uint32_t)nrows * kbytes);  // rows past the tile read as zero
    const rsrc_t rg = make_rsrc(wb, (uint32_t)kBN * kbytes);
    const rsrc_t ru = make_rsrc(wb + (int64_t)inter * kbytes, (uint32_t)kBN * kbytes);

    // loader role: 8 threads per 128-byte row segment, 32 rows per pass
    const int lrow = t >> 3, lch = t & 7;
    uint32_t voff[4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
        voff[i] = (uint32_t)(lrow + 32 * i) * kbytes + (uint32_t)lch * 16u;
    const uint32_t lds_w = (uint32_t)lrow * kRowBytes + (uint32_t)lch * 16u;

    // compute role
    const int lane = t & 63, wv = t >> 6;
    const int wm = wv >> 1, wn = wv & 1;
    const int l32 = lane & 31, lh = lane >> 5;
    const uint32_t a_rd = (uint32_t)(wm * 64 + l32) * kRowBytes + (uint32_t)lh * 16u;
    const uint32_t g_rd = (uint32_t)(kARows + wn * 64 + l32) * kRowBytes + (uint32_t)lh * 16u;
    const uint32_t u_rd = g_rd + (uint32_t)kBN * kRowBytes;

    uint4 rx[4], rgw[4], ruw[4];
    auto fetch = [&](int kt) {
        const uint32_t so = (uint32_t)kt * (kBK * 2);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            rx[i] = gload(ra, voff[i], so);
            rgw[i] = gload(rg, voff[i], so);
            ruw[i] = gload(ru, voff[i], so);
        }
    };
    auto stash = [&](int buf) {
        char *s = smem + buf * kStageBytes + lds_w;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            *reinterpret_cast<uint4 *>(s + (32 * i) * kRowBytes) = rx[i];
            *reinterpret_cast<uint4 *>(s + (kARows + 32 * i) * kRowBytes) = rgw[i];
            *reinterpret_cast<uint4 *>(s + (kARows + kBN + 32 * i) * kRowBytes) = ruw[i];
        }
    };

    f32x16 accg[2][2], accu[2][2];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            accg[i][j] = f32x16{};
            accu[i][j] = f32x16{};
        }

    auto compute = [&](int buf) {
        const char *s = smem + buf * kStageBytes;
#pragma unroll
        for (int kk = 0; kk < kBK / 16; ++kk) {
            bf16x8 a[2], bg[2], bu[2];
#pragma unroll
            for (int i = 0; i < 2; ++i) {
                a[i] = *reinterpret_cast<const bf16x8 *>(s + a_rd + i * 32 * kRowBytes + kk * 32);
                bg[i] = *reinterpret_cast<const bf16x8 *>(s + g_rd + i * 32 * kRowBytes + kk * 32);
                bu[i] = *reinterpret_cast<const bf16x8 *>(s + u_rd + i * 32 * kRowBytes + kk * 32);
            }
#pragma unroll
            for (int i = 0; i < 2; ++i)
#pragma unroll
                for (int j = 0; j < 2; ++j) {
                    accg[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[i], bg[j], accg[i][j], 0, 0, 0);
                    accu[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[i], bu[j], accu[i][j], 0, 0, 0);
                }
        }
    };

    const int nk = hidden / kBK;
    fetch(0);
    stash(0);
    __syncthreads();
    for (int kt = 0; kt + 1 < nk; ++kt) {
        fetch(kt + 1);
        // keep the next stage's loads in flight across the whole compute phase
        __builtin_amdgcn_sched_barrier(0);
        compute(kt & 1);
        stash((kt + 1) & 1);
        __syncthreads();
    }
    compute((nk - 1) & 1);
    __syncthreads();  // every wavefront is done with the stage buffers

    // ---- epilogue: activation on the accumulators, staged through LDS as bf16
    char *sy = smem;                            // [kBM][kYRowBytes]
    char *sgu = smem + kBM * kYRowBytes;        // [kBM][kGuRowBytes]
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                // MFMA 32x32 result layout: register r of lane l holds row
                // (r/4)*8 + (l/32)*4 + r%4, column l%32 of the block
                const int row = wm * 64 + i * 32 + (r >> 2) * 8 + lh * 4 + (r & 3);
                const int col = wn * 64 + j * 32 + l32;
                const float g = accg[i][j][r], u = accu[i][j][r];
                st_bf16(sy + row * kYRowBytes + col * 2, fwd_elem<LB, FAST, false>(g, u, s_rs[row], gk, uk));
                if (GU) {
                    st_bf16(sgu + row * kGuRowBytes + col * 2, g);
                    st_bf16(sgu + row * kGuRowBytes + (kBN + col) * 2, u);
                }
            }
    __syncthreads();

    // Y: 16 vectors of 16 bytes per row, 16 rows per pass
    const uint32_t ybytes = (uint32_t)inter * 2u;
    const rsrc_t ro = make_rsrc(static_cast<char *>(out) + (int64_t)row0 * ybytes, (uint32_t)nrows * ybytes);
    {
        const int c = t & 15, r0 = t >> 4;
#pragma unroll
        for (int p = 0; p < kBM / 16; ++p) {
            const int row = r0 + 16 * p;
            const uint4 v = *reinterpret_cast<const uint4 *>(sy + row * kYRowBytes + c * 16);
            // rows past the tile fall outside the descriptor: the store is dropped
            bstore(ro, (uint32_t)row * ybytes + (uint32_t)(n0 * 2 + c * 16), v);
        }
    }
    if (GU) {
        const uint32_t gbytes = 2u * ybytes;
        const rsrc_t rq =
            make_rsrc(static_cast<char *>(gate_up) + (int64_t)row0 * gbytes, (uint32_t)nrows * gbytes);
        const int c = t & 31, r0 = t >> 5;   // 16 gate vectors then 16 up vectors per row
        const uint32_t colb = c < 16 ? (uint32_t)(n0 * 2 + c * 16) : (uint32_t)((inter + n0) * 2 + (c - 16) * 16);
#pragma unroll
        for (int p = 0; p < kBM / 8; ++p) {
            const int row = r0 + 8 * p;
            const uint4 v = *reinterpret_cast<const uint4 *>(sgu + row * kGuRowBytes + c * 16);
            bstore(rq, (uint32_t)row * gbytes + colb, v);
        }
    }
}

using GemmFn = void (*)(const void *, const void *, const int32_t *, int64_t, int, int, int, int, const void *,
                        int, int64_t, void *, void *, GateK, UpK);

template <bool LB, bool FAST>
GemmFn pick_gu(bool gu)
{
    return gu ? situ_glu_grouped_fwd_kernel<LB, FAST, true> : situ_glu_grouped_fwd_kernel<LB, FAST, false>;
}

}  // namespace

int grouped_slots(int64_t rows, int experts) { return (int)(rows / kBM) + experts; }

int launch_grouped_fwd(const GroupedLaunch &L, void *stream)
{
    const int slots = grouped_slots(L.rows, L.experts);
    const int64_t blocks = (int64_t)slots * (L.inter / kBN);
    if (blocks <= 0)
        return 0;
    GemmFn fn = L.lb ? (L.fast ? pick_gu<true, true>(L.gate_up) : pick_gu<true, false>(L.gate_up))
                     : (L.fast ? pick_gu<false, true>(L.gate_up) : pick_gu<false, false>(L.gate_up));
    hipLaunchKernelGGL(fn, dim3((unsigned)blocks), dim3(kThreads), 0, static_cast<hipStream_t>(stream), L.x, L.w,
                       L.offsets, L.rows, L.hidden, L.experts, L.inter, slots, L.rw, L.rw_bf16, L.rw_stride, L.out,
                       L.gate_up, L.gk, L.uk);
    return (int)hipGetLastError();
}

}  // namespace situ
