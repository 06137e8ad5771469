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
//   * a workgroup of 256 threads (4 wavefronts) computes a tile of kBM = 256
//     rows x kBN = 128 output columns, i.e. 128 gate and the 128 matching up
//     projection columns.  Wavefront (wm, wn) owns rows wm*128.. and output
//     columns wn*64..: 4 x 2 blocks of 32 x 32 for G and the same for U, 16
//     accumulators of v_mfma_f32_32x32x16_bf16 (the whole accumulation
//     register file).  G and U of one output element sit in the same lane and
//     register, so the activation is applied on the accumulators directly.
//     Per 16-wide k step a wavefront reads 8 operand fragments from LDS for
//     16 matrix instructions.
//   * the hidden axis is consumed in stages of kBK: the x and w rows of a
//     stage go from global memory straight into LDS (16-byte buffer loads
//     that write LDS, no register staging), one stage ahead of the one being
//     multiplied; one barrier per stage.  Rows are not padded:
//     chunk c (16 bytes) of row R is stored at chunk c ^ f(R), a swizzle
//     under which the fragment reads of 16 consecutive rows hit distinct
//     banks.
//   * the epilogue stages the bf16 results in LDS and writes whole 16-byte
//     vectors of each row.
//
// Grouping on the device: the group offsets stay in device memory (a router
// produces them there).  Row tiles are numbered by slots: expert e's tiles
// occupy slots floor(offsets[e] / kBM) + e onwards, which never overlap the
// next expert's and need at most floor(M / kBM) + E slots in total; a slot
// past an expert's rows exits at once.  Each workgroup finds its expert with
// one parallel comparison over the offsets.
#include <type_traits>

#include "situ_glu_device.h"

namespace situ {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kBM = 256;               // rows of a tile
constexpr int kBN = 128;               // output columns of a tile
constexpr int kBK = 64;                // hidden elements per stage (two stage buffers)
constexpr int kThreads = 256;
constexpr int kCh = kBK / 8;                        // 16-byte chunks of a row in one stage
constexpr int kRowB = kBK * 2;                      // bytes of a row in one stage
constexpr int kRowsPerBank = 256 / kRowB;           // rows per 256 bytes (the bank period)
constexpr int kARows = kBM, kBRows = 2 * kBN;       // x rows, then gate rows and up rows
constexpr int kStageBytes = (kARows + kBRows) * kRowB;
constexpr int kRowsPerLoad = 64 / kCh;              // rows one wavefront-wide load fills
constexpr int kLoads = (kARows + kBRows) / kRowsPerLoad / 4;  // loads per thread and stage
constexpr int kYRowBytes = kBN * 2 + 16;            // epilogue staging row (272 bytes)
constexpr int kEpiBytes = kBM * kYRowBytes;         // one staged [kBM, kBN] bf16 block
static_assert(kBK % 16 == 0 && kCh * kRowsPerBank == 16, "the swizzle assumes 16 rows per bank cycle");
static_assert(kLoads == 2 * kCh, "x and w rows split evenly over the loads");
constexpr int kBufBytes = kStageBytes > kEpiBytes ? kStageBytes : kEpiBytes;
constexpr int kGroupM = 16;            // row tiles of a super tile (column tiles not a multiple of 16)
constexpr int kXcdRows = 8;            // row tiles of an XCD's block in the XCD-aware order (x 4 columns)
constexpr int kFirstLoads = 8;         // of a stage's 16 loads per thread: issued at the boundary, the rest
                                       // during the next k step
constexpr int kLoadSpacing = 2;        // products between consecutive loads

using lds_ptr_t = __attribute__((address_space(3))) void *;

// the swizzle of row r: logical chunk c of the row sits in slot c ^ swz(r)
__device__ __forceinline__ int swz(int r) { return (r / kRowsPerBank) % kCh; }

// Tile (slot, column tile) of workgroup b.  Workgroups are dealt to the 8
// XCDs round robin (b % 8), each XCD with its own L2, and 256 (one per CU)
// run at a time.  With the column tiles a multiple of 16, one such wave of
// 256 covers a super tile of 16 row slots x 16 column tiles, and inside it
// XCD x takes the 8 x 4 block of rows (x % 2) * 8.. and columns (x / 2) * 4..:
// its 32 workgroups then share 8 x tiles and 4 weight tiles in its L2 (every
// stage needs 12 distinct tiles, not 32 x 2).  Otherwise super tiles of
// kGroupM row slots x all column tiles, row slots fastest.  Returns false
// for a workgroup past the grid's real tiles.
__device__ __forceinline__ bool tile_of(int b, int slots, int ntn, int &rt, int &ct)
{
    if (ntn % 16 == 0) {
        const int x = b & 7, k = b >> 3;
        const int round = k >> 5, q = k & 31;
        const int scols = ntn >> 4;
        const int sr = round / scols, sc = round - sr * scols;
        constexpr int XR = kXcdRows, XC = 32 / XR, NR = 16 / XR;
        rt = sr * 16 + (x % NR) * XR + q % XR;
        ct = sc * 16 + (x / NR) * XC + q / XR;
        return rt < slots;
    }
    const int per = kGroupM * ntn;
    const int s = b / per, p = b - s * per;
    const int gm = min(kGroupM, slots - s * kGroupM);
    rt = s * kGroupM + p % gm;
    ct = p / gm;
    return true;
}

// Workgroups in the grid: whole super tiles in the XCD mapping.
__host__ __device__ inline int64_t grid_blocks(int slots, int ntn)
{
    if (ntn % 16 == 0)
        return (int64_t)((slots + 15) / 16) * 16 * ntn;
    return (int64_t)slots * ntn;
}

__device__ __forceinline__ void st_bf16(char *p, float v)
{
    *reinterpret_cast<uint16_t *>(p) = f32_to_bf16(v);
}

// s_waitcnt with only the vector-memory counter constrained (gfx9 encoding:
// vmcnt bits 3:0 and 15:14, expcnt 6:4 and lgkmcnt 11:8 left at their maxima)
template <int N>
__device__ __forceinline__ void wait_vmcnt()
{
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

template <bool LB, bool FAST, bool GU>
__global__ void __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(1, 1)))
situ_glu_grouped_fwd_kernel(const void *__restrict__ x, const void *__restrict__ w,
                            const int32_t *__restrict__ offsets, int64_t rows, int hidden, int experts,
                            int inter, int slots, const void *__restrict__ rw, int rw_bf16, int64_t rw_stride,
                            void *__restrict__ out, void *__restrict__ gate_up, GateK gk, UpK uk)
{
    // Two stage buffers as two objects: the compiler then knows that loads
    // landing in one do not alias the fragment reads of the other, and does
    // not make those reads wait for the loads in flight.
    __shared__ __attribute__((aligned(1024))) char smem0[kBufBytes];
    __shared__ __attribute__((aligned(1024))) char smem1[kBufBytes];
    __shared__ float s_rs[kBM];
    __shared__ int s_expert;

    const int t = threadIdx.x;
    const int ntn = inter / kBN;
    int rt, ct;
    if (!tile_of(blockIdx.x, slots, ntn, rt, ct))
        return;  // past the last row slot (padding of the last super tile)

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
    {
        float r = 0.0f;
        if (t < nrows)
            r = load_rw(rw, rw_bf16, (int64_t)(row0 + t) * rw_stride);
        s_rs[t] = LB ? r * gk.beta1 * uk.beta2 : r * gk.beta1;
    }

    // ---- operand descriptors.  Loads of rows 0..kBM-1 of one region: x rows
    // of the tile (past nrows they read as zero), gate rows 0..kBN-1 and, via
    // a base kBN rows early, up rows kBN..2kBN-1 of the same offsets.
    const uint32_t kbytes = (uint32_t)hidden * 2u;
    const char *xb = static_cast<const char *>(x) + (int64_t)row0 * kbytes;
    const char *wb = static_cast<const char *>(w) + ((int64_t)e * 2 * inter + n0) * kbytes;
    const rsrc_t ra = make_rsrc(xb, (uint32_t)nrows * kbytes);
    const rsrc_t rg = make_rsrc(wb, (uint32_t)kBN * kbytes);
    const rsrc_t ru = make_rsrc(wb + ((int64_t)inter - kBN) * kbytes, (uint32_t)(2 * kBN) * kbytes);

    // loader role: load j of wavefront wv fills rows (4 j + wv) * kRowsPerLoad..
    // of the 512-row stage (x rows first); lane l takes row + l / kCh and the
    // logical chunk whose slot is l % kCh.
    // the wavefront index is uniform: keep it scalar so that the LDS
    // addresses of the loads (the M0 operand) are scalar arithmetic
    const int lane = t & 63, wv = __builtin_amdgcn_readfirstlane(t >> 6);
    uint32_t voff[kCh];
#pragma unroll
    for (int j = 0; j < kCh; ++j) {
        const int r = (4 * j + wv) * kRowsPerLoad + lane / kCh;
        voff[j] = (uint32_t)r * kbytes + (uint32_t)(((lane % kCh) ^ swz(r)) * 16);
    }
    const int nk = hidden / kBK;
    const rsrc_t rz = make_rsrc(xb, 0u);  // reads as zero: the padding stage of an odd count
    auto issue = [&](int kt, auto buf, int j0 = 0, int j1 = kLoads) {
        const uint32_t so = (uint32_t)kt * kRowB;
        char *base = decltype(buf)::value ? smem1 : smem0;
        const bool live = kt < nk;
#pragma unroll
        for (int j = j0; j < j1; ++j) {
            const int blk = 4 * j + wv;
            const rsrc_t r = !live ? rz : j < kCh ? ra : (j - kCh < kCh / 2 ? rg : ru);
            __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_ptr_t)(base + blk * 1024), 16, (int)voff[j % kCh],
                                                     (int)so, 0, 0);
        }
    };

    // compute role
    const int wm = wv >> 1, wn = wv & 1;
    const int l32 = lane & 31, lh = lane >> 5;
    const int f = swz(l32);  // the swizzle of every row this lane reads (row bases are multiples of 32)
    uint32_t rda[kBK / 16], rdb[kBK / 16];
#pragma unroll
    for (int kk = 0; kk < kBK / 16; ++kk) {
        const uint32_t c = (uint32_t)(((2 * kk + lh) ^ f) * 16);
        rda[kk] = (uint32_t)(wm * 128 + l32) * kRowB + c;
        rdb[kk] = (uint32_t)(kARows + wn * 64 + l32) * kRowB + c;
    }

    f32x16 accg[4][2], accu[4][2];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            accg[i][j] = f32x16{};
            accu[i][j] = f32x16{};
        }

    struct Frags {
        bf16x8 a[4], g[2], u[2];
    };
    auto read_frags = [&](const char *s, int kk, Frags &f) {
#pragma unroll
        for (int i = 0; i < 4; ++i)
            f.a[i] = *reinterpret_cast<const bf16x8 *>(s + rda[kk] + i * 32 * kRowB);
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            f.g[j] = *reinterpret_cast<const bf16x8 *>(s + rdb[kk] + j * 32 * kRowB);
            f.u[j] = *reinterpret_cast<const bf16x8 *>(s + rdb[kk] + (kBN + j * 32) * kRowB);
        }
    };
    auto mfmas = [&](const Frags &f) {
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int j = 0; j < 2; ++j) {
                accg[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(f.a[i], f.g[j], accg[i][j], 0, 0, 0);
                accu[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(f.a[i], f.u[j], accu[i][j], 0, 0, 0);
            }
    };
    // Interleave one k step's 16 products with the 8 fragment reads of the
    // next step: a read between consecutive products keeps LDS requests
    // flowing while the matrix core works.
    auto pattern = []() {
#pragma unroll
        for (int q = 0; q < 8; ++q) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // a product
            __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // a fragment read
        }
        __builtin_amdgcn_sched_group_barrier(0x008, 8, 0);
    };
    using Buf0 = std::integral_constant<int, 0>;
    using Buf1 = std::integral_constant<int, 1>;
    Frags f0, f1;
    constexpr int kFirst = kFirstLoads, kSpread = kLoadSpacing;
    // k steps 0..2 of a stage: products of step kk, fragments of step kk + 1
    // (and the remaining loads of stage kt_next into the other buffer)
    auto first_steps = [&](auto buf, int kt_next) {
        const char *s = decltype(buf)::value ? smem1 : smem0;
        read_frags(s, 1, f1);
        if (kFirst < kLoads)
            issue(kt_next, std::integral_constant<int, 1 - decltype(buf)::value>{}, kFirst, kLoads);
        mfmas(f0);
        if (kFirst < kLoads) {
#pragma unroll
            for (int q = 0; q < 16; ++q) {
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                if (q % kSpread == 0 && q / kSpread < kLoads - kFirst)
                    __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
                if (q < 8)
                    __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
            }
        } else {
            pattern();
        }
        read_frags(s, 2, f0);
        mfmas(f1);
        pattern();
        read_frags(s, 3, f1);
        mfmas(f0);
        pattern();
    };
    // the stage boundary: once every wavefront has read its last fragments of
    // the stage in `buf` and its loads of the next stage (other buffer) have
    // landed, one barrier; then the next stage's first fragments and the
    // loads of stage kt_next (into `buf`) go out while the last 16 products
    // of the stage run
    auto boundary = [&](auto buf, int kt_next) {
        constexpr int nb = 1 - decltype(buf)::value;
        wait_vmcnt<0>();
        __syncthreads();
        read_frags(nb ? smem1 : smem0, 0, f0);
        issue(kt_next, buf, 0, kFirst);
        mfmas(f1);
        __builtin_amdgcn_sched_group_barrier(0x100, 8, 0);
#pragma unroll
        for (int q = 0; q < 16; ++q) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
            if (q % kSpread == 0 && q / kSpread < kFirst)
                __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
        }
        __builtin_amdgcn_sched_barrier(0);
    };

    // ---- main loop.  Stage kt lives in buffer kt % 2; the loads of stage
    // kt + 1 are in flight while stage kt is multiplied.  The body is two
    // stages (one per buffer) with no tail: an odd stage count gets one more
    // stage of zeros (an empty descriptor), which adds nothing.
    issue(0, Buf0{});
    wait_vmcnt<0>();
    __syncthreads();
    read_frags(smem0, 0, f0);
    issue(1, Buf1{}, 0, kFirst);
    // (the second half of stage 1's loads: issued with stage 0's first step)
    for (int kt = 0; kt < nk; kt += 2) {
        first_steps(Buf0{}, kt + 1);
        boundary(Buf0{}, kt + 2);
        first_steps(Buf1{}, kt + 2);
        boundary(Buf1{}, kt + 3);
    }
    wait_vmcnt<0>();  // loads past the last stage (zeros) have landed
    __syncthreads();  // every wavefront is done with the stage buffers

    // ---- epilogue: activation on the accumulators, staged through LDS as bf16
    char *sy = smem0;
    char *sg = smem1;
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                // MFMA 32x32 result layout: register r of lane l holds row
                // (r/4)*8 + (l/32)*4 + r%4, column l%32 of the block
                const int row = wm * 128 + i * 32 + (r >> 2) * 8 + lh * 4 + (r & 3);
                const int col = wn * 64 + j * 32 + l32;
                const float g = accg[i][j][r], u = accu[i][j][r];
                st_bf16(sy + row * kYRowBytes + col * 2, fwd_elem<LB, FAST, false>(g, u, s_rs[row], gk, uk));
                if (GU)
                    st_bf16(sg + row * kYRowBytes + col * 2, g);
                // one 32 x 32 block at a time: bounds the registers the
                // activation takes while all accumulators are still live
                if (r == 15)
                    __builtin_amdgcn_sched_barrier(0);
            }
    __syncthreads();

    // whole rows of 16 vectors of 16 bytes, 16 rows per pass; rows past the
    // tile fall outside the descriptors and their stores are dropped
    const int c16 = t & 15, r16 = t >> 4;
    const uint32_t ybytes = (uint32_t)inter * 2u;
    const rsrc_t ro = make_rsrc(static_cast<char *>(out) + (int64_t)row0 * ybytes, (uint32_t)nrows * ybytes);
#pragma unroll 4
    for (int p = 0; p < kBM / 16; ++p) {
        const int row = r16 + 16 * p;
        const uint4 v = *reinterpret_cast<const uint4 *>(sy + row * kYRowBytes + c16 * 16);
        bstore(ro, (uint32_t)row * ybytes + (uint32_t)(n0 * 2 + c16 * 16), v);
    }
    if (GU) {
        const uint32_t gbytes = 2u * ybytes;
        const rsrc_t rq =
            make_rsrc(static_cast<char *>(gate_up) + (int64_t)row0 * gbytes, (uint32_t)nrows * gbytes);
#pragma unroll 4
        for (int p = 0; p < kBM / 16; ++p) {
            const int row = r16 + 16 * p;
            const uint4 v = *reinterpret_cast<const uint4 *>(sg + row * kYRowBytes + c16 * 16);
            bstore(rq, (uint32_t)row * gbytes + (uint32_t)(n0 * 2 + c16 * 16), v);
        }
        __syncthreads();
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int j = 0; j < 2; ++j)
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int row = wm * 128 + i * 32 + (r >> 2) * 8 + lh * 4 + (r & 3);
                    const int col = wn * 64 + j * 32 + l32;
                    st_bf16(sy + row * kYRowBytes + col * 2, accu[i][j][r]);
                }
        __syncthreads();
#pragma unroll 4
        for (int p = 0; p < kBM / 16; ++p) {
            const int row = r16 + 16 * p;
            const uint4 v = *reinterpret_cast<const uint4 *>(sy + row * kYRowBytes + c16 * 16);
            bstore(rq, (uint32_t)row * gbytes + (uint32_t)((inter + n0) * 2 + c16 * 16), v);
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

int64_t grouped_slots(int64_t rows, int64_t experts) { return rows / kBM + experts; }

int64_t grouped_grid_blocks(int64_t rows, int64_t experts, int64_t inter)
{
    const int64_t slots = grouped_slots(rows, experts), ntn = inter / kBN;
    return ntn % 16 == 0 ? (slots + 15) / 16 * 16 * ntn : slots * ntn;
}

int launch_grouped_fwd(const GroupedLaunch &L, void *stream)
{
    const int slots = (int)grouped_slots(L.rows, L.experts);
    const int64_t blocks = grid_blocks(slots, L.inter / kBN);
    if (blocks <= 0)
        return 0;
    if (blocks > 0x7fffffff)
        return (int)hipErrorInvalidConfiguration;  // the host API rejects such shapes first
    GemmFn fn = L.lb ? (L.fast ? pick_gu<true, true>(L.gate_up) : pick_gu<true, false>(L.gate_up))
                     : (L.fast ? pick_gu<false, true>(L.gate_up) : pick_gu<false, false>(L.gate_up));
    hipLaunchKernelGGL(fn, dim3((unsigned)blocks), dim3(kThreads), 0, static_cast<hipStream_t>(stream), L.x, L.w,
                       L.offsets, L.rows, L.hidden, L.experts, L.inter, slots, L.rw, L.rw_bf16, L.rw_stride, L.out,
                       L.gate_up, L.gk, L.uk);
    return (int)hipGetLastError();
}

}  // namespace situ
