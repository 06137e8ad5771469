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
//   * the hidden axis is consumed in stages of kBK, two LDS stage buffers,
//     one barrier per stage.  The x and w rows of a stage come in as 16-byte
//     buffer loads (16 per thread and stage) into a ring of registers that
//     holds two stages: during stage kt each slot of stage kt + 1 is written
//     to the free LDS buffer and at once reloaded with stage kt + 3, so every
//     load has two stages to land and the loads go out evenly over the
//     stage.  Rows are not padded: chunk c (16 bytes) of row R is stored at
//     chunk c ^ f(R), a swizzle under which the fragment reads of 16
//     consecutive rows hit distinct banks.
//   * the epilogue stages the bf16 results in LDS and writes whole 16-byte
//     vectors of each row.
//
// MX fp8 operands (E4M3 or E5M2 codes, one E8M0 scale byte per 32 values
// along the hidden axis): the same tiling with 128 hidden values per 128-byte
// stage row, two 64-wide k steps of v_mfma_scale_f32_32x32x64_f8f6f4 per
// stage, each lane giving the scale byte of its row and 32-wide block; the
// operands and scale bytes of a stage go from global memory straight into
// LDS (buffer loads that write LDS) one stage ahead, instead of through the
// register ring.  A lane's 32 operand bytes are two 16-byte chunks of the step, taken in an
// order (the same for both operands) under which the instruction's first 32
// k are exactly the step's first MX block.  The kernel takes the scale bytes
// stage-major, one dword (the 4 scale bytes of a stage) per row and stage,
// rows contiguous: situ_mx_scales_stage_major_kernel rewrites the row-major
// MX scale arrays that way first, so that one 64-lane load of a stage's
// scales covers 64 consecutive rows (256 contiguous bytes) instead of
// touching 64 cache lines, one per row.  The scaled instruction truncates
// each group of 8 products to 13 bits below the group's largest exponent sum
// before adding them, so on these operands a projection carries that
// instruction's rounding, not fp32's.
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
typedef int i32x8 __attribute__((ext_vector_type(8)));

// Operand kinds: bf16, or MX block-scaled fp8 (E4M3 / E5M2 codes with one
// E8M0 scale byte per 32 values along the hidden axis).
enum { OP_BF16 = 0, OP_E4M3 = 1, OP_E5M2 = 2 };

// Stage stride (dwords) of a stage-major scale array of R rows: R rounded up
// to a whole 128-byte line, plus one line, so that the stages of a tile's
// rows do not all fall into the same L2 sets (an unpadded stride of 64 Ki
// rows is 256 KiB).
__host__ __device__ inline int64_t stage_stride(int64_t R) { return (R + 31) / 32 * 32 + 32; }

constexpr int kBM = 256;               // rows of a tile
constexpr int kBN = 128;               // output columns of a tile
constexpr int kBK = 64;                // bf16 hidden elements per stage (two stage buffers)
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
// fp8 operands go from global memory straight into LDS (buffer loads that
// write LDS), one stage ahead: of a stage's 16 loads per thread, 12 at the
// stage boundary, the rest one per product of the next k step (two k steps
// per stage, each product twice the work of a bf16 one)
constexpr int kFirstLoadsF8 = 12;
constexpr int kLoadSpacingF8 = 1;
// bf16: register ring slots written to LDS (each followed by its reload) in
// k steps 0, 1 and 2 of a stage; the slots must be in LDS before the stage's
// barrier
constexpr int kRingMoves0 = 6, kRingMoves1 = 11;

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

template <int OP, bool LB, bool FAST, bool GU>
__global__ void __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(1, 1)))
situ_glu_grouped_fwd_kernel(const void *__restrict__ x, const void *__restrict__ w,
                            const uint8_t *__restrict__ xs, const uint8_t *__restrict__ ws,
                            const int32_t *__restrict__ offsets, int64_t rows, int hidden, int experts,
                            int inter, int slots, const void *__restrict__ rw, int rw_bf16, int64_t rw_stride,
                            void *__restrict__ out, void *__restrict__ gate_up, GateK gk, UpK uk)
{
    // bf16: 64 hidden elements per 128-byte stage row, four 16-wide k steps;
    // fp8: 128 per row, two 64-wide k steps of scaled products
    constexpr bool F8 = OP != OP_BF16;
    constexpr int kStageK = F8 ? 128 : kBK;
    constexpr int kSteps = F8 ? 2 : 4;
    constexpr int kFragReads = F8 ? 16 : 8;  // LDS reads of one k step's fragments
    // Two stage buffers as two objects: the compiler then knows that loads
    // landing in one do not alias the fragment reads of the other, and does
    // not make those reads wait for the loads in flight.
    __shared__ __attribute__((aligned(1024))) char smem0[kBufBytes];
    __shared__ __attribute__((aligned(1024))) char smem1[kBufBytes];
    // fp8: the stage's scale bytes, one dword (4 blocks of 32) per x row (0..255)
    // and per gate / up row (256..511), per buffer
    __shared__ __attribute__((aligned(16))) uint32_t ssc0[F8 ? 2 * kBM : 1];
    __shared__ __attribute__((aligned(16))) uint32_t ssc1[F8 ? 2 * kBM : 1];
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
    const uint32_t kbytes = (uint32_t)hidden * (F8 ? 1u : 2u);
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
    const int nk = hidden / kStageK;
    const rsrc_t rz = make_rsrc(xb, 0u);  // reads as zero: the padding stage of an odd count
    // fp8 scales, stage-major: the dword of row r for stage kt is at
    // kt * stage_stride(R) + r (R = rows for x, E * 2I for w; stage_stride(R)
    // * nk < 2^30, checked on the host, so byte offsets fit 32 bits).  The descriptors start at the
    // tile's first row and end with the array: rows past the tile read other
    // rows' scales, which only multiply the zero codes of those rows
    // (results never stored)
    const uint32_t sxs = (uint32_t)stage_stride(rows) * 4u;
    const uint32_t sws = (uint32_t)stage_stride((int64_t)experts * 2 * inter) * 4u;
    rsrc_t rsa = rz, rsg = rz, rsu = rz;
    if (F8) {
        const uint32_t xend = (uint32_t)nk * sxs, wend = (uint32_t)nk * sws;
        rsa = make_rsrc(xs + (int64_t)row0 * 4, xend - (uint32_t)row0 * 4u);
        const uint32_t wg = ((uint32_t)e * 2u * (uint32_t)inter + (uint32_t)n0) * 4u;
        const uint32_t wu = wg + ((uint32_t)inter - kBN) * 4u;
        rsg = make_rsrc(ws + wg, wend - wg);
        rsu = make_rsrc(ws + wu, wend - wu);
    }
    // wavefront wv loads the stage's scale dwords of x rows and of w rows
    // 64 wv..64 wv + 63 (the up rows via a base kBN rows early, as for the
    // operands)
    auto issue_scales = [&](int kt, auto buf) {
        if (!F8)
            return;
        uint32_t *base = decltype(buf)::value ? ssc1 : ssc0;
        const bool live = kt < nk;
        const uint32_t vo = (uint32_t)(64 * wv + lane) * 4u;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(live ? rsa : rz, (lds_ptr_t)(base + 64 * wv), 4, (int)vo,
                                                 (int)((uint32_t)kt * sxs), 0, 0);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(live ? (wv < 2 ? rsg : rsu) : rz,
                                                 (lds_ptr_t)(base + kBM + 64 * wv), 4, (int)vo,
                                                 (int)((uint32_t)kt * sws), 0, 0);
    };
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
    // fragment addresses of each k step.  bf16: 16 bytes at logical chunk
    // 2 kk + lh.  fp8: two 16-byte pieces at chunks 4 s + lh and 4 s + 2 + lh,
    // which the scaled product takes as its 32 bytes in the order k =
    // 16 c + 8 lh + (0..7) (c = 8-byte piece): a consistent permutation of
    // the 64 k of the step for both operands that keeps each 32-wide scale
    // block (hardware k 0..31 = this step's first MX block) whole
    uint32_t rda[kSteps][F8 ? 2 : 1], rdb[kSteps][F8 ? 2 : 1];
#pragma unroll
    for (int st = 0; st < kSteps; ++st)
#pragma unroll
        for (int h = 0; h < (F8 ? 2 : 1); ++h) {
            const int chunk = F8 ? 4 * st + 2 * h + lh : 2 * st + lh;
            const uint32_t c = (uint32_t)((chunk ^ f) * 16);
            rda[st][h] = (uint32_t)(wm * 128 + l32) * kRowB + c;
            rdb[st][h] = (uint32_t)(kARows + wn * 64 + l32) * kRowB + c;
        }

    f32x16 accg[4][2], accu[4][2];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            accg[i][j] = f32x16{};
            accu[i][j] = f32x16{};
        }

    using FragT = typename std::conditional<F8, i32x8, bf16x8>::type;
    struct Frags {
        FragT a[4], g[2], u[2];
    };
    auto frag = [&](const char *s, uint32_t r0, uint32_t r1, int off) -> FragT {
        if constexpr (F8) {
            const u32x4 lo = *reinterpret_cast<const u32x4 *>(s + r0 + off);
            const u32x4 hi = *reinterpret_cast<const u32x4 *>(s + r1 + off);
            return i32x8{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
        } else {
            return *reinterpret_cast<const bf16x8 *>(s + r0 + off);
        }
    };
    auto read_frags = [&](const char *s, int st, Frags &fr) {
        const uint32_t a0 = rda[st][0], a1 = rda[st][F8 ? 1 : 0];
        const uint32_t b0 = rdb[st][0], b1 = rdb[st][F8 ? 1 : 0];
#pragma unroll
        for (int i = 0; i < 4; ++i)
            fr.a[i] = frag(s, a0, a1, i * 32 * kRowB);
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            fr.g[j] = frag(s, b0, b1, j * 32 * kRowB);
            fr.u[j] = frag(s, b0, b1, (kBN + j * 32) * kRowB);
        }
    };
    // fp8: scale dwords of the rows this lane feeds (x rows of a[i], weight
    // rows of g[j] / u[j]); byte 2 st + lh is the scale of step st's block lh
    struct Scales {
        uint32_t a[4], g[2], u[2];
    };
    auto read_scales = [&](const uint32_t *sc, Scales &q) {
#pragma unroll
        for (int i = 0; i < 4; ++i)
            q.a[i] = sc[wm * 128 + i * 32 + l32];
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            q.g[j] = sc[kBM + wn * 64 + j * 32 + l32];
            q.u[j] = sc[kBM + kBN + wn * 64 + j * 32 + l32];
        }
    };
    constexpr int kCbsz = OP == OP_E5M2 ? 1 : 0;  // operand format of the scaled product (same for both)
    auto mfmas = [&](const Frags &fr, const Scales &q, int st) {
        const uint32_t sh = (uint32_t)(8 * (2 * st + lh));
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int j = 0; j < 2; ++j) {
                if constexpr (F8) {
                    const int sa = (int)(q.a[i] >> sh);
                    accg[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
                        fr.a[i], fr.g[j], accg[i][j], kCbsz, kCbsz, 0, sa, 0, (int)(q.g[j] >> sh));
                    accu[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
                        fr.a[i], fr.u[j], accu[i][j], kCbsz, kCbsz, 0, sa, 0, (int)(q.u[j] >> sh));
                } else {
                    accg[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fr.a[i], fr.g[j], accg[i][j], 0, 0, 0);
                    accu[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fr.a[i], fr.u[j], accu[i][j], 0, 0, 0);
                }
            }
    };
    using Buf0 = std::integral_constant<int, 0>;
    using Buf1 = std::integral_constant<int, 1>;
    Frags f0, f1;
    Scales q0, q1;  // scales of the stage in buffer 0 / buffer 1 (fp8)
    constexpr int kFirst = kFirstLoadsF8, kSpread = kLoadSpacingF8;
    // fp8, k step 0 of a stage: its products, fragments of step 1 (and the
    // remaining loads of stage kt_next into the other buffer)
    auto first_steps = [&](auto buf, int kt_next) {
        const char *s = decltype(buf)::value ? smem1 : smem0;
        const Scales &q = decltype(buf)::value ? q1 : q0;
        read_frags(s, 1, f1);
        issue(kt_next, std::integral_constant<int, 1 - decltype(buf)::value>{}, kFirst, kLoads);
        mfmas(f0, q, 0);
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
            if (i % kSpread == 0 && i / kSpread < kLoads - kFirst)
                __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
            if (i < kFragReads)
                __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
        }
    };
    // fp8, the stage boundary: once every wavefront has read its last fragments of
    // the stage in `buf` and its loads of the next stage (other buffer) have
    // landed, one barrier; then the next stage's first fragments (and
    // scales) and the loads of stage kt_next (into `buf`) go out while the
    // last 16 products of the stage run
    auto boundary = [&](auto buf, int kt_next) {
        constexpr int nb = 1 - decltype(buf)::value;
        const Scales &q = decltype(buf)::value ? q1 : q0;
        wait_vmcnt<0>();
        __syncthreads();
        read_frags(nb ? smem1 : smem0, 0, f0);
        if (F8)
            read_scales(nb ? ssc1 : ssc0, nb ? q1 : q0);
        issue_scales(kt_next, buf);
        issue(kt_next, buf, 0, kFirst);
        mfmas(f1, q, kSteps - 1);
        __builtin_amdgcn_sched_group_barrier(0x100, F8 ? kFragReads + 8 : kFragReads, 0);
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
            if (i % kSpread == 0 && i / kSpread < kFirst + (F8 ? 2 : 0))
                __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
        }
        __builtin_amdgcn_sched_barrier(0);
    };

    // ---- main loop.  Stage kt lives in LDS buffer kt % 2.  The body is two
    // stages (one per buffer) with no tail: an odd stage count gets one more
    // stage of zeros (an empty descriptor), which adds nothing.
    if constexpr (F8) {
        // the loads of stage kt + 1 are in flight into the other buffer while
        // stage kt is multiplied
        issue_scales(0, Buf0{});
        issue(0, Buf0{});
        wait_vmcnt<0>();
        __syncthreads();
        read_frags(smem0, 0, f0);
        if (F8)
            read_scales(ssc0, q0);
        issue_scales(1, Buf1{});
        issue(1, Buf1{}, 0, kFirst);
        for (int kt = 0; kt < nk; kt += 2) {
            first_steps(Buf0{}, kt + 1);
            boundary(Buf0{}, kt + 2);
            first_steps(Buf1{}, kt + 2);
            boundary(Buf1{}, kt + 3);
        }
    } else {
        // register ring: ring0 / ring1 hold the even / odd stages in flight,
        // slot j of a stage = load j of this thread
        u32x4 ring0[kLoads], ring1[kLoads];
        auto gload = [&](int kt, int j) -> u32x4 {
            const rsrc_t r = kt >= nk ? rz : j < kCh ? ra : (j - kCh < kCh / 2 ? rg : ru);
            return __builtin_amdgcn_raw_buffer_load_b128(r, (int)voff[j % kCh], (int)((uint32_t)kt * kRowB), 0);
        };
        // slot j lands where the direct-to-LDS load j would write: 1 KiB block
        // 4 j + wv, 16 bytes per lane
        auto lwrite = [&](char *base, int j, const u32x4 &v) {
            *reinterpret_cast<u32x4 *>(base + (4 * j + wv) * 1024 + lane * 16) = v;
        };
        // a barrier that waits for this wavefront's LDS operations only (the
        // ring's global loads stay in flight); the empty asm statements keep
        // the compiler from moving LDS accesses across it
        auto lds_barrier = []() {
            asm volatile("" ::: "memory");
            __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0); vmcnt and expcnt at their maxima
            __builtin_amdgcn_s_barrier();
            asm volatile("" ::: "memory");
        };
        // slots j0..j1-1 of ring R: write to LDS buffer ns, then reload with stage kt_load
        auto move = [&](auto &R, char *ns, int kt_load, int j0, int j1) {
#pragma unroll
            for (int j = j0; j < j1; ++j) {
                lwrite(ns, j, R[j]);
                R[j] = gload(kt_load, j);
            }
        };
        // a k step's order: a product, then a fragment read (first nr
        // products), and after every second product one slot write + reload
        // (first nw)
        auto steps = [](int nr, int nw) {
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                if (i < nr)
                    __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
                if (i % 2 == 1 && i / 2 < nw) {
                    __builtin_amdgcn_sched_group_barrier(0x200, 1, 0);
                    __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
                }
            }
        };
        const Scales qn{};  // unused by bf16 products
        // stage kt from buffer `buf`: its four k steps; stage kt + 1 moves from
        // ring R into the other buffer and R refills with stage kt + 3
        auto stage = [&](auto buf, auto &R, int kt) {
            constexpr int b = decltype(buf)::value;
            const char *s = b ? smem1 : smem0;
            char *ns = b ? smem0 : smem1;
            read_frags(s, 1, f1);
            move(R, ns, kt + 3, 0, kRingMoves0);
            mfmas(f0, qn, 0);
            steps(kFragReads, kRingMoves0);
            read_frags(s, 2, f0);
            move(R, ns, kt + 3, kRingMoves0, kRingMoves1);
            mfmas(f1, qn, 1);
            steps(kFragReads, kRingMoves1 - kRingMoves0);
            read_frags(s, 3, f1);
            move(R, ns, kt + 3, kRingMoves1, kLoads);
            mfmas(f0, qn, 2);
            steps(kFragReads, kLoads - kRingMoves1);
            __builtin_amdgcn_sched_barrier(0);
            lds_barrier();
            // the last k step's products run while the next stage's first
            // fragments are read
            read_frags(ns, 0, f0);
            mfmas(f1, qn, 3);
            steps(kFragReads, 0);
            __builtin_amdgcn_sched_barrier(0);
        };
#pragma unroll
        for (int j = 0; j < kLoads; ++j)
            ring0[j] = gload(0, j);
#pragma unroll
        for (int j = 0; j < kLoads; ++j)
            ring1[j] = gload(1, j);
        move(ring0, smem0, 2, 0, kLoads);
        lds_barrier();
        read_frags(smem0, 0, f0);
        for (int kt = 0; kt < nk; kt += 2) {
            stage(Buf0{}, ring1, kt);
            stage(Buf1{}, ring0, kt + 1);
        }
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

// Row-major MX scales (R rows of nk dwords: a row's 4 scale bytes per
// 128-wide stage) to stage-major (nk rows of R dwords).  A workgroup moves a
// 64 x 64 tile through LDS: reads of 64 consecutive dwords of one row, writes
// of 64 consecutive rows of one stage.
constexpr int kTrTile = 64;

__global__ __launch_bounds__(256) void situ_mx_scales_stage_major_kernel(const uint32_t *__restrict__ in,
                                                                         uint32_t *__restrict__ out, int64_t R,
                                                                         int nk, int64_t stride)
{
    __shared__ uint32_t tile[kTrTile][kTrTile + 1];
    const int64_t r0 = (int64_t)blockIdx.x * kTrTile;
    const int s0 = blockIdx.y * kTrTile;
    const int t = threadIdx.x;
#pragma unroll
    for (int k = 0; k < kTrTile * kTrTile / 256; ++k) {
        const int idx = t + 256 * k, i = idx / kTrTile, j = idx % kTrTile;
        if (r0 + i < R && s0 + j < nk)
            tile[i][j] = in[(r0 + i) * nk + s0 + j];
    }
    __syncthreads();
#pragma unroll
    for (int k = 0; k < kTrTile * kTrTile / 256; ++k) {
        const int idx = t + 256 * k, j = idx / kTrTile, i = idx % kTrTile;
        if (r0 + i < R && s0 + j < nk)
            out[(int64_t)(s0 + j) * stride + r0 + i] = tile[i][j];
    }
}

int launch_stage_major(const void *in, void *out, int64_t R, int nk, hipStream_t st)
{
    if (R <= 0 || nk <= 0)
        return 0;
    const dim3 grid((unsigned)((R + kTrTile - 1) / kTrTile), (unsigned)((nk + kTrTile - 1) / kTrTile));
    hipLaunchKernelGGL(situ_mx_scales_stage_major_kernel, grid, dim3(256), 0, st,
                       static_cast<const uint32_t *>(in), static_cast<uint32_t *>(out), R, nk, stage_stride(R));
    return (int)hipGetLastError();
}

using GemmFn = void (*)(const void *, const void *, const uint8_t *, const uint8_t *, const int32_t *, int64_t, int,
                        int, int, int, const void *, int, int64_t, void *, void *, GateK, UpK);

template <int OP, bool LB, bool FAST>
GemmFn pick_gu(bool gu)
{
    return gu ? situ_glu_grouped_fwd_kernel<OP, LB, FAST, true> : situ_glu_grouped_fwd_kernel<OP, LB, FAST, false>;
}

template <int OP>
GemmFn pick(bool lb, bool fast, bool gu)
{
    return lb ? (fast ? pick_gu<OP, true, true>(gu) : pick_gu<OP, true, false>(gu))
              : (fast ? pick_gu<OP, false, true>(gu) : pick_gu<OP, false, false>(gu));
}

}  // namespace

int64_t grouped_slots(int64_t rows, int64_t experts) { return rows / kBM + experts; }

int64_t grouped_mx_stage_stride(int64_t rows) { return stage_stride(rows); }

int64_t grouped_mx_scale_bytes(int64_t rows, int64_t hidden)
{
    return (stage_stride(rows) * (hidden / 128) * 4 + 255) / 256 * 256;
}

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
    const bool gu = L.gate_up != nullptr;
    hipStream_t st = static_cast<hipStream_t>(stream);
    const void *xs = L.x_scales, *ws = L.w_scales;
    if (L.op != OP_BF16) {
        // scales to stage-major in the workspace: x first, then the weights
        char *wsp = static_cast<char *>(L.workspace);
        const int nk = L.hidden / 128;
        const int64_t wrows = (int64_t)L.experts * 2 * L.inter;
        int err = launch_stage_major(L.x_scales, wsp, L.rows, nk, st);
        if (!err)
            err = launch_stage_major(L.w_scales, wsp + grouped_mx_scale_bytes(L.rows, L.hidden), wrows, nk, st);
        if (err)
            return err;
        xs = wsp;
        ws = wsp + grouped_mx_scale_bytes(L.rows, L.hidden);
    }
    const GemmFn fn = L.op == OP_E4M3 ? pick<OP_E4M3>(L.lb, L.fast, gu)
                      : L.op == OP_E5M2 ? pick<OP_E5M2>(L.lb, L.fast, gu)
                                        : pick<OP_BF16>(L.lb, L.fast, gu);
    hipLaunchKernelGGL(fn, dim3((unsigned)blocks), dim3(kThreads), 0, st, L.x, L.w,
                       static_cast<const uint8_t *>(xs), static_cast<const uint8_t *>(ws), L.offsets,
                       L.rows, L.hidden, L.experts, L.inter, slots, L.rw, L.rw_bf16, L.rw_stride, L.out, L.gate_up,
                       L.gk, L.uk);
    return (int)hipGetLastError();
}

}  // namespace situ
