// Internal interface between the host API (situ_glu_api.cpp) and the HIP
// kernels (situ_glu_kernels.hip).  Not installed; not part of the C ABI.
#pragma once

#include <stddef.h>
#include <stdint.h>

namespace situ {

// Gate-branch constants for one beta (b1), computed on the host.
//   e1 = exp(-2|G|/b1) = exp2(-|G| * k1)
//   y1 = 2|G|/b1       = |G| * y1k    (argument of 1 - e1 = 1 - exp(-y1))
// The root window: dT_g/dG vanishes at G* < 0, where its two terms cancel.
// Inside |G - win_ghi| <= win_hw the fp32-io kernels evaluate dT_g/dG as the
// degree-7 polynomial c0 + c1 d + ... + c7 d^7 in d = G - win_ghi (the Taylor expansion
// at the fp32 number nearest G*) instead of the cancelling difference; the
// bf16-io kernels, whose inputs are bf16 values, replace dT_g/dG / 4 at the
// one bf16 value nearest G* (gsub) by its exact value (tsub); at every
// other bf16 value the plain formula loses at most a factor ~250 to the
// cancellation (about 3e-5 relative), far inside a bf16 ulp.
struct GateK {
    float beta1;
    float k1;
    float y1k;
    float win_ghi;
    float win_hw;
    float c0, c1, c2, c3, c4, c5, c6, c7;
    float gsub, tsub;
};

// Up-branch constants (only used when linear_beta is given):
//   v = exp(-2|U|/b2) = exp2(-|U| * ku)
// and for the bf16-io kernels' polynomial tanh(U/b2): x = U * inv_b2 (the
// backward) or U P(U^2) (the forwards), valid for
// |U| <= small_max = b2/4, the odd Taylor coefficients of tanh with the
// powers of 1/b2 folded in: P(w) = p1 + p3 w + p5 w^2 + p7 w^3,
// p1 = 1/b2, p3 = -1/(3 b2^3), p5 = 2/(15 b2^5), p7 = -17/(315 b2^7).
// small_max < 0 (the polynomial never taken) when a coefficient is not a
// normal float.
struct UpK {
    float beta2;
    float ku;
    float inv_b2;
    float small_max;
    float p1, p3, p5, p7;
};

enum { IO_F32 = 0, IO_BF16 = 1 };

// Work split of the 128-bit path.  A chunk is 64 lanes x one 16-byte vector
// of every stream: 1 KiB of each half row.  A wavefront takes `k`
// consecutive chunks (loads of the next issued before the math of the
// current one).  Flat mapping: chunks numbered row-major over the whole
// tensor, wavefront w takes chunks w k .. w k + k - 1, `wpb` wavefronts per
// workgroup.  Row mapping (routing-weight gradient): a row's chunks go to
// `wpr` wavefronts of one workgroup, `rpb` rows per workgroup, and the
// row's partial sums meet in LDS.
struct ChunkGeom {
    uint32_t half;        // bytes of a half row (= bytes of an output row)
    int cpr;              // chunks per row
    uint32_t magic;       // chunk index / cpr = mulhi(index, magic) >> shift (cpr > 1)
    int shift;
    int k;                // chunks per wavefront
    int wpr;              // row mapping: wavefronts per row
    uint32_t wmagic;      // row mapping: slot / wpr = (slot * wmagic) >> 8 for slot < 16
};

// A launch of the 128-bit path: geometry, chunks of the tensor (flat
// mapping), workgroups and threads per workgroup.
struct ChunkSplit {
    ChunkGeom geom;
    uint32_t total;
    unsigned grid;
    int block;
};

struct FwdLaunch {
    const void *gate_up;
    const void *rw;
    int rw_bf16;          // routing-weight dtype is bf16
    int64_t rw_stride;    // 1: one weight per row, 0: one weight for all rows
    void *out;
    int64_t rows;
    int inter;
    int io;               // IO_F32 / IO_BF16
    int vec;              // 1: 128-bit path, 0: element path
    int lb;               // linear_beta given
    int fast;             // beta1 == 4 specialisation
    ChunkSplit split;     // 128-bit path
    GateK gk;
    UpK uk;
};

struct BwdLaunch {
    const void *gate_up;
    const void *rw;
    int rw_bf16;
    int64_t rw_stride;
    const void *grad_out;
    void *d_gate_up;
    void *d_rw;           // NULL: no routing-weight gradient
    float *row_partials;  // workspace, [rows] fp32, used when rw_stride == 0 and d_rw
    int64_t rows;
    int inter;
    int io;
    int vec;
    int lb;
    int fast;
    ChunkSplit split;     // 128-bit path (row mapping when d_rw)
    GateK gk;
    UpK uk;
};

enum { FP8_E4M3 = 0, FP8_E5M2 = 1 };

// Forward with MXFP8 output: codes [rows, inter] bytes, scales
// [rows, ceil(inter / 32)] bytes.
struct FwdMxLaunch {
    const void *gate_up;
    const void *rw;
    int rw_bf16;
    int64_t rw_stride;
    void *codes;
    void *scales;
    int64_t rows;
    int inter;
    int io;
    int vec;              // 1: 128-bit loads, 8-byte (bf16) / 4-byte (fp32) code stores
    int lb;
    int fast;
    int fmt;              // FP8_E4M3 / FP8_E5M2
    int ceil_mode;        // 0: floor(log2 amax) - emax, 1: no element saturates
    int rows_per_block;   // element path
    ChunkSplit split;     // 128-bit path
    GateK gk;
    UpK uk;
};

// Backward with MXFP8 d_gate_up: codes [rows, 2 inter] bytes (dG, then dU),
// scales [rows, 2 ceil(inter / 32)] bytes (dG's blocks, then dU's).
struct BwdMxLaunch {
    const void *gate_up;
    const void *rw;
    int rw_bf16;
    int64_t rw_stride;
    const void *grad_out;
    void *codes;
    void *scales;
    void *d_rw;           // NULL: no routing-weight gradient
    float *row_partials;  // workspace, [rows] fp32, used when rw_stride == 0 and d_rw
    int64_t rows;
    int inter;
    int io;
    int vec;              // 1: 128-bit loads, 8-byte (bf16) / 4-byte (fp32) code stores
    int lb;
    int fast;
    int fmt;
    int ceil_mode;
    int rows_per_block;
    GateK gk;
    UpK uk;
};

// MXFP8 quantisation of x [rows, cols] (io dtype).
struct MxQuantLaunch {
    const void *x;
    void *codes;
    void *scales;
    int64_t rows;
    int cols;
    int io;
    int vec;
    int fmt;
    int ceil_mode;
    int rows_per_block;
};

// Attention-residual mixing: values = blocks [tokens, m, hidden] followed by
// prefix [tokens, hidden] (when not NULL) along the block axis, nb = m (+1).
struct AresLaunch {
    const void *blocks;
    const void *prefix;
    int64_t tokens;
    int m;
    int nb;
    int hidden;
    const void *norm_w;
    const void *proj_w;
    int w_bf16;
    float eps;
    void *out;
    int io;               // values' dtype
    int out_io;           // output dtype
    int vec;              // 16-byte aligned buffers, rows a whole number of 128-bit vectors
};
// Fused FC1 grouped GEMM + SiTU-GLU: x [rows, hidden], w [experts,
// 2 inter, hidden], offsets [experts + 1] int32 in device memory; bf16
// operands (hidden a multiple of 64) or MX fp8 codes with scale bytes
// [rows, hidden / 32] and [experts, 2 inter, hidden / 32] (hidden a multiple
// of 128; the launch first rewrites them stage-major into `workspace`,
// grouped_mx_scale_bytes(rows, hidden) + grouped_mx_scale_bytes(experts *
// 2 inter, hidden) bytes, 256-byte aligned); inter a multiple of 128;
// operands 16-byte aligned.
struct GroupedLaunch {
    int op;               // 0 bf16, 1 MX E4M3, 2 MX E5M2
    const void *x;
    const void *w;
    const void *x_scales;
    const void *w_scales;
    const int32_t *offsets;
    int64_t rows;
    int hidden;
    int experts;
    int inter;
    const void *rw;
    int rw_bf16;
    int64_t rw_stride;
    void *out;
    void *gate_up;        // NULL: projections not written
    int lb;
    int fast;
    GateK gk;
    UpK uk;
    void *workspace;      // fp8: stage-major scales (see above)
};
// Stage-major scales: the stage stride in dwords of an array of `rows` rows
// (rows rounded up to a 128-byte line, plus one line), and the bytes of the
// whole array (a 256-byte multiple).
int64_t grouped_mx_stage_stride(int64_t rows);
int64_t grouped_mx_scale_bytes(int64_t rows, int64_t hidden);
// Row-tile slots of the grouped GEMM grid (floor(rows / 256) + experts) and
// the workgroups of its launch.
int64_t grouped_slots(int64_t rows, int64_t experts);
int64_t grouped_grid_blocks(int64_t rows, int64_t experts, int64_t inter);

// Which kernel serves a shape: 0 element path; 1, 3 one 128-bit vector per
// lane (up to 12 / 16 blocks); 2 two vectors per lane; 4 the streaming kernel.
int attn_res_path(int io, int hidden, int nb, int vec_ok);

// Enqueue the kernels; return the hipError_t of the launches (0 = success).
int launch_fwd(const FwdLaunch &L, void *stream);
int launch_bwd(const BwdLaunch &L, void *stream);
int launch_fwd_mx(const FwdMxLaunch &L, void *stream);
int launch_bwd_mx(const BwdMxLaunch &L, void *stream);
int launch_mx_quant(const MxQuantLaunch &L, void *stream);
// Fixed-order sum of the [rows] fp32 partials into the one routing-weight
// gradient (broadcast weight).
int launch_dr_reduce(const float *row_partials, int64_t rows, void *d_rw, int rw_bf16, void *stream);
int launch_attn_res(const AresLaunch &L, void *stream);
int launch_grouped_fwd(const GroupedLaunch &L, void *stream);
// The library's per-device scratch array (a file-scope __device__ array of
// SITU_NOALLOC_MAX_ROWS floats in situ_glu_kernels.hip): its device address
// on the current device, looked up once per device; NULL with *err set to the
// hipError_t when the lookup fails.
float *device_scratch(int *err);
// Zero `bytes` bytes at device pointer p with a fill kernel.
int launch_zero(void *p, int64_t bytes, void *stream);
const char *device_error_string(int err);

// Host-side construction of GateK for a beta (root window included).
GateK make_gate_consts(double beta1);
UpK make_up_consts(double beta2);

}  // namespace situ
