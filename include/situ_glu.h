/*
 * situ_glu.h - weighted SiTU-GLU forward and backward on AMD Instinct MI355X
 * (gfx950), C ABI.
 *
 * The operation (Megatron-LM PR "[Dev] Add SiTU-GLU through Transformer
 * Engine", section "Activation"; NeMo AutoModel page
 * "nemo_automodel.components.models.kimi_k3.situ", `_situ_fwd_core`):
 *
 *     T_g(G) = beta * tanh(G / beta) * sigmoid(G)                gate branch
 *     T_u(U) = linear_beta * tanh(U / linear_beta)               up branch
 *              (T_u(U) = U when linear_beta is NULL, i.e. None)
 *     Y      = r * T_g(G) * T_u(U)
 *
 * with sigmoid the logistic function, G the first half and U the second half
 * of each row of gate_up (`_WeightedSiTUFunction.forward`: "gate in the first
 * half of the last axis, up in the second"), and r the routing weight of the
 * row.  The Kimi K3 defaults are beta = 4 and linear_beta = 25.
 *
 * Layout (all buffers contiguous, row major, device memory):
 *   gate_up          [rows, 2*intermediate]   io dtype; G = cols [0, I), U = cols [I, 2I)
 *   out, grad_out    [rows, intermediate]     io dtype
 *   d_gate_up        [rows, 2*intermediate]   io dtype; dG first, dU second
 *   routing_weights  [rw_rows]                rw dtype; rw_rows == rows (one
 *                    weight per row, the page's row-aligned [tokens, 1]) or
 *                    rw_rows == 1 (one weight broadcast over every row)
 *   d_routing_weights[rw_rows]                rw dtype
 * Leading dimensions of [..., 2I] tensors are flattened into `rows` by the
 * caller.  Every pointer must be aligned to its element size (2 bytes for
 * bf16, 4 for fp32; SITU_ERR_INVALID_ARG otherwise); beyond that any
 * alignment is accepted, and 16-byte-aligned buffers with intermediate a
 * multiple of 8 (bf16) or 4 (fp32) take the 128-bit path.
 *
 * Precision: inputs are widened to fp32, every intermediate is fp32 (the
 * NeMo page's fp32 chain over low-precision saved inputs), and results are
 * rounded once to the output dtype (round to nearest even).
 *
 * Ownership and streams: the caller allocates and owns every buffer.  The
 * library never allocates, frees or keeps a pointer, and keeps no state
 * between the forward and the backward: the caller keeps gate_up and
 * routing_weights alive for the backward, as the autograd context does on the
 * NeMo page.  Calls enqueue work on `stream` (a hipStream_t; NULL = the null
 * stream) and return without synchronising.  Launch failures are returned;
 * faults during execution surface at the caller's next synchronisation.
 *
 * Errors: every argument is validated before anything is launched; on any
 * error nothing is written and nothing is launched, and a description is
 * available from situ_glu_last_error() (thread local).  rows == 0 or
 * intermediate == 0 is a valid empty call: SITU_OK, no launch.
 *
 * Determinism: results are bitwise reproducible for identical inputs and
 * launch parameters, and each output row depends only on its own input row
 * (and, for d_routing_weights with one broadcast weight, on a fixed-order sum
 * over rows).
 */
#ifndef SITU_GLU_H
#define SITU_GLU_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define SITU_GLU_ABI_VERSION 8

/* return codes */
#define SITU_OK 0
#define SITU_ERR_INVALID_ARG 1  /* a rejected argument (see each entry point) */
#define SITU_ERR_UNSUPPORTED 2  /* valid but not supported (e.g. too large) */
#define SITU_ERR_DEVICE 3       /* the HIP runtime reported an error */

/* element types */
#define SITU_DTYPE_F32 0
#define SITU_DTYPE_BF16 1

/* MXFP8 element formats (OCP 8-bit floating point: E4M3 with bias 7, no
 * infinities, largest 448; E5M2 with bias 15, largest 57344) and scale modes
 * (OCP Microscaling Formats (MX) v1.0, see situ_glu_fwd_mxfp8) */
#define SITU_FP8_E4M3 0
#define SITU_FP8_E5M2 1
#define SITU_MX_SCALE_FLOOR 0   /* s = floor(log2(amax)) - emax_elem (the MX rule) */
#define SITU_MX_SCALE_CEIL 1    /* smallest s with amax <= max_finite * 2^s */
#define SITU_MX_BLOCK 32        /* values per scale, along each row */

/*
 * Forward: out = r * T_g(G) * T_u(U).
 * NeMo page, `_WeightedSiTUFunction.forward(ctx, gate_up, routing_weights,
 * beta, linear_beta)` and `_situ_fwd_core`.
 *
 *   gate_up          device pointer, [rows, 2*intermediate] of io_dtype
 *   io_dtype         SITU_DTYPE_F32 or SITU_DTYPE_BF16; also the dtype of out
 *   rows, intermediate  >= 0; rows * 2 * intermediate must fit in int64
 *   routing_weights  device pointer, [rw_rows] of rw_dtype
 *   rw_dtype         SITU_DTYPE_F32 or SITU_DTYPE_BF16
 *   rw_rows          rows, or 1 (one weight for every row)
 *   beta             gate beta; finite and > 0
 *   linear_beta      host pointer to the up-branch beta (finite, > 0), or
 *                    NULL for None (up branch = U)
 *   out              device pointer, [rows, intermediate] of io_dtype; must
 *                    not overlap gate_up or routing_weights
 *   stream           hipStream_t or NULL
 * Returns SITU_OK, SITU_ERR_INVALID_ARG (bad dtype, beta, linear_beta,
 * rw_rows, NULL pointer, negative size, overlapping output), or
 * SITU_ERR_DEVICE (launch failed).
 */
int situ_glu_fwd(const void *gate_up, int io_dtype, int64_t rows,
                 int64_t intermediate, const void *routing_weights,
                 int rw_dtype, int64_t rw_rows, double beta,
                 const double *linear_beta, void *out, void *stream);

/*
 * Backward: recomputes the fp32 intermediates from the saved inputs and
 * writes the analytic gradients of L = sum(grad_out * Y):
 *     dG = grad_out * r * T_u(U) * dT_g/dG,   dU = grad_out * r * T_g(G) * dT_u/dU
 *     dr_i = sum_j grad_out_ij * T_g(G_ij) * T_u(U_ij)        (rw_rows == rows)
 *     dr_0 = sum_i sum_j grad_out_ij * T_g(G_ij) * T_u(U_ij)  (rw_rows == 1)
 * with dT_g/dG = sigmoid(G) sech^2(G/beta) + beta tanh(G/beta) sigmoid(G)
 * sigmoid(-G) and dT_u/dU = sech^2(U/linear_beta) (1 when linear_beta is
 * NULL).  NeMo page, `_WeightedSiTUFunction.backward(ctx, grad_out) ->
 * (d_gate_up, d_routing_weights, None, None)` and `_situ_bwd_core(g, u0, w,
 * go, beta, linear_beta, want_drw)`.
 *
 *   gate_up, io_dtype, rows, intermediate, routing_weights, rw_dtype,
 *   rw_rows, beta, linear_beta   as for situ_glu_fwd (the forward's inputs)
 *   grad_out         device pointer, [rows, intermediate] of io_dtype
 *   d_gate_up        device pointer, [rows, 2*intermediate] of io_dtype
 *   d_routing_weights device pointer, [rw_rows] of rw_dtype, or NULL when the
 *                    routing-weight gradient is not wanted (want_drw false)
 *   workspace        device scratch of at least
 *                    situ_glu_bwd_workspace_bytes(rows, intermediate, rw_rows)
 *                    bytes (NULL allowed when that is 0); caller owned,
 *                    contents on entry are ignored, clobbered on exit
 *   workspace_bytes  size of workspace
 *   stream           hipStream_t or NULL
 * Outputs must not overlap any input or each other.  Returns as
 * situ_glu_fwd; a too-small workspace is SITU_ERR_INVALID_ARG.
 */
int situ_glu_bwd(const void *gate_up, int io_dtype, int64_t rows,
                 int64_t intermediate, const void *routing_weights,
                 int rw_dtype, int64_t rw_rows, double beta,
                 const double *linear_beta, const void *grad_out,
                 void *d_gate_up, void *d_routing_weights, void *workspace,
                 size_t workspace_bytes, void *stream);

/*
 * Bytes of workspace situ_glu_bwd needs: 0 unless one weight is broadcast
 * over several rows (rw_rows == 1 < rows), where the fixed-order reduction of
 * the routing-weight gradient keeps one fp32 partial per row.  Returns 0 for
 * invalid sizes.
 */
size_t situ_glu_bwd_workspace_bytes(int64_t rows, int64_t intermediate,
                                    int64_t rw_rows);

/* Rows of the library's own scratch array (situ_glu_bwd_noalloc). */
#define SITU_NOALLOC_MAX_ROWS 262144

/*
 * situ_glu_bwd without a workspace argument and without any allocation, for
 * callers that cannot allocate device memory (code under stream capture into
 * a HIP graph, tight serving loops, harnesses that forbid hipMalloc).
 * Arguments, layout, results and errors as situ_glu_bwd; where situ_glu_bwd
 * would need a workspace (one routing weight broadcast over rows > 1 rows,
 * with d_routing_weights), the per-row partials go to a scratch array the
 * library holds on every device it runs on (SITU_NOALLOC_MAX_ROWS floats,
 * 1 MiB, kept until the process ends), and more rows than that are
 * SITU_ERR_UNSUPPORTED (nothing is launched).  The call allocates nothing
 * (no hipMalloc, no hipFree, no allocating library routine); the first call
 * on a device looks the scratch array's address up once.
 * Every call on one GPU shares that GPU's scratch array: two calls that may
 * run at the same time on one GPU (different streams, no ordering between
 * them) race on it, and their routing-weight gradients are then undefined.
 * Every partial it reads was written by the same call, so nothing needs
 * clearing between calls.
 */
int situ_glu_bwd_noalloc(const void *gate_up, int io_dtype, int64_t rows,
                         int64_t intermediate, const void *routing_weights,
                         int rw_dtype, int64_t rw_rows, double beta,
                         const double *linear_beta, const void *grad_out,
                         void *d_gate_up, void *d_routing_weights,
                         void *stream);

/*
 * Forward with MXFP8 output: Y = r * T_g(G) * T_u(U) as in situ_glu_fwd,
 * written as MXFP8 blocks instead of io_dtype values.  The Megatron-LM PR
 * "[Dev] Add SiTU-GLU through Transformer Engine" (section "Test results") runs
 * the activation under MXFP8 block scaling; the format is the OCP
 * Microscaling Formats (MX) v1.0 one:
 *   - each row of Y is cut into blocks of SITU_MX_BLOCK (32) consecutive
 *     values, the last block of a row holding intermediate % 32 values when
 *     that is not 0;
 *   - each block has one E8M0 scale X = 2^s, stored as the byte s + 127;
 *     SITU_MX_SCALE_FLOOR: s = floor(log2(amax)) - emax_elem (emax_elem = 8
 *     for E4M3, 15 for E5M2), where amax is the block's largest |Y|;
 *     SITU_MX_SCALE_CEIL: the smallest s with amax <= max_finite * 2^s (no
 *     element saturates); s is clamped to [-127, 127], so an all-zero block
 *     gets the byte 0;
 *   - each value is stored as the element code nearest Y / X (ties to the
 *     even code), magnitudes past the largest finite value clamped to it;
 *   - a block holding a NaN or an infinity gets the scale byte 255 (NaN); its
 *     element bytes are unspecified.
 * Y is computed in fp32 as for situ_glu_fwd; the rounding to the element
 * format is the only rounding after it.
 *
 *   gate_up ... linear_beta  as for situ_glu_fwd
 *   fp8_format       SITU_FP8_E4M3 or SITU_FP8_E5M2
 *   scale_mode       SITU_MX_SCALE_FLOOR or SITU_MX_SCALE_CEIL
 *   codes            device pointer, [rows, intermediate] bytes (row major)
 *   scales           device pointer, [rows, ceil(intermediate / 32)] bytes
 *   stream           hipStream_t or NULL
 * codes and scales must not overlap the inputs or each other.  Input
 * pointers aligned to their element size; beyond that any alignment is
 * accepted, and a 16-byte-aligned gate_up with intermediate a
 * multiple of 8 (bf16) or 4 (fp32) and codes aligned to 8 (bf16) or 4 (fp32)
 * bytes take the 128-bit path.  Returns as situ_glu_fwd; an unknown format or
 * mode is SITU_ERR_INVALID_ARG.
 */
int situ_glu_fwd_mxfp8(const void *gate_up, int io_dtype, int64_t rows,
                       int64_t intermediate, const void *routing_weights,
                       int rw_dtype, int64_t rw_rows, double beta,
                       const double *linear_beta, int fp8_format,
                       int scale_mode, void *codes, void *scales,
                       void *stream);

/*
 * Backward with MXFP8 output: dG, dU and dr as situ_glu_bwd computes them
 * (fp32, from the saved inputs), with d_gate_up written as MXFP8 blocks
 * instead of io_dtype values — the form the next projection's gradient GEMM
 * takes under the MXFP8 recipe in which the Megatron-LM PR "[Dev] Add
 * SiTU-GLU through Transformer Engine" (section "Test results") runs the MoE
 * forward and backward.  Blocks, scales and element rounding as for
 * situ_glu_fwd_mxfp8, with dG and dU of a row quantised as two separate rows
 * of `intermediate` values (a block never mixes them); blocks run along the
 * intermediate axis (row-wise).
 *
 *   gate_up ... grad_out   as for situ_glu_bwd
 *   fp8_format, scale_mode as for situ_glu_fwd_mxfp8
 *   d_codes      device pointer, [rows, 2*intermediate] bytes: dG's codes,
 *                then dU's, per row
 *   d_scales     device pointer, [rows, 2*ceil(intermediate / 32)] bytes:
 *                dG's block scales, then dU's, per row
 *   d_routing_weights, workspace, workspace_bytes, stream   as for
 *                situ_glu_bwd (situ_glu_bwd_workspace_bytes gives the size)
 * Outputs must not overlap the inputs or each other.  Input pointers aligned
 * to their element size; beyond that any alignment is accepted, and
 * 16-byte-aligned gate_up and grad_out with intermediate a
 * multiple of 8 (bf16) or 4 (fp32) and d_codes aligned to 8 (bf16) or 4
 * (fp32) bytes take the 128-bit path.  Returns as situ_glu_bwd; an unknown
 * format or mode is SITU_ERR_INVALID_ARG.
 */
int situ_glu_bwd_mxfp8(const void *gate_up, int io_dtype, int64_t rows,
                       int64_t intermediate, const void *routing_weights,
                       int rw_dtype, int64_t rw_rows, double beta,
                       const double *linear_beta, const void *grad_out,
                       int fp8_format, int scale_mode, void *d_codes,
                       void *d_scales, void *d_routing_weights,
                       void *workspace, size_t workspace_bytes,
                       void *stream);

/*
 * The MXFP8 block quantiser of situ_glu_fwd_mxfp8 on its own: x [rows, cols]
 * (io_dtype, row major, device memory) becomes codes [rows, cols] bytes and
 * scales [rows, ceil(cols / 32)] bytes, with the blocks, scale modes and
 * rounding described above, by the same device code.  For callers that hold
 * Y (or any other activation) in fp32 or bf16.
 *   x                device pointer, [rows, cols] of io_dtype
 *   io_dtype         SITU_DTYPE_F32 or SITU_DTYPE_BF16
 *   rows, cols       >= 0 (cols <= 2^30 - 1, rows <= 2^31 - 1)
 *   fp8_format, scale_mode, codes, scales, stream   as for situ_glu_fwd_mxfp8
 * Returns SITU_OK, SITU_ERR_INVALID_ARG (bad dtype, format, mode, NULL
 * pointer, negative size, overlapping buffers), SITU_ERR_UNSUPPORTED (too
 * large) or SITU_ERR_DEVICE (launch failed).  rows == 0 or cols == 0 is a
 * valid empty call.
 */
int situ_glu_mx_quantize(const void *x, int io_dtype, int64_t rows,
                         int64_t cols, int fp8_format, int scale_mode,
                         void *codes, void *scales, void *stream);

/*
 * Attention-residual mixing (NeMo AutoModel page
 * "nemo_automodel.components.models.kimi_k3.situ", `_attn_res_core` and
 * `_apply_attn_res`; the Kimi-K3 "dense-kda-layers / store" page,
 * `_forward_attn_residual`, for the call sites).  For every token t the
 * values are the nblocks stored block sums followed by the current prefix sum
 * (when prefix is not NULL), NB = nblocks (+ 1) rows of `hidden` values:
 *     r_b   = 1 / sqrt(mean_h x_bh^2 + eps)                 RMSNorm
 *     l_b   = sum_h (x_bh r_b norm_weight_h) proj_weight_h   projection
 *     P     = softmax over b of l                             (over the blocks)
 *     out_h = sum_b P_b x_bh                                  raw values
 * computed in fp32 and rounded once to out_dtype.
 *
 *   blocks       device pointer, [tokens, nblocks, hidden] of io_dtype (the
 *                stored sums, or the whole stacked values when prefix is NULL)
 *   tokens, nblocks, hidden   >= 0; 1 <= NB <= 16 when tokens and hidden are
 *                not 0; hidden <= 2^30 - 1; tokens <= 2^31 - 1
 *   prefix       device pointer, [tokens, hidden] of io_dtype (the running
 *                sum, the last block), or NULL
 *   io_dtype     SITU_DTYPE_F32 or SITU_DTYPE_BF16 (blocks and prefix)
 *   norm_weight, proj_weight  device pointers, [hidden] of w_dtype
 *   w_dtype      SITU_DTYPE_F32 or SITU_DTYPE_BF16
 *   eps          RMSNorm epsilon, finite and >= 0
 *   out          device pointer, [tokens, hidden] of out_dtype; must not
 *                overlap any input
 *   out_dtype    SITU_DTYPE_F32 or SITU_DTYPE_BF16
 *   stream       hipStream_t or NULL
 * 16-byte-aligned buffers with hidden a multiple of 8 (bf16) or 4 (fp32),
 * hidden * element size < 2^31 and (hidden / values per 16 bytes, NB) within
 * (1024, 16) or (2048, 8) read every value once; other shapes take a
 * two-pass element path.  Results are bitwise reproducible and each token's
 * output depends only on that token's values.  Returns SITU_OK,
 * SITU_ERR_INVALID_ARG (bad dtype, eps, block count, NULL pointer, negative
 * size, overlap), SITU_ERR_UNSUPPORTED (too large) or SITU_ERR_DEVICE.
 */
int situ_glu_attn_res_fwd(const void *blocks, int64_t tokens, int64_t nblocks,
                          int64_t hidden, const void *prefix, int io_dtype,
                          const void *norm_weight, const void *proj_weight,
                          int w_dtype, double eps, void *out, int out_dtype,
                          void *stream);

/* Limits of situ_glu_grouped_fwd. */
#define SITU_GROUPED_MAX_EXPERTS 4096
#define SITU_GROUPED_MAX_HIDDEN (1 << 20)
#define SITU_GROUPED_MAX_INTERMEDIATE (1 << 20)

/*
 * Fused FC1 of routed experts + weighted SiTU-GLU (Megatron-LM PR "[Dev] Add
 * SiTU-GLU through Transformer Engine", section "Design": the routed experts'
 * FC1 is a grouped GEMM, fused with the scaled SiTU-GLU when the backend
 * supports it; the activation as in section "Activation").  The rows of x
 * are grouped by expert: expert e owns rows group_offsets[e] ..
 * group_offsets[e+1] - 1, and for such a row m and j < intermediate
 *     G = sum_k x[m,k] weight[e,j,k]
 *     U = sum_k x[m,k] weight[e,intermediate+j,k]
 *     out[m,j] = r_m * T_g(G) * T_u(U)
 * with bf16 products summed in fp32 on the matrix cores, the activation
 * applied to the fp32 sums (they are not rounded to bf16 first), and out
 * rounded once to bf16.
 *
 *   x              device pointer, [rows, hidden] bf16, row major
 *   io_dtype       SITU_DTYPE_BF16 (the only one supported)
 *   rows           >= 0, <= 2^31 - 1
 *   hidden         the contraction length: a multiple of 64, 64 ..
 *                  SITU_GROUPED_MAX_HIDDEN
 *   weight         device pointer, [experts, 2*intermediate, hidden] bf16:
 *                  expert e's FC1 weight, its intermediate gate rows first,
 *                  then its intermediate up rows (a Linear weight, [out, in])
 *   experts        1 .. SITU_GROUPED_MAX_EXPERTS
 *   intermediate   a multiple of 128, <= SITU_GROUPED_MAX_INTERMEDIATE
 *   group_offsets  device pointer, [experts + 1] int32, non-decreasing from
 *                  0 to rows.  They are read on the device only (no host
 *                  synchronisation).  Offsets outside [0, rows] are clamped
 *                  and a decreasing pair is an empty group: malformed
 *                  offsets never make the kernel access memory outside the
 *                  buffers, but rows no group covers are not written and
 *                  rows that two groups claim get either group's result.
 *   routing_weights, rw_dtype, rw_rows, beta, linear_beta   as in
 *                  situ_glu_fwd (rw_rows == rows or 1)
 *   out            device pointer, [rows, intermediate] bf16
 *   gate_up_out    device pointer, [rows, 2*intermediate] bf16, or NULL: the
 *                  projections [G | U] rounded to bf16, the input the
 *                  backward (situ_glu_bwd) takes
 *   stream         hipStream_t or NULL
 * x, weight, out and gate_up_out must be 16-byte aligned; out and gate_up_out
 * must not overlap each other or any input.  The result of each row depends
 * only on that row and its expert's weight, and is bitwise reproducible.
 * Returns SITU_OK, SITU_ERR_INVALID_ARG (bad dtype, beta, count, alignment,
 * NULL pointer, overlap), SITU_ERR_UNSUPPORTED (a dtype other than bf16, a
 * shape outside the limits, or one whose grid of 256-row x 128-column tiles
 * would exceed 2^31 - 1 workgroups) or SITU_ERR_DEVICE.
 */
int situ_glu_grouped_fwd(const void *x, int io_dtype, int64_t rows,
                         int64_t hidden, const void *weight, int64_t experts,
                         int64_t intermediate, const int32_t *group_offsets,
                         const void *routing_weights, int rw_dtype,
                         int64_t rw_rows, double beta,
                         const double *linear_beta, void *out,
                         void *gate_up_out, void *stream);

/*
 * situ_glu_grouped_fwd on MXFP8 operands: the FC1 GEMM of the routed experts
 * in the MXFP8 block-scaled recipe under which the Megatron-LM PR "[Dev] Add
 * SiTU-GLU through Transformer Engine" validates the activation (sections
 * "Design" and "Test results"), with x and weight held as OCP Microscaling
 * Formats (MX) v1.0 blocks along the contraction axis: 32 consecutive
 * elements of a row share one E8M0 scale byte s, and element k of x row m
 * stands for
 *     x^[m,k] = decode(x_codes[m,k]) * 2^(x_scales[m, k/32] - 127)
 * (likewise w^ from w_codes and w_scales).  Then, as for situ_glu_grouped_fwd,
 *     G = sum_k x^[m,k] w^[e,j,k],  U = sum_k x^[m,k] w^[e,intermediate+j,k]
 *     out[m,j] = r_m * T_g(G) * T_u(U)
 * with the products summed on the scaled matrix cores, the activation applied
 * to the fp32 sums and out rounded once to bf16.  The scaled matrix
 * instruction is not an fp32 dot product: within each group of 8 consecutive
 * k it truncates the (exact) products toward zero to 13 bits below the
 * group's largest exponent sum, so a projection is accurate to about
 * 2^-10 sum_g 2^(Ex_g + Ew_g) (Ex_g, Ew_g the largest operand exponents in
 * group g) plus fp32 accumulation error.
 *
 *   x_codes        device pointer, [rows, hidden] fp8 codes (bytes)
 *   x_scales       device pointer, [rows, hidden / 32] E8M0 bytes
 *   rows           >= 0, <= 2^31 - 1
 *   hidden         a multiple of 128, 128 .. SITU_GROUPED_MAX_HIDDEN
 *   w_codes        device pointer, [experts, 2*intermediate, hidden] fp8
 *                  codes: expert e's gate rows, then its up rows
 *   w_scales       device pointer, [experts, 2*intermediate, hidden / 32]
 *                  E8M0 bytes
 *   experts, intermediate, group_offsets, routing_weights, rw_dtype,
 *   rw_rows, beta, linear_beta, out, gate_up_out, stream   as for
 *                  situ_glu_grouped_fwd
 *   fp8_format     SITU_FP8_E4M3 or SITU_FP8_E5M2 (x and weight alike)
 *   workspace      device pointer, 16-byte aligned, at least
 *                  situ_glu_grouped_fwd_mxfp8_workspace_bytes(rows, hidden,
 *                  experts, intermediate) bytes, owned by the caller: the
 *                  call first rewrites both scale arrays there stage-major
 *                  (a row's 4 scale bytes of each 128-wide slice of the
 *                  hidden axis, rows contiguous), the layout the matrix-core
 *                  kernel reads; its contents afterwards are unspecified
 *   workspace_bytes  its size
 * (rows + 64) * hidden / 128 and (experts * 2 * intermediate + 64) *
 * hidden / 128 must be below 2^30 (else SITU_ERR_UNSUPPORTED).  x_codes, w_codes, out,
 * gate_up_out and workspace must be 16-byte aligned, the scale arrays 4-byte
 * aligned; out, gate_up_out and workspace must not overlap each other or any
 * input.  Codes that encode NaN or infinity, the scale byte 255 (NaN) and
 * scale pairs whose products leave the fp32 range give unspecified values in
 * the rows and columns they reach.  Results are bitwise reproducible.
 * Returns as situ_glu_grouped_fwd; an unknown fp8_format, or a workspace that
 * is NULL, too small or misaligned, is SITU_ERR_INVALID_ARG.
 */
int situ_glu_grouped_fwd_mxfp8(const void *x_codes, const void *x_scales,
                               int64_t rows, int64_t hidden,
                               const void *w_codes, const void *w_scales,
                               int64_t experts, int64_t intermediate,
                               int fp8_format, const int32_t *group_offsets,
                               const void *routing_weights, int rw_dtype,
                               int64_t rw_rows, double beta,
                               const double *linear_beta, void *out,
                               void *gate_up_out, void *workspace,
                               size_t workspace_bytes, void *stream);

/*
 * Bytes of workspace situ_glu_grouped_fwd_mxfp8 needs for these sizes: the
 * two stage-major scale arrays, each of hidden / 128 slices of R' dwords,
 * where R' is its row count (rows, or experts * 2 * intermediate) rounded up
 * to a multiple of 32 plus 32 (the padding keeps successive slices off the
 * same cache sets), each array rounded up to a multiple of 256 bytes.  Host
 * only.
 * Returns 0 for negative sizes or sizes beyond the SITU_GROUPED_MAX_* limits.
 */
size_t situ_glu_grouped_fwd_mxfp8_workspace_bytes(int64_t rows,
                                                  int64_t hidden,
                                                  int64_t experts,
                                                  int64_t intermediate);

/* Message describing the last error on the calling thread ("" if none). */
const char *situ_glu_last_error(void);

/* SITU_GLU_ABI_VERSION of the loaded library. */
int situ_glu_abi_version(void);

/*
 * Diagnostic: the constants the kernels use near the root G* < 0 of dT_g/dG
 * for a given beta (host only, no device work).  There the two terms of
 * dT_g/dG cancel (Megatron-LM PR "Add SiTU-GLU through Transformer Engine",
 * section "Activation": T_g has its minimum at G*), so inside
 * |G - out[0]| <= out[1] the fp32-io kernels evaluate dT_g/dG as
 * out[2] + out[3] d + out[4] d^2 + ... + out[9] d^7 with d = G - out[0]
 * (out[0] = G* rounded to fp32).  The bf16-io kernels, whose inputs are bf16
 * values, take dT_g/dG = out[11] at the one bf16 input G = out[10] nearest
 * G* (the only bf16 value where the cancellation costs more than ~3e-5
 * relative) and the plain formula elsewhere.  out must hold 12 floats.
 * Returns SITU_OK or SITU_ERR_INVALID_ARG (bad beta, NULL out).
 */
int situ_glu_gate_window(double beta, float *out);

/*
 * Diagnostic: the work split of the 128-bit path for a call with these sizes
 * (host only, no device work).  direction: 0 situ_glu_fwd, 1 situ_glu_bwd
 * without d_routing_weights, 2 with it, 3 situ_glu_fwd_mxfp8 (bf16 with
 * chunks per row a multiple of 4: four chunks per wavefront, an aligned
 * group of one row, whose scale bytes leave in one store).  A chunk is 64 lanes x 16 bytes
 * (1 KiB) of each half row; out must hold 10 int64:
 *   out[0] chunks per row, out[1] chunks of the tensor, out[2] chunks per
 *   wavefront, out[3] wavefronts per row (direction 2; else 0: chunks are
 *   numbered over the whole tensor), out[4] workgroups, out[5] threads per
 *   workgroup, out[6], out[7] the multiplier and shift that divide a chunk
 *   index by out[0] (index / out[0] = (index * out[6]) >> (32 + out[7]) for
 *   index < 2^31), out[8] the multiplier that divides a wavefront slot by
 *   out[3] ((slot * out[8]) >> 8 for slot < 16), out[9] bytes of a half row.
 * Returns SITU_OK; SITU_ERR_INVALID_ARG for a bad dtype or direction, NULL
 * out, sizes out of range, or sizes that take the element path (I times the
 * element size not a multiple of 16); SITU_ERR_UNSUPPORTED beyond 2^31
 * chunks.
 */
int situ_glu_split(int io_dtype, int64_t rows, int64_t intermediate,
                   int linear_beta_given, int direction, int64_t *out);

#ifdef __cplusplus
}
#endif

#endif /* SITU_GLU_H */
