"""Python entry points of the weighted SiTU-GLU library (same names as the C ABI).

These functions marshal torch tensors into the C ABI of libsitu_glu.so; every
step of the computation runs in its HIP kernels.  There is no CPU fallback:
without the built library or a GPU they raise.

Semantics follow the NeMo AutoModel page "nemo_automodel.components.models.
kimi_k3.situ": ``_WeightedSiTUFunction.forward(ctx, gate_up, routing_weights,
beta, linear_beta)`` and ``backward(ctx, grad_out) -> (d_gate_up,
d_routing_weights, None, None)``; ``_situ_rw_is_row_aligned`` for the routing
weight layout (one weight per gate_up row, ``[..., 1]``, or a single weight
broadcast over all rows).
"""
from __future__ import annotations

import functools

import torch

from . import _capi

_DT = {torch.float32: _capi.SITU_DTYPE_F32, torch.bfloat16: _capi.SITU_DTYPE_BF16}


def _io_dtype(t: torch.Tensor, what: str) -> int:
    try:
        return _DT[t.dtype]
    except KeyError:
        raise TypeError(f"{what} must be float32 or bfloat16, got {t.dtype}") from None


def _check_device(*ts):
    dev = None
    for t in ts:
        if t is None:
            continue
        if not t.is_cuda:
            raise ValueError("situ_glu runs on the GPU only: every tensor must be on a cuda device")
        if dev is None:
            dev = t.device
        elif t.device != dev:
            raise ValueError(f"every tensor of one call must be on the same device ({dev} and {t.device})")


def _on_tensor_device(fn):
    """Run an entry point with its tensors' GPU as the current device, so that
    the launch goes to that device and to its current stream."""
    @functools.wraps(fn)
    def wrapper(*args, **kwargs):
        for a in list(args) + list(kwargs.values()):
            if isinstance(a, torch.Tensor) and a.is_cuda:
                with torch.cuda.device(a.device):
                    return fn(*args, **kwargs)
        return fn(*args, **kwargs)
    return wrapper


def _refuse_grad(name: str, *ts, hint: str = ""):
    """The forward-only entry points have no backward: refuse inputs that
    would need one (grad mode on and a tensor requiring grad) instead of
    returning an output detached from the graph."""
    if torch.is_grad_enabled() and any(t is not None and t.requires_grad for t in ts):
        raise RuntimeError(f"{name} has no backward: call it on tensors that do not require grad, or under "
                           f"torch.no_grad(){hint}")


def _flatten(gate_up: torch.Tensor, routing_weights: torch.Tensor):
    if gate_up.dim() < 1 or gate_up.shape[-1] % 2:
        raise ValueError(f"gate_up must be [..., 2*intermediate], got {tuple(gate_up.shape)}")
    if not gate_up.is_contiguous():
        raise ValueError("gate_up must be contiguous")
    inter = gate_up.shape[-1] // 2
    lead = tuple(gate_up.shape[:-1])
    rows = 1
    for d in lead:
        rows *= d
    rw = routing_weights
    if not rw.is_contiguous():
        raise ValueError("routing_weights must be contiguous")
    if rw.numel() == 1:
        rw_rows = 1
    elif tuple(rw.shape) == lead + (1,) or (tuple(rw.shape) == lead and len(lead) > 0):
        rw_rows = rows
    else:
        raise ValueError(
            f"routing_weights of shape {tuple(rw.shape)} is neither row aligned with gate_up "
            f"{tuple(gate_up.shape)} (expected {lead + (1,)}) nor a single broadcast weight")
    return lead, rows, inter, rw_rows


def _stream():
    return torch.cuda.current_stream().cuda_stream


@_on_tensor_device
def situ_glu_fwd(gate_up: torch.Tensor, routing_weights: torch.Tensor, beta: float = 4.0,
                 linear_beta: float | None = 25.0, out: torch.Tensor | None = None) -> torch.Tensor:
    """Y = r * (beta tanh(G/beta) sigmoid(G)) * (linear_beta tanh(U/linear_beta) or U).

    gate_up [..., 2I] (float32 or bfloat16; G first, U second),
    routing_weights [..., 1] row aligned, or one weight.  Returns [..., I] in
    gate_up's dtype.
    """
    _refuse_grad("situ_glu_fwd", gate_up, routing_weights,
                 hint="; ffn_gated_activation_amd.weighted_situ is the differentiable form")
    lib = _capi.load()
    _check_device(gate_up, routing_weights, out)
    io = _io_dtype(gate_up, "gate_up")
    rwd = _io_dtype(routing_weights, "routing_weights")
    lead, rows, inter, rw_rows = _flatten(gate_up, routing_weights)
    if out is None:
        out = torch.empty(lead + (inter,), dtype=gate_up.dtype, device=gate_up.device)
    elif out.dtype != gate_up.dtype or tuple(out.shape) != lead + (inter,) or not out.is_contiguous():
        raise ValueError("out must be a contiguous tensor of gate_up's dtype and shape [..., I]")
    _capi.check(lib.situ_glu_fwd(gate_up.data_ptr(), io, rows, inter, routing_weights.data_ptr(),
                                 rwd, rw_rows, float(beta), _capi.lb_ptr(linear_beta),
                                 out.data_ptr(), _stream()), lib)
    return out


def situ_glu_bwd_workspace_bytes(rows: int, intermediate: int, rw_rows: int) -> int:
    return int(_capi.load().situ_glu_bwd_workspace_bytes(rows, intermediate, rw_rows))


@_on_tensor_device
def situ_glu_bwd(gate_up: torch.Tensor, routing_weights: torch.Tensor, grad_out: torch.Tensor,
                 beta: float = 4.0, linear_beta: float | None = 25.0, want_drw: bool = True,
                 d_gate_up: torch.Tensor | None = None, d_routing_weights: torch.Tensor | None = None,
                 workspace: torch.Tensor | None = None):
    """Analytic backward: returns (d_gate_up [..., 2I], d_routing_weights or None).

    d_routing_weights has routing_weights' shape and dtype; with one broadcast
    weight it is the sum over all rows.
    """
    lib = _capi.load()
    _check_device(gate_up, routing_weights, grad_out, d_gate_up, d_routing_weights, workspace)
    io = _io_dtype(gate_up, "gate_up")
    rwd = _io_dtype(routing_weights, "routing_weights")
    lead, rows, inter, rw_rows = _flatten(gate_up, routing_weights)
    if grad_out.dtype != gate_up.dtype or tuple(grad_out.shape) != lead + (inter,):
        raise ValueError(f"grad_out must be {lead + (inter,)} of dtype {gate_up.dtype}")
    if not grad_out.is_contiguous():
        raise ValueError("grad_out must be contiguous")
    if d_gate_up is None:
        d_gate_up = torch.empty_like(gate_up)
    elif d_gate_up.dtype != gate_up.dtype or d_gate_up.shape != gate_up.shape or not d_gate_up.is_contiguous():
        raise ValueError("d_gate_up must be a contiguous tensor like gate_up")
    if want_drw and d_routing_weights is None:
        d_routing_weights = torch.empty_like(routing_weights)
    if not want_drw:
        d_routing_weights = None
    need = int(lib.situ_glu_bwd_workspace_bytes(rows, inter, rw_rows)) if want_drw else 0
    if need and (workspace is None or workspace.numel() * workspace.element_size() < need):
        workspace = torch.empty(need, dtype=torch.uint8, device=gate_up.device)
    ws_ptr = workspace.data_ptr() if (need and workspace is not None) else None
    ws_bytes = workspace.numel() * workspace.element_size() if ws_ptr else 0
    _capi.check(lib.situ_glu_bwd(
        gate_up.data_ptr(), io, rows, inter, routing_weights.data_ptr(), rwd, rw_rows, float(beta),
        _capi.lb_ptr(linear_beta), grad_out.data_ptr(), d_gate_up.data_ptr(),
        d_routing_weights.data_ptr() if d_routing_weights is not None else None,
        ws_ptr, ws_bytes, _stream()), lib)
    return d_gate_up, d_routing_weights


_FP8 = {"e4m3": _capi.SITU_FP8_E4M3, "e5m2": _capi.SITU_FP8_E5M2}
_MODES = {"floor": _capi.SITU_MX_SCALE_FLOOR, "ceil": _capi.SITU_MX_SCALE_CEIL}


def _mx_args(fp8_format: str, scale_mode: str):
    try:
        return _FP8[fp8_format], _MODES[scale_mode]
    except KeyError:
        raise ValueError(f"fp8_format must be one of {sorted(_FP8)} and scale_mode one of {sorted(_MODES)}, "
                         f"got {fp8_format!r}, {scale_mode!r}") from None


def _mx_outputs(lead, cols, device, codes, scales):
    nblk = -(-cols // _capi.SITU_MX_BLOCK)
    if codes is None:
        codes = torch.empty(lead + (cols,), dtype=torch.uint8, device=device)
    elif codes.dtype != torch.uint8 or tuple(codes.shape) != lead + (cols,) or not codes.is_contiguous():
        raise ValueError(f"codes must be a contiguous uint8 tensor of shape {lead + (cols,)}")
    if scales is None:
        scales = torch.empty(lead + (nblk,), dtype=torch.uint8, device=device)
    elif scales.dtype != torch.uint8 or tuple(scales.shape) != lead + (nblk,) or not scales.is_contiguous():
        raise ValueError(f"scales must be a contiguous uint8 tensor of shape {lead + (nblk,)}")
    return codes, scales


@_on_tensor_device
def situ_glu_fwd_mxfp8(gate_up: torch.Tensor, routing_weights: torch.Tensor, beta: float = 4.0,
                       linear_beta: float | None = 25.0, fp8_format: str = "e4m3", scale_mode: str = "floor",
                       codes: torch.Tensor | None = None, scales: torch.Tensor | None = None):
    """Forward with MXFP8 output: returns (codes uint8 [..., I], scales uint8
    [..., ceil(I / 32)]), blocks of 32 along the last axis with E8M0 scales.

    ``codes.view(torch.float8_e4m3fn)`` (or ``float8_e5m2``) gives the
    elements; the value of element j is element * 2^(scales[..., j // 32] - 127).
    """
    _refuse_grad("situ_glu_fwd_mxfp8", gate_up, routing_weights)
    lib = _capi.load()
    _check_device(gate_up, routing_weights, codes, scales)
    io = _io_dtype(gate_up, "gate_up")
    rwd = _io_dtype(routing_weights, "routing_weights")
    fmt, mode = _mx_args(fp8_format, scale_mode)
    lead, rows, inter, rw_rows = _flatten(gate_up, routing_weights)
    codes, scales = _mx_outputs(lead, inter, gate_up.device, codes, scales)
    _capi.check(lib.situ_glu_fwd_mxfp8(gate_up.data_ptr(), io, rows, inter, routing_weights.data_ptr(), rwd,
                                       rw_rows, float(beta), _capi.lb_ptr(linear_beta), fmt, mode,
                                       codes.data_ptr(), scales.data_ptr(), _stream()), lib)
    return codes, scales


@_on_tensor_device
def situ_glu_bwd_mxfp8(gate_up: torch.Tensor, routing_weights: torch.Tensor, grad_out: torch.Tensor,
                       beta: float = 4.0, linear_beta: float | None = 25.0, want_drw: bool = True,
                       fp8_format: str = "e4m3", scale_mode: str = "floor", d_codes: torch.Tensor | None = None,
                       d_scales: torch.Tensor | None = None, d_routing_weights: torch.Tensor | None = None,
                       workspace: torch.Tensor | None = None):
    """Backward with MXFP8 d_gate_up: returns (d_codes uint8 [..., 2I],
    d_scales uint8 [..., 2 ceil(I / 32)], d_routing_weights or None).

    Per row, d_codes holds dG's codes then dU's, d_scales dG's block scales
    then dU's (blocks of 32 along I, never mixing dG and dU); the value of
    dG element j is code * 2^(d_scales[..., j // 32] - 127) and of dU element
    j is code * 2^(d_scales[..., nblk + j // 32] - 127), nblk = ceil(I / 32).
    """
    lib = _capi.load()
    _check_device(gate_up, routing_weights, grad_out, d_codes, d_scales, d_routing_weights, workspace)
    io = _io_dtype(gate_up, "gate_up")
    rwd = _io_dtype(routing_weights, "routing_weights")
    fmt, mode = _mx_args(fp8_format, scale_mode)
    lead, rows, inter, rw_rows = _flatten(gate_up, routing_weights)
    if grad_out.dtype != gate_up.dtype or tuple(grad_out.shape) != lead + (inter,):
        raise ValueError(f"grad_out must be {lead + (inter,)} of dtype {gate_up.dtype}")
    if not grad_out.is_contiguous():
        raise ValueError("grad_out must be contiguous")
    nblk = -(-inter // _capi.SITU_MX_BLOCK)
    if d_codes is None:
        d_codes = torch.empty(lead + (2 * inter,), dtype=torch.uint8, device=gate_up.device)
    elif d_codes.dtype != torch.uint8 or tuple(d_codes.shape) != lead + (2 * inter,) or not d_codes.is_contiguous():
        raise ValueError(f"d_codes must be a contiguous uint8 tensor of shape {lead + (2 * inter,)}")
    if d_scales is None:
        d_scales = torch.empty(lead + (2 * nblk,), dtype=torch.uint8, device=gate_up.device)
    elif d_scales.dtype != torch.uint8 or tuple(d_scales.shape) != lead + (2 * nblk,) or not d_scales.is_contiguous():
        raise ValueError(f"d_scales must be a contiguous uint8 tensor of shape {lead + (2 * nblk,)}")
    if want_drw and d_routing_weights is None:
        d_routing_weights = torch.empty_like(routing_weights)
    if not want_drw:
        d_routing_weights = None
    need = int(lib.situ_glu_bwd_workspace_bytes(rows, inter, rw_rows)) if want_drw else 0
    if need and (workspace is None or workspace.numel() * workspace.element_size() < need):
        workspace = torch.empty(need, dtype=torch.uint8, device=gate_up.device)
    ws_ptr = workspace.data_ptr() if (need and workspace is not None) else None
    ws_bytes = workspace.numel() * workspace.element_size() if ws_ptr else 0
    _capi.check(lib.situ_glu_bwd_mxfp8(
        gate_up.data_ptr(), io, rows, inter, routing_weights.data_ptr(), rwd, rw_rows, float(beta),
        _capi.lb_ptr(linear_beta), grad_out.data_ptr(), fmt, mode, d_codes.data_ptr(), d_scales.data_ptr(),
        d_routing_weights.data_ptr() if d_routing_weights is not None else None, ws_ptr, ws_bytes, _stream()), lib)
    return d_codes, d_scales, d_routing_weights


@_on_tensor_device
def situ_glu_mx_quantize(x: torch.Tensor, fp8_format: str = "e4m3", scale_mode: str = "floor",
                         codes: torch.Tensor | None = None, scales: torch.Tensor | None = None):
    """MXFP8 block quantisation of x [..., cols] (float32 or bfloat16) along its
    last axis: returns (codes uint8 [..., cols], scales uint8 [..., ceil(cols / 32)])."""
    _refuse_grad("situ_glu_mx_quantize", x)
    lib = _capi.load()
    _check_device(x, codes, scales)
    io = _io_dtype(x, "x")
    fmt, mode = _mx_args(fp8_format, scale_mode)
    if x.dim() < 1 or not x.is_contiguous():
        raise ValueError("x must be a contiguous tensor with at least one dimension")
    lead = tuple(x.shape[:-1])
    cols = x.shape[-1]
    rows = x.numel() // cols if cols else 0
    if cols == 0:
        rows = 1
        for d in lead:
            rows *= d
    codes, scales = _mx_outputs(lead, cols, x.device, codes, scales)
    _capi.check(lib.situ_glu_mx_quantize(x.data_ptr(), io, rows, cols, fmt, mode, codes.data_ptr(),
                                         scales.data_ptr(), _stream()), lib)
    return codes, scales


@_on_tensor_device
def situ_glu_attn_res_fwd(blocks: torch.Tensor | None, prefix: torch.Tensor | None, norm_weight: torch.Tensor,
                          proj_weight: torch.Tensor, eps: float, out_dtype: torch.dtype | None = None,
                          out: torch.Tensor | None = None) -> torch.Tensor:
    """Attention-residual mixing of the values = blocks [T, m, H] followed by
    prefix [T, H] (either may be None) along the block axis: RMSNorm (weight
    norm_weight, epsilon eps), projection to one logit per block
    (proj_weight), softmax over the blocks, and the weighted sum of the raw
    values.  Returns [T, H] in out_dtype (default: the values' dtype)."""
    _refuse_grad("situ_glu_attn_res_fwd", blocks, prefix, norm_weight, proj_weight)
    lib = _capi.load()
    _check_device(blocks, prefix, norm_weight, proj_weight, out)
    ref = blocks if blocks is not None else prefix
    if ref is None:
        raise ValueError("attention-residual mixing needs blocks or a prefix")
    io = _io_dtype(ref, "values")
    if blocks is not None:
        if blocks.dim() != 3 or not blocks.is_contiguous():
            raise ValueError(f"blocks must be a contiguous [tokens, blocks, hidden] tensor, got {tuple(blocks.shape)}")
        tokens, m, hidden = blocks.shape
    else:
        m = 0
    if prefix is not None:
        if prefix.dtype != ref.dtype or prefix.dim() != 2 or not prefix.is_contiguous():
            raise ValueError("prefix must be a contiguous [tokens, hidden] tensor of the blocks' dtype")
        if blocks is not None and tuple(prefix.shape) != (tokens, hidden):
            raise ValueError(f"prefix must be [{tokens}, {hidden}], got {tuple(prefix.shape)}")
        tokens, hidden = prefix.shape
    wd = _io_dtype(norm_weight, "norm_weight")
    if proj_weight.dtype != norm_weight.dtype:
        raise TypeError("norm_weight and proj_weight must share a dtype")
    for w, name in ((norm_weight, "norm_weight"), (proj_weight, "proj_weight")):
        if w.numel() != hidden or not w.is_contiguous():
            raise ValueError(f"{name} must be a contiguous tensor of {hidden} values")
    out_dtype = ref.dtype if out_dtype is None else out_dtype
    od = _io_dtype(torch.empty(0, dtype=out_dtype), "out_dtype")
    if out is None:
        out = torch.empty(tokens, hidden, dtype=out_dtype, device=ref.device)
    elif out.dtype != out_dtype or tuple(out.shape) != (tokens, hidden) or not out.is_contiguous():
        raise ValueError(f"out must be a contiguous [{tokens}, {hidden}] tensor of {out_dtype}")
    _capi.check(lib.situ_glu_attn_res_fwd(
        blocks.data_ptr() if blocks is not None else None, tokens, m, hidden,
        prefix.data_ptr() if prefix is not None else None, io, norm_weight.data_ptr(), proj_weight.data_ptr(), wd,
        float(eps), out.data_ptr(), od, _stream()), lib)
    return out


def attn_res_core(values: torch.Tensor, norm_weight: torch.Tensor, proj_weight: torch.Tensor,
                  variance_epsilon: float, out_dtype: torch.dtype) -> torch.Tensor:
    """The NeMo page's `_attn_res_core(values, norm_weight, proj_weight,
    variance_epsilon, out_dtype)`: values [T, B+1, H] already stacked."""
    return situ_glu_attn_res_fwd(values, None, norm_weight, proj_weight, variance_epsilon, out_dtype)


def apply_attn_res(prefix_sum: torch.Tensor, block_residual: torch.Tensor, norm_weight: torch.Tensor,
                   proj_weight: torch.Tensor, eps: float, out_dtype: torch.dtype | None = None) -> torch.Tensor:
    """The NeMo page's `_apply_attn_res(prefix_sum, block_residual, ...)`: the
    stored sums [T, m, H] and the running sum [T, H], mixed without
    concatenating them first."""
    return situ_glu_attn_res_fwd(block_residual, prefix_sum.reshape(-1, prefix_sum.shape[-1]), norm_weight,
                                 proj_weight, eps, out_dtype)


def _grouped_outputs(rows, experts, two_i, group_offsets, routing_weights, out, want_gate_up, gate_up_out,
                     device):
    inter = two_i // 2
    if group_offsets.dtype != torch.int32 or group_offsets.numel() != experts + 1 or not group_offsets.is_contiguous():
        raise ValueError(f"group_offsets must be a contiguous int32 tensor of {experts + 1} values")
    rwd = _io_dtype(routing_weights, "routing_weights")
    rw_rows = routing_weights.numel()
    if rw_rows not in (rows, 1) or not routing_weights.is_contiguous():
        raise ValueError(f"routing_weights must hold {rows} row-aligned values or one weight")
    if out is None:
        out = torch.empty(rows, inter, dtype=torch.bfloat16, device=device)
    elif out.dtype != torch.bfloat16 or tuple(out.shape) != (rows, inter) or not out.is_contiguous():
        raise ValueError(f"out must be a contiguous [{rows}, {inter}] bfloat16 tensor")
    if want_gate_up and gate_up_out is None:
        gate_up_out = torch.empty(rows, two_i, dtype=torch.bfloat16, device=device)
    if gate_up_out is not None and (gate_up_out.dtype != torch.bfloat16 or tuple(gate_up_out.shape) != (rows, two_i)
                                    or not gate_up_out.is_contiguous()):
        raise ValueError(f"gate_up_out must be a contiguous [{rows}, {two_i}] bfloat16 tensor")
    return rwd, rw_rows, out, gate_up_out


@_on_tensor_device
def situ_glu_grouped_fwd(x: torch.Tensor, weight: torch.Tensor, group_offsets: torch.Tensor,
                         routing_weights: torch.Tensor, beta: float = 4.0, linear_beta: float | None = 25.0,
                         want_gate_up: bool = False, out: torch.Tensor | None = None,
                         gate_up_out: torch.Tensor | None = None):
    """Fused FC1 of routed experts + weighted SiTU-GLU.

    x [M, K] bf16 with rows grouped by expert, weight [E, 2I, K] bf16 (each
    expert's FC1 weight, gate rows first), group_offsets [E + 1] int32 on the
    device (expert e owns rows group_offsets[e] .. group_offsets[e+1]),
    routing_weights [M] / [M, 1] or one weight.  Returns out [M, I] bf16, or
    (out, gate_up [M, 2I] bf16) when want_gate_up."""
    _refuse_grad("situ_glu_grouped_fwd", x, weight, routing_weights)
    lib = _capi.load()
    _check_device(x, weight, group_offsets, routing_weights, out, gate_up_out)
    if x.dtype != torch.bfloat16 or weight.dtype != torch.bfloat16:
        raise TypeError("the grouped GEMM takes bfloat16 x and weight")
    if x.dim() != 2 or weight.dim() != 3 or not x.is_contiguous() or not weight.is_contiguous():
        raise ValueError("x must be a contiguous [M, K] and weight a contiguous [E, 2I, K] tensor")
    rows, hidden = x.shape
    experts, two_i, k2 = weight.shape
    if k2 != hidden or two_i % 2:
        raise ValueError(f"weight must be [E, 2I, {hidden}], got {tuple(weight.shape)}")
    rwd, rw_rows, out, gate_up_out = _grouped_outputs(rows, experts, two_i, group_offsets, routing_weights, out,
                                                      want_gate_up, gate_up_out, x.device)
    _capi.check(lib.situ_glu_grouped_fwd(
        x.data_ptr(), _capi.SITU_DTYPE_BF16, rows, hidden, weight.data_ptr(), experts, two_i // 2,
        group_offsets.data_ptr(), routing_weights.data_ptr(), rwd, rw_rows, float(beta), _capi.lb_ptr(linear_beta),
        out.data_ptr(), gate_up_out.data_ptr() if gate_up_out is not None else None, _stream()), lib)
    return (out, gate_up_out) if gate_up_out is not None else out


_FP8_CODE_DTYPES = {"e4m3": (torch.uint8, torch.float8_e4m3fn), "e5m2": (torch.uint8, torch.float8_e5m2)}


@_on_tensor_device
def situ_glu_grouped_fwd_mxfp8(x_codes: torch.Tensor, x_scales: torch.Tensor, weight_codes: torch.Tensor,
                               weight_scales: torch.Tensor, group_offsets: torch.Tensor,
                               routing_weights: torch.Tensor, fp8_format: str = "e4m3", beta: float = 4.0,
                               linear_beta: float | None = 25.0, want_gate_up: bool = False,
                               out: torch.Tensor | None = None, gate_up_out: torch.Tensor | None = None,
                               workspace: torch.Tensor | None = None):
    """situ_glu_grouped_fwd on MXFP8 operands.

    x_codes [M, K] and weight_codes [E, 2I, K] hold fp8 codes (uint8, or the
    torch float8 dtype of fp8_format), x_scales [M, K / 32] and weight_scales
    [E, 2I, K / 32] their E8M0 scale bytes (uint8): element k of a row is
    decode(code) * 2^(scale[k / 32] - 127).  workspace: a device buffer of at
    least situ_glu_grouped_fwd_mxfp8_workspace_bytes(...) bytes (allocated
    here when not given).  The rest is as for situ_glu_grouped_fwd."""
    _refuse_grad("situ_glu_grouped_fwd_mxfp8", routing_weights)
    lib = _capi.load()
    fmt = _mx_args(fp8_format, "floor")[0]
    _check_device(x_codes, x_scales, weight_codes, weight_scales, group_offsets, routing_weights, out, gate_up_out)
    ok = _FP8_CODE_DTYPES[fp8_format]
    if x_codes.dtype not in ok or weight_codes.dtype not in ok:
        raise TypeError(f"x_codes and weight_codes must be uint8 or {ok[1]} tensors")
    if x_scales.dtype != torch.uint8 or weight_scales.dtype != torch.uint8:
        raise TypeError("x_scales and weight_scales must be uint8 tensors")
    ts = (x_codes, x_scales, weight_codes, weight_scales)
    if x_codes.dim() != 2 or weight_codes.dim() != 3 or not all(t.is_contiguous() for t in ts):
        raise ValueError("x_codes must be a contiguous [M, K] and weight_codes a contiguous [E, 2I, K] tensor")
    rows, hidden = x_codes.shape
    experts, two_i, k2 = weight_codes.shape
    if k2 != hidden or two_i % 2:
        raise ValueError(f"weight_codes must be [E, 2I, {hidden}], got {tuple(weight_codes.shape)}")
    if hidden % _capi.SITU_MX_BLOCK:
        raise ValueError(f"hidden must be a multiple of {_capi.SITU_MX_BLOCK}, got {hidden}")
    sb = hidden // _capi.SITU_MX_BLOCK
    if tuple(x_scales.shape) != (rows, sb) or tuple(weight_scales.shape) != (experts, two_i, sb):
        raise ValueError(f"x_scales must be [{rows}, {sb}] and weight_scales [{experts}, {two_i}, {sb}]")
    rwd, rw_rows, out, gate_up_out = _grouped_outputs(rows, experts, two_i, group_offsets, routing_weights, out,
                                                      want_gate_up, gate_up_out, x_codes.device)
    need = situ_glu_grouped_fwd_mxfp8_workspace_bytes(rows, hidden, experts, two_i // 2)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=x_codes.device)
    _check_device(workspace)
    if not workspace.is_contiguous():
        raise ValueError("workspace must be contiguous")
    _capi.check(lib.situ_glu_grouped_fwd_mxfp8(
        x_codes.data_ptr(), x_scales.data_ptr(), rows, hidden, weight_codes.data_ptr(), weight_scales.data_ptr(),
        experts, two_i // 2, fmt, group_offsets.data_ptr(), routing_weights.data_ptr(), rwd, rw_rows, float(beta),
        _capi.lb_ptr(linear_beta), out.data_ptr(), gate_up_out.data_ptr() if gate_up_out is not None else None,
        workspace.data_ptr(), workspace.numel() * workspace.element_size(), _stream()), lib)
    return (out, gate_up_out) if gate_up_out is not None else out


def situ_glu_grouped_fwd_mxfp8_workspace_bytes(rows: int, hidden: int, experts: int, intermediate: int) -> int:
    return int(_capi.load().situ_glu_grouped_fwd_mxfp8_workspace_bytes(rows, hidden, experts, intermediate))


def situ_glu_last_error() -> str:
    return _capi.last_error()


def situ_glu_split(io_dtype: torch.dtype, rows: int, intermediate: int, linear_beta_given: bool,
                   direction: int) -> dict:
    """The 128-bit path's work split for a call with these sizes (host only):
    direction 0 forward, 1 backward, 2 backward with d_routing_weights, 3 the
    MXFP8 forward."""
    import ctypes
    lib = _capi.load()
    out = (ctypes.c_int64 * 10)()
    _capi.check(lib.situ_glu_split(_DT[io_dtype], int(rows), int(intermediate), int(bool(linear_beta_given)),
                                   int(direction), out), lib)
    keys = ("chunks_per_row", "chunks", "chunks_per_wave", "waves_per_row", "workgroups", "threads",
            "magic", "shift", "slot_magic", "half_row_bytes")
    return dict(zip(keys, (int(v) for v in out)))


def situ_glu_abi_version() -> int:
    return int(_capi.load().situ_glu_abi_version())


def situ_glu_gate_window(beta: float = 4.0):
    """(G*_f32, half width, c0, ..., c7, bf16 value nearest G*, dT_g/dG
    there): the constants the kernels use near the root of dT_g/dG."""
    import ctypes
    lib = _capi.load()
    out = (ctypes.c_float * 12)()
    _capi.check(lib.situ_glu_gate_window(float(beta), out), lib)
    return tuple(float(v) for v in out)
