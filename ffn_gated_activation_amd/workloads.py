"""Seeded synthetic inputs for the weighted SiTU-GLU workloads.

This module only draws random numbers; it holds none of the method's
arithmetic, and both the oracle-side tests and the GPU path take their inputs
from it.  The pages measure on no dataset: every workload is synthetic, with
the shapes and value distributions below.

Recipes (all draws from one torch.Generator seeded with `seed` on the chosen
device, in the order gate_up -> [stress mask, magnitude, sign] -> routing
weights -> grad_out; generated in fp32, then rounded to the io dtype with
torch's round-to-nearest-even; "N(0, s)" means s * randn):

  fp32_small    fp32 gate_up [256, 2*512] ~ N(0, 2); routing weights [256, 1]
                ~ U(0, 1); grad_out ~ N(0, 1); beta 4, linear_beta 25;
                forward + backward with d_routing_weights.
  top1_fwd      bf16 gate_up [8192, 2*2048] ~ N(0, 1.5); routing weights
                [8192, 1] = 0.2 + 0.8 U(0, 1) (stand-in for top-1 softmax
                probabilities); beta 4, linear_beta 25; forward only.
  dense_ffn     bf16 gate_up [16384, 2*18432] ~ N(0, 1); one routing weight
                1.0 broadcast over all rows; linear_beta None; grad_out bf16
                ~ N(0, 1); forward + backward, no d_routing_weights.
  routed_top8   bf16 gate_up [65536, 2*2048] ~ N(0, 1), rows = 8192 tokens x
                top-8 (row 8t+k); routing weights = softmax over the 8 draws
                of N(0, 1) per token, [65536, 1] fp32; grad_out bf16 ~ N(0, 1);
                beta 4, linear_beta 25; forward + backward with
                d_routing_weights.
  stress_sat    bf16 gate_up [131072, 2*2048]: N(0, 8), with 5% of entries
                (mask U(0,1) < 0.05) replaced by sign * (30 + 30 U(0,1)),
                sign -1 where U(0,1) < 0.5 else +1 (saturation of tanh and
                sigmoid); routing weights [131072, 1] ~ U(0, 1); grad_out bf16
                ~ N(0, 1); beta 4, linear_beta 25; forward + backward with
                d_routing_weights; rows in natural order.
  routed_top8_mxfp8
                the routed_top8 inputs (same draws), forward only, with the
                output written as MXFP8 (E4M3 elements, 32-value blocks,
                floor scale rule) instead of bf16.
  routed_top8_mxfp8_train
                the routed_top8 inputs (same draws, grad_out included),
                forward + backward + d_routing_weights, with Y and d_gate_up
                written as MXFP8 (E4M3, row-wise 32-value blocks of Y, dG and
                dU, floor scale rule).

Attention-residual mixing (make_attn_res_inputs; draws in the order stored
sums -> prefix -> norm weight -> projection weight, fp32, then rounded):

  attn_res_mix  8192 tokens, 8 stored block sums + the running prefix sum
                (9 blocks, the most a Kimi-K3 layer mixes: its 93 layers in
                blocks of 12), hidden 7168, bf16 values / weights / output;
                stored sum b ~ N(0, 2^(b/2)) (sums of more layers are larger),
                prefix ~ N(0, 2); RMSNorm weight 1 + N(0, 0.1); projection
                weight N(0, 2/sqrt(7168)) (logits of order 2); eps 1e-6.

Fused FC1 grouped GEMM + SiTU-GLU (make_grouped_inputs; draws in the order
group sizes -> x -> weight -> routing weights):

  grouped_fc1_top8
                8192 tokens x top-8 = 65536 routed rows over 16 local experts,
                hidden 7168, expert intermediate 2048 (FC1 weight [16, 4096,
                7168]); rows per expert = a multinomial draw of 65536 over the
                probabilities softmax(N(0, 0.5)) of the 16 experts (load
                imbalance of a real router), rows grouped by expert; x ~ N(0, 1)
                bf16; weight ~ N(0, 1/sqrt(7168)) bf16 (projections of unit
                scale); routing weights = softmax over 8 N(0, 1) draws per token
                (the routed_top8 recipe), fp32; beta 4, linear_beta 25.
  grouped_fc1_top8_mxfp8
                the grouped_fc1_top8 shape on MXFP8 operands
                (make_grouped_mx_inputs; draws in the order group sizes ->
                x codes -> x scales -> weight codes -> weight scales ->
                routing weights): codes = the E4M3 (or E5M2) bytes of
                64 N(0, 1) clamped to the format's largest finite value
                (a block quantiser maps a block's largest value near the top
                of the element range), x scale bytes uniform in 118 .. 122,
                weight scale bytes uniform in 113 .. 117 (per 32 values along
                hidden; the decoded x is then of order 2^-3 .. 2, the decoded
                weight of order 2^-8 .. 2^-4, projections of order 1); routing
                weights and group sizes as above.
"""
from __future__ import annotations

from dataclasses import dataclass

import torch


@dataclass(frozen=True)
class Workload:
    name: str
    rows: int
    inter: int
    dtype: torch.dtype
    beta: float
    linear_beta: float | None
    backward: bool
    want_drw: bool
    broadcast_rw: bool
    description: str
    recipe: str | None = None      # draw the inputs of this workload instead (same seed, same order)
    mx: str | None = None          # forward output as MXFP8 with this element format


WORKLOADS = {
    "fp32_small": Workload("fp32_small", 256, 512, torch.float32, 4.0, 25.0, True, True, False,
                           "fp32 gate_up [256, 2*512] ~ N(0,2), r ~ U(0,1), fwd+bwd+dr"),
    "top1_fwd": Workload("top1_fwd", 8192, 2048, torch.bfloat16, 4.0, 25.0, False, False, False,
                         "bf16 gate_up [8192, 2*2048] ~ N(0,1.5), r = 0.2+0.8 U(0,1), fwd only"),
    "dense_ffn": Workload("dense_ffn", 16384, 18432, torch.bfloat16, 4.0, None, True, False, True,
                          "bf16 dense FFN gate_up [16384, 2*18432] ~ N(0,1), r = 1.0 broadcast, "
                          "linear_beta None, fwd+bwd"),
    "routed_top8": Workload("routed_top8", 65536, 2048, torch.bfloat16, 4.0, 25.0, True, True, False,
                            "bf16 routed-expert rows 8192 tokens x top-8, gate_up [65536, 2*2048] "
                            "~ N(0,1), r = per-token softmax of 8 N(0,1) draws, fwd+bwd+dr"),
    "stress_sat": Workload("stress_sat", 131072, 2048, torch.bfloat16, 4.0, 25.0, True, True, False,
                           "bf16 gate_up [131072, 2*2048] N(0,8) with 5% at +-U(30,60), "
                           "r ~ U(0,1), fwd+bwd+dr"),
    "routed_top8_mxfp8": Workload("routed_top8_mxfp8", 65536, 2048, torch.bfloat16, 4.0, 25.0, False, False,
                                  False, "routed_top8 inputs, forward only, output MXFP8 (E4M3, blocks of 32, "
                                  "E8M0 floor scales)", recipe="routed_top8", mx="e4m3"),
    "routed_top8_mxfp8_train": Workload("routed_top8_mxfp8_train", 65536, 2048, torch.bfloat16, 4.0, 25.0, True,
                                        True, False, "routed_top8 inputs, forward + backward + dr with the "
                                        "forward's Y and the backward's d_gate_up written as MXFP8 (E4M3, "
                                        "row-wise blocks of 32, E8M0 floor scales)", recipe="routed_top8",
                                        mx="e4m3"),
}
ORDER = ["fp32_small", "top1_fwd", "dense_ffn", "routed_top8", "stress_sat", "routed_top8_mxfp8",
         "routed_top8_mxfp8_train"]


def make_inputs(name: str, device="cpu", seed: int = 0, rows: int | None = None,
                inter: int | None = None) -> dict:
    """Draw one workload's inputs.  `rows` / `inter` override the shape (a
    smaller or ragged instance of the same recipe; for routed_top8 rows must be
    a multiple of 8)."""
    w = WORKLOADS[name]
    if w.recipe is not None:
        x = make_inputs(w.recipe, device, seed, rows, inter)
        x.update(workload=w, want_drw=w.want_drw)
        if not w.backward:
            x.update(grad_out=None)
        return x
    rows = w.rows if rows is None else int(rows)
    if inter is not None:
        from dataclasses import replace
        w = replace(w, inter=int(inter))
    dev = torch.device(device)
    gen = torch.Generator(device=dev)
    gen.manual_seed(seed)

    def randn(*shape):
        return torch.randn(*shape, generator=gen, device=dev, dtype=torch.float32)

    def rand(*shape):
        return torch.rand(*shape, generator=gen, device=dev, dtype=torch.float32)

    shape = (rows, 2 * w.inter)
    if name == "fp32_small":
        gate_up = 2.0 * randn(*shape)
    elif name == "top1_fwd":
        gate_up = 1.5 * randn(*shape)
    elif name in ("dense_ffn", "routed_top8"):
        gate_up = randn(*shape)
    elif name == "stress_sat":
        gate_up = 8.0 * randn(*shape)
        mask = rand(*shape) < 0.05
        mag = 30.0 + 30.0 * rand(*shape)
        sign = torch.where(rand(*shape) < 0.5, -1.0, 1.0)
        gate_up = torch.where(mask, sign * mag, gate_up)
        del mask, mag, sign
    else:
        raise KeyError(name)
    gate_up = gate_up.to(w.dtype)

    if name == "fp32_small" or name == "stress_sat":
        rw = rand(rows, 1)
    elif name == "top1_fwd":
        rw = 0.2 + 0.8 * rand(rows, 1)
    elif name == "dense_ffn":
        rw = torch.ones(1, device=dev, dtype=torch.float32)
    else:  # routed_top8
        if rows % 8:
            raise ValueError("routed_top8 rows must be a multiple of 8 (tokens x top-8)")
        z = randn(rows // 8, 8)
        rw = torch.softmax(z, dim=1).reshape(rows, 1).contiguous()

    grad_out = randn(rows, w.inter).to(w.dtype) if w.backward else None
    return {"workload": w, "gate_up": gate_up, "routing_weights": rw, "grad_out": grad_out,
            "beta": w.beta, "linear_beta": w.linear_beta, "want_drw": w.want_drw}


def algorithmic_bytes(name: str, rows: int | None = None) -> dict:
    """Bytes the method must move: read every input once, write every output once.

    forward : gate_up + routing weights + out (MXFP8 output: one byte per
              value plus one scale byte per 32-value block)
    backward: gate_up + routing weights + grad_out + d_gate_up (+ d_routing_weights);
              d_gate_up as MXFP8 when the workload's outputs are: one byte per
              value plus one scale byte per 32-value block of dG and of dU
    """
    w = WORKLOADS[name]
    rows = w.rows if rows is None else rows
    s = torch.finfo(w.dtype).bits // 8
    rw_bytes = 4 * (1 if w.broadcast_rw else rows)
    out_bytes = rows * (w.inter + -(-w.inter // 32)) if w.mx else rows * w.inter * s
    fwd = rows * 2 * w.inter * s + rw_bytes + out_bytes
    bwd = 0
    if w.backward:
        dgu_bytes = rows * 2 * (w.inter + -(-w.inter // 32)) if w.mx else rows * 2 * w.inter * s
        bwd = rows * 2 * w.inter * s + rw_bytes + rows * w.inter * s + dgu_bytes
        if w.want_drw:
            bwd += rw_bytes
    return {"fwd": fwd, "bwd": bwd, "total": fwd + bwd}


@dataclass(frozen=True)
class AttnResWorkload:
    name: str
    tokens: int
    stored: int          # stored block sums; the prefix sum is one more block
    hidden: int
    dtype: torch.dtype
    eps: float
    description: str


ATTN_RES = {
    "attn_res_mix": AttnResWorkload("attn_res_mix", 8192, 8, 7168, torch.bfloat16, 1e-6,
                                    "attention-residual mixing, 8192 tokens x (8 stored sums + prefix) x 7168, "
                                    "bf16 values/weights/output"),
}


def make_attn_res_inputs(tokens: int, stored: int, hidden: int, prefix: bool = True, dtype=torch.bfloat16,
                         w_dtype=torch.bfloat16, device="cpu", seed: int = 0, eps: float = 1e-6) -> dict:
    """Seeded inputs for attention-residual mixing (recipe in the module doc)."""
    dev = torch.device(device)
    gen = torch.Generator(device=dev)
    gen.manual_seed(seed)

    def randn(*shape):
        return torch.randn(*shape, generator=gen, device=dev, dtype=torch.float32)

    scale = torch.exp2(torch.arange(stored, device=dev, dtype=torch.float32) / 2).reshape(1, stored, 1)
    blocks = (randn(tokens, stored, hidden) * scale).to(dtype)
    pre = (2.0 * randn(tokens, hidden)).to(dtype) if prefix else None
    norm_w = (1.0 + 0.1 * randn(hidden)).to(w_dtype)
    proj_w = (randn(hidden) * (2.0 / hidden ** 0.5)).to(w_dtype)
    return {"blocks": blocks, "prefix": pre, "norm_weight": norm_w, "proj_weight": proj_w, "eps": eps}


def attn_res_bytes(name: str) -> int:
    """Bytes the mixing must move: every value read once, both weights once,
    the output written once."""
    w = ATTN_RES[name]
    s = torch.finfo(w.dtype).bits // 8
    return w.tokens * (w.stored + 1) * w.hidden * s + 2 * w.hidden * s + w.tokens * w.hidden * s


@dataclass(frozen=True)
class GroupedWorkload:
    name: str
    rows: int
    experts: int
    hidden: int
    inter: int
    beta: float
    linear_beta: float | None
    description: str


GROUPED = {
    "grouped_fc1_top8": GroupedWorkload("grouped_fc1_top8", 65536, 16, 7168, 2048, 4.0, 25.0,
                                        "fused FC1 grouped GEMM + SiTU-GLU, 65536 routed rows (8192 tokens x "
                                        "top-8) over 16 experts, hidden 7168, intermediate 2048, bf16"),
}


def make_grouped_inputs(rows: int, experts: int, hidden: int, inter: int, device="cpu", seed: int = 0,
                        counts=None, rw_mode: str = "top8") -> dict:
    """Seeded inputs for the fused grouped GEMM (recipe in the module doc).

    counts: rows per expert (a list summing to rows) instead of the
    multinomial draw.  rw_mode: "top8" (per-token softmax of 8 draws; rows a
    multiple of 8), "uniform" (U(0, 1) per row) or "one" (a single weight)."""
    dev = torch.device(device)
    gen = torch.Generator(device=dev)
    gen.manual_seed(seed)
    if counts is None:
        p = torch.softmax(0.5 * torch.randn(experts, generator=gen, device=dev), 0)
        idx = torch.multinomial(p, rows, replacement=True, generator=gen) if rows else \
            torch.zeros(0, dtype=torch.int64, device=dev)
        counts = torch.bincount(idx, minlength=experts).cpu().tolist()
    counts = [int(c) for c in counts]
    if len(counts) != experts or sum(counts) != rows:
        raise ValueError("counts must hold one count per expert summing to rows")
    offsets = [0]
    for c in counts:
        offsets.append(offsets[-1] + c)
    x = torch.randn(rows, hidden, generator=gen, device=dev).to(torch.bfloat16)
    w = (torch.randn(experts, 2 * inter, hidden, generator=gen, device=dev) * hidden ** -0.5).to(torch.bfloat16)
    if rw_mode == "top8":
        if rows % 8:
            raise ValueError("top8 routing weights need rows to be a multiple of 8")
        rw = torch.softmax(torch.randn(rows // 8, 8, generator=gen, device=dev), 1).reshape(rows).contiguous()
    elif rw_mode == "uniform":
        rw = torch.rand(rows, generator=gen, device=dev)
    elif rw_mode == "one":
        rw = torch.ones(1, device=dev)
    else:
        raise ValueError(rw_mode)
    return {"x": x, "weight": w, "offsets": offsets, "counts": counts, "routing_weights": rw}


def grouped_flops(name: str) -> int:
    """Floating-point operations of the projections: 2 M K (2 I)."""
    w = GROUPED[name]
    return 2 * w.rows * w.hidden * 2 * w.inter


GROUPED_MX = {
    "grouped_fc1_top8_mxfp8": GroupedWorkload("grouped_fc1_top8_mxfp8", 65536, 16, 7168, 2048, 4.0, 25.0,
                                              "fused FC1 grouped GEMM + SiTU-GLU on MXFP8 (E4M3) x and weight, "
                                              "65536 routed rows over 16 experts, hidden 7168, intermediate "
                                              "2048, bf16 output"),
}

_FP8_TORCH = {"e4m3": (torch.float8_e4m3fn, 448.0), "e5m2": (torch.float8_e5m2, 57344.0)}


def make_grouped_mx_inputs(rows: int, experts: int, hidden: int, inter: int, fp8_format: str = "e4m3",
                           device="cpu", seed: int = 0, counts=None, rw_mode: str = "top8") -> dict:
    """Seeded MXFP8 operands for the fused grouped GEMM (recipe in the module
    doc): uint8 codes and E8M0 scale bytes of x [rows, hidden] and weight
    [experts, 2 inter, hidden], group offsets and routing weights."""
    if hidden % 32:
        raise ValueError("hidden must be a multiple of 32")
    dt, fmax = _FP8_TORCH[fp8_format]
    dev = torch.device(device)
    gen = torch.Generator(device=dev)
    gen.manual_seed(seed)
    if counts is None:
        p = torch.softmax(0.5 * torch.randn(experts, generator=gen, device=dev), 0)
        idx = torch.multinomial(p, rows, replacement=True, generator=gen) if rows else \
            torch.zeros(0, dtype=torch.int64, device=dev)
        counts = torch.bincount(idx, minlength=experts).cpu().tolist()
    counts = [int(c) for c in counts]
    if len(counts) != experts or sum(counts) != rows:
        raise ValueError("counts must hold one count per expert summing to rows")
    offsets = [0]
    for c in counts:
        offsets.append(offsets[-1] + c)

    def codes(*shape):
        v = (64.0 * torch.randn(*shape, generator=gen, device=dev)).clamp(-fmax, fmax)
        return v.to(dt).view(torch.uint8).contiguous()

    sb = hidden // 32
    xc = codes(rows, hidden)
    xs = torch.randint(118, 123, (rows, sb), generator=gen, device=dev, dtype=torch.int32).to(torch.uint8)
    wc = codes(experts, 2 * inter, hidden)
    ws = torch.randint(113, 118, (experts, 2 * inter, sb), generator=gen, device=dev,
                       dtype=torch.int32).to(torch.uint8)
    if rw_mode == "top8":
        if rows % 8:
            raise ValueError("top8 routing weights need rows to be a multiple of 8")
        rw = torch.softmax(torch.randn(rows // 8, 8, generator=gen, device=dev), 1).reshape(rows).contiguous()
    elif rw_mode == "uniform":
        rw = torch.rand(rows, generator=gen, device=dev)
    elif rw_mode == "one":
        rw = torch.ones(1, device=dev)
    else:
        raise ValueError(rw_mode)
    return {"x_codes": xc, "x_scales": xs, "weight_codes": wc, "weight_scales": ws, "fp8_format": fp8_format,
            "offsets": offsets, "counts": counts, "routing_weights": rw}


def grouped_mx_flops(name: str) -> int:
    """Floating-point operations of the projections: 2 M K (2 I)."""
    w = GROUPED_MX[name]
    return 2 * w.rows * w.hidden * 2 * w.inter
