"""Autograd drop-in for the weighted SiTU-GLU.

Mirrors the NeMo AutoModel page "nemo_automodel.components.models.kimi_k3.situ":
``_WeightedSiTUFunction`` saves only the low-precision inputs (``gate_up`` and
``routing_weights``, in their own dtypes) and recomputes everything in the
backward, which returns ``(d_gate_up, d_routing_weights, None, None)``;
``_weighted_situ(gate_up, routing_weights, beta, linear_beta)`` applies it.
Both directions run in the HIP kernels of libsitu_glu.so (no CPU path, no
chunking: the kernels stream every row once).

Routing weights are row aligned (``[..., 1]`` with gate_up's leading
dimensions) or a single weight for every row; other broadcast shapes raise.
"""
from __future__ import annotations

import torch

from .situ_glu import situ_glu_bwd, situ_glu_fwd


class WeightedSiTUFunction(torch.autograd.Function):
    """Y = r * (beta tanh(G/beta) sigmoid(G)) * (linear_beta tanh(U/linear_beta) or U)."""

    @staticmethod
    def forward(ctx, gate_up: torch.Tensor, routing_weights: torch.Tensor, beta: float = 4.0,
                linear_beta: float | None = 25.0) -> torch.Tensor:
        gate_up = gate_up.contiguous()
        routing_weights = routing_weights.contiguous()
        y = situ_glu_fwd(gate_up, routing_weights, beta, linear_beta)
        ctx.save_for_backward(gate_up, routing_weights)
        ctx.beta = float(beta)
        ctx.linear_beta = None if linear_beta is None else float(linear_beta)
        return y

    @staticmethod
    def backward(ctx, grad_out: torch.Tensor):
        gate_up, routing_weights = ctx.saved_tensors
        want_dgu, want_drw = ctx.needs_input_grad[0], ctx.needs_input_grad[1]
        if not (want_dgu or want_drw):
            return None, None, None, None
        dgu, drw = situ_glu_bwd(gate_up, routing_weights, grad_out.contiguous(), ctx.beta, ctx.linear_beta,
                                want_drw=want_drw)
        return (dgu if want_dgu else None), drw, None, None


def weighted_situ(gate_up: torch.Tensor, routing_weights: torch.Tensor, beta: float = 4.0,
                  linear_beta: float | None = 25.0) -> torch.Tensor:
    """Apply the weighted SiTU-GLU to ``[..., 2 * intermediate]`` projections (autograd aware)."""
    return WeightedSiTUFunction.apply(gate_up, routing_weights, beta, linear_beta)
