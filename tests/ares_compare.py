"""Comparison of the GPU attention-residual mixing with the fp64 oracle.

The kernels compute the chain in fp32 (the NeMo page's `_attn_res_core` is an
fp32 chain too).  The bound on |out_gpu - out_ref| per element is derived from
that arithmetic, with the oracle's magnitudes (attn_res_oracle.c):

  S_th   = sum_b P_tb |x_tbh|             the combine's own magnitude
  a_tb   = r_tb sum_h |x_tbh w_h p_h|     the magnitude the logit sums over
  |dl_tb| <= 2^-24 (80 a_tb + 32 |l_tb|)  the logit's fp32 error: at most ~64
           sequential roundings in the lane / DPP / wavefront sums, the w p
           product, the sum of squares feeding the rsqrt, and the rsqrt
  |dP_tb| <= P_tb (|dl_tb| + max_c |dl_tc|) + 4 2^-24 P_tb   (softmax)
  T_th   = 2^-24 (NB + 8) S_th + 2 max_b |dl_tb| S_th       fp32 chain bound

bfloat16 output: within 1 ulp (ordinal distance of the bf16 patterns, as
elsewhere), or within T_th plus one bf16 ulp of the reference (where the
combine cancels and 1 ulp of a small result is finer than the chain's
bound).  float32 output: |gpu - ref| <= T_th + 2^-24 |ref|.
"""
from __future__ import annotations

import numpy as np
import torch

from compare import bf16_ulp_distance

U = 2.0 ** -24


def chain_bound(ref: dict, nb: int) -> np.ndarray:
    dl = U * (80.0 * ref["absdot"] + 32.0 * np.abs(ref["logits"]))
    lam = dl.max(axis=1, keepdims=True)
    return U * (nb + 8) * ref["scale"] + 2.0 * lam * ref["scale"]


def _bf16_ulp(x: np.ndarray) -> np.ndarray:
    ax = np.maximum(np.abs(x), 2.0 ** -126)
    return 2.0 ** (np.floor(np.log2(ax)) - 7)


def assert_ares_close(name: str, gpu: torch.Tensor, ref: dict, nb: int) -> dict:
    want = ref["out"]
    T = chain_bound(ref, nb)
    g = gpu.detach().float().cpu().numpy().astype(np.float64).reshape(want.shape)
    err = np.abs(g - want)
    if gpu.dtype == torch.bfloat16:
        d = bf16_ulp_distance(gpu.reshape(want.shape), want)
        ok = (d <= 1) | (err <= T + _bf16_ulp(want))
    else:
        ok = err <= T + U * np.abs(want)
    if not ok.all():
        i = tuple(np.argwhere(~ok)[0])
        raise AssertionError(f"{name}: {int((~ok).sum())} of {ok.size} outputs outside the bound; first at {i}: "
                             f"gpu={g[i]!r} oracle={want[i]!r} bound={T[i]!r} scale={ref['scale'][i]!r}")
    with np.errstate(divide="ignore", invalid="ignore"):
        rel = np.where(ref["scale"] > 0, err / ref["scale"], 0.0)
    return {"max_err_over_scale": float(rel.max()) if rel.size else 0.0,
            "median_bound_over_scale": float(np.median(T / np.maximum(ref["scale"], 1e-300))) if T.size else 0.0}
