"""Tolerance of the fused grouped GEMM + SiTU-GLU against the fp64 oracle.

The kernel sums bf16 products in fp32 on the matrix cores and applies the
activation to the fp32 sums.  Taking each v_mfma_f32_32x32x16_bf16 as adding
its 16 exact products to the accumulator with at most 16 fp32 roundings, the
K / 16 instructions of a projection make a chain of at most K / 16 + 16
roundings, so (first order, u = 2^-24)

    |G_kernel - G| <= eG = (K / 16 + 16) u sG,   sG = sum_k |x_k w_k|

(likewise U).  Through the activation, with |T_g''|, |T_u''| <= 1 and
|T_u'| <= 1 (true for every beta >= 1),

    |Y(G^, U^) - Y(G, U)| <= r [(|T_g'| eG + eG^2 / 2)(|T_u| + eU)
                                + |T_g| (|T_u'| eU + eU^2 / 2)]

then the fp32 evaluation of the activation itself (the relative bound of
mx_compare.y_error_bound) and one rounding of Y to bf16 (half an ulp, at most
2^-8 |Y|) are added.  The stored projections get eG plus their own bf16
rounding.  The test reports the largest observed error as a fraction of this
bound, which is far from tight: errors above it mean a wrong result."""
from __future__ import annotations

import numpy as np
import torch

from mx_compare import y_error_bound

U32 = 2.0 ** -24
BF16_HALF_ULP = 2.0 ** -8
TINY = 2.0 ** -133


def projection_bound(s: np.ndarray, hidden: int) -> np.ndarray:
    return (hidden / 16 + 16) * U32 * s


def output_bound(ref: dict, hidden: int, beta: float, linear_beta) -> np.ndarray:
    eG = projection_bound(ref["sG"], hidden)
    eU = projection_bound(ref["sU"], hidden)
    r = np.abs(ref["r"])
    prop = r * ((np.abs(ref["Tg_prime"]) * eG + eG * eG / 2) * (np.abs(ref["Tu"]) + eU)
                + np.abs(ref["Tg"]) * (np.abs(ref["Tu_prime"]) * eU + eU * eU / 2))
    y = np.abs(ref["out"])
    act = y_error_bound(ref["gate_up"], beta, linear_beta, io_bf16=True) * (y + prop)
    pre = prop + act
    return pre + BF16_HALF_ULP * (y + pre) + TINY


def _np(t: torch.Tensor) -> np.ndarray:
    return t.detach().to("cpu", torch.float64).numpy()


def assert_grouped_close(name: str, out: torch.Tensor, ref: dict, hidden: int, beta: float, linear_beta,
                         rows=None) -> float:
    """Element-by-element check of out (rows `rows` of the kernel's output,
    or all of them) against the oracle's result dict; returns the largest
    error / bound ratio."""
    y = _np(out if rows is None else out[rows])
    bound = output_bound(ref, hidden, beta, linear_beta)
    err = np.abs(y - ref["out"])
    bad = ~(err <= bound)
    if bad.any():
        i, j = np.argwhere(bad)[0]
        raise AssertionError(
            f"{name}: {int(bad.sum())} of {bad.size} outputs outside the bound; first at ({i}, {j}): "
            f"kernel {y[i, j]!r}, oracle {ref['out'][i, j]!r}, bound {bound[i, j]:.3g}, "
            f"G {ref['gate_up'][i, j]!r}")
    return float((err / bound).max()) if err.size else 0.0


def assert_gate_up_close(name: str, gu: torch.Tensor, ref: dict, hidden: int, rows=None) -> float:
    g = _np(gu if rows is None else gu[rows])
    inter = g.shape[1] // 2
    e = projection_bound(np.concatenate([ref["sG"], ref["sU"]], axis=1), hidden)
    bound = e + BF16_HALF_ULP * (np.abs(ref["gate_up"]) + e) + TINY
    err = np.abs(g - ref["gate_up"])
    bad = ~(err <= bound)
    if bad.any():
        i, j = np.argwhere(bad)[0]
        raise AssertionError(f"{name}: {int(bad.sum())} projections outside the bound; first at ({i}, {j}) "
                             f"({'gate' if j < inter else 'up'}): kernel {g[i, j]!r}, oracle "
                             f"{ref['gate_up'][i, j]!r}, bound {bound[i, j]:.3g}")
    return float((err / bound).max()) if err.size else 0.0
