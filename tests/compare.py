"""Comparison of GPU results with the fp64 oracle, with the tolerances of the
weighted SiTU-GLU parity bar:

  * bfloat16 outputs (Y, dG, dU): at most 1 ulp apart, measured as the
    ordinal distance between the GPU's bf16 value and the oracle's fp64 value
    rounded once to bf16 (round to nearest even); +0 and -0 are the same point.
  * float32 outputs: |gpu - ref| <= 1e-5 |ref| for Y and dU.  For dG the
    reference magnitude is the sum of the magnitudes of the two terms of
    dT_g/dG (they cancel at the gate's minimum, where a relative bound on the
    difference would measure only that cancellation).
  * dr: |gpu - ref| <= 1e-4 * sum_j |go T_g T_u| (the row sum's own condition
    scale), plus one ulp of the routing-weight dtype for its final rounding.
"""
from __future__ import annotations

import numpy as np
import torch

import oracle

BF16_ULP_BAR = 1
F32_REL = 1e-5
DR_REL = 1e-4


def bf16_bits(t: torch.Tensor) -> np.ndarray:
    assert t.dtype == torch.bfloat16
    return t.detach().cpu().contiguous().view(torch.int16).numpy().view(np.uint16)


def _ordinal16(bits: np.ndarray) -> np.ndarray:
    b = bits.astype(np.int32)
    mag = b & 0x7FFF
    return np.where(b & 0x8000, -mag, mag)


def bf16_ulp_distance(gpu: torch.Tensor, ref64: np.ndarray) -> np.ndarray:
    gb = bf16_bits(gpu).reshape(ref64.shape)
    rb = oracle.round_bf16_bits(ref64)
    nan_g = (gb & 0x7F80) == 0x7F80
    nan_g &= (gb & 0x007F) != 0
    d = np.abs(_ordinal16(gb) - _ordinal16(rb))
    d = np.where(nan_g | np.isnan(ref64), np.iinfo(np.int32).max, d)
    return d


def assert_bf16_close(name: str, gpu: torch.Tensor, ref64: np.ndarray, bar: int = BF16_ULP_BAR):
    d = bf16_ulp_distance(gpu, ref64)
    bad = np.argwhere(d > bar)
    if bad.size:
        i = tuple(bad[0])
        g = gpu.detach().float().cpu().numpy().reshape(ref64.shape)[i]
        raise AssertionError(
            f"{name}: {bad.shape[0]} of {d.size} elements more than {bar} bf16 ulp from the oracle; "
            f"first at {i}: gpu={g!r} oracle={ref64[i]!r} distance={d[i]}")
    return int(d.max()) if d.size else 0


def assert_f32_close(name: str, gpu: torch.Tensor, ref64: np.ndarray, scale64: np.ndarray | None = None,
                     rel: float = F32_REL):
    g = gpu.detach().cpu().numpy().astype(np.float64).reshape(ref64.shape)
    s = np.abs(ref64) if scale64 is None else np.maximum(np.abs(ref64), scale64)
    # the smallest fp32 subnormal: values below it cannot be represented at all
    err = np.abs(g - ref64)
    ok = err <= rel * s + 2.0 ** -149
    if not ok.all():
        i = tuple(np.argwhere(~ok)[0])
        raise AssertionError(
            f"{name}: {int((~ok).sum())} of {ok.size} fp32 elements outside {rel} relative; "
            f"first at {i}: gpu={g[i]!r} oracle={ref64[i]!r} scale={s[i]!r}")
    with np.errstate(divide="ignore", invalid="ignore"):
        return float(np.nanmax(np.where(s > 0, err / s, 0.0))) if err.size else 0.0


def assert_dr_close(name: str, gpu: torch.Tensor, ref64: np.ndarray, abs_scale64: np.ndarray,
                    rel: float = DR_REL):
    g = gpu.detach().float().cpu().numpy().astype(np.float64).reshape(ref64.shape)
    ulp = 2.0 ** -8 if gpu.dtype == torch.bfloat16 else 2.0 ** -24
    tol = rel * abs_scale64 + ulp * np.abs(ref64) + 2.0 ** -149
    err = np.abs(g - ref64)
    ok = err <= tol
    if not ok.all():
        i = tuple(np.argwhere(~ok)[0])
        raise AssertionError(
            f"{name}: {int((~ok).sum())} of {ok.size} dr values outside tolerance; first at {i}: "
            f"gpu={g[i]!r} oracle={ref64[i]!r} scale={abs_scale64[i]!r}")
    return float(np.max(err / np.maximum(abs_scale64, 1e-300))) if err.size else 0.0


def assert_close(name: str, gpu: torch.Tensor, ref64: np.ndarray, scale64: np.ndarray | None = None):
    if gpu.dtype == torch.bfloat16:
        return assert_bf16_close(name, gpu, ref64)
    return assert_f32_close(name, gpu, ref64, scale64)
