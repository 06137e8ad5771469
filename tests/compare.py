"""Comparison of GPU results with the fp64 oracle, with the tolerances of the
weighted SiTU-GLU parity bar:

  * bfloat16 outputs (Y, dG, dU): at most 1 ulp apart, measured as the
    ordinal distance between the GPU's bf16 value and the oracle's fp64 value
    rounded once to bf16 (round to nearest even); +0 and -0 are the same point.
  * float32 outputs: |gpu - ref| <= 1e-5 |ref| for Y, dU and dG.  Where the
    two terms of dT_g/dG cancel by a factor of at least 100 (near the gate's
    minimum, where a relative bound on the difference would measure only that
    cancellation), dG's reference magnitude is the sum of the magnitudes of
    the two terms instead; the count of elements that pass only under that
    relaxed scale is returned, so that the tests can report it.
  * dr: |gpu - ref| <= 1e-4 * sum_j |go T_g T_u| (the row sum's own condition
    scale), plus one ulp of the routing-weight dtype for its final rounding.

Relative bars are floored at fp32's smallest normal number, 2^-126: below it
fp32 has only the absolute resolution 2^-149.  In the same way, an fp32 chain
whose intermediate falls into the subnormal range (T_g ~ -b1 e^G for G below
about -87, sech^2(U/b2) for |U| above about 44 b2) carries an absolute error of
a few 2^-149 in that intermediate, which the other (bounded) factors of the
product then scale: `allow` is that allowance, 64 * 2^-149 times a bound on the
other factors (subnormal_allowance below), for the backward's products.  The
fp32 forward multiplies the two factors of e^G into its already scaled
product one at a time and so rounds Y once in the subnormal range: its
allowance is 2 * 2^-149.  Only such extreme inputs reach either.
"""
from __future__ import annotations

import numpy as np
import torch

import oracle

BF16_ULP_BAR = 1
F32_REL = 1e-5
DR_REL = 1e-4
F32_MIN_NORMAL = 2.0 ** -126
CANCEL_MIN = 100.0   # term-scale / |dG| from which dG's bar takes the term scale

# Session tally of fp32 dG checks: elements checked, and elements inside the
# bar only under the cancellation scale (printed at the end of the run).
RELAXED_TALLY = {"checked": 0, "relaxed": 0}


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


SUBNORMAL_QUANTA = 64 * 2.0 ** -149
Y_SUBNORMAL_QUANTA = 2 * 2.0 ** -149


def subnormal_allowance(gate_up64: np.ndarray, r64: np.ndarray, go64: np.ndarray | None, beta: float,
                        linear_beta) -> dict:
    """Absolute allowance for an fp32 intermediate rounded in the subnormal
    range, scaled by bounds of the factors it multiplies (see module doc)."""
    inter = gate_up64.shape[1] // 2
    U = np.abs(gate_up64[:, inter:])
    tub = U if linear_beta is None else np.minimum(U, linear_beta)
    r = np.abs(np.broadcast_to(r64.reshape(-1, 1), (gate_up64.shape[0], 1)))
    out = {"y": np.full(np.broadcast_shapes(U.shape, r.shape), Y_SUBNORMAL_QUANTA)}
    if go64 is not None:
        go = np.abs(go64)
        out["dG"] = SUBNORMAL_QUANTA * go * r * (tub + 1.0 + beta / 4.0)
        out["dU"] = SUBNORMAL_QUANTA * go * r * (beta + 1.0)
        out["dr"] = SUBNORMAL_QUANTA * np.sum(go * (tub + beta), axis=1)
    return out


def assert_f32_close(name: str, gpu: torch.Tensor, ref64: np.ndarray, scale64: np.ndarray | None = None,
                     rel: float = F32_REL, allow64: np.ndarray | None = None):
    """fp32 parity.  Without scale64: the maximum relative error.  With
    scale64 (dG's term scale): {"max_rel": ..., "relaxed": n}, n = elements
    inside the bar only because their terms cancel by >= CANCEL_MIN."""
    g = gpu.detach().cpu().numpy().astype(np.float64).reshape(ref64.shape)
    plain = np.maximum(np.abs(ref64), F32_MIN_NORMAL)
    s = plain
    if scale64 is not None:
        cancels = scale64 >= CANCEL_MIN * np.abs(ref64)
        s = np.where(cancels, np.maximum(plain, scale64), plain)
    err = np.abs(g - ref64)
    extra = 0.0 if allow64 is None else allow64
    ok = err <= rel * s + extra
    if not ok.all():
        i = tuple(np.argwhere(~ok)[0])
        raise AssertionError(
            f"{name}: {int((~ok).sum())} of {ok.size} fp32 elements outside {rel} relative; "
            f"first at {i}: gpu={g[i]!r} oracle={ref64[i]!r} scale={s[i]!r}")
    with np.errstate(divide="ignore", invalid="ignore"):
        max_rel = float(np.nanmax(np.where(s > 0, err / s, 0.0))) if err.size else 0.0
    if scale64 is None:
        return max_rel
    relaxed = int(np.sum(err > rel * plain + extra))
    RELAXED_TALLY["checked"] += int(err.size)
    RELAXED_TALLY["relaxed"] += relaxed
    return {"max_rel": max_rel, "relaxed": relaxed}


def assert_dr_close(name: str, gpu: torch.Tensor, ref64: np.ndarray, abs_scale64: np.ndarray,
                    rel: float = DR_REL, allow64: np.ndarray | None = None):
    g = gpu.detach().float().cpu().numpy().astype(np.float64).reshape(ref64.shape)
    ulp = 2.0 ** -8 if gpu.dtype == torch.bfloat16 else 2.0 ** -24
    tol = rel * np.maximum(abs_scale64, F32_MIN_NORMAL) + ulp * np.abs(ref64)
    if allow64 is not None:
        tol = tol + allow64
    err = np.abs(g - ref64)
    ok = err <= tol
    if not ok.all():
        i = tuple(np.argwhere(~ok)[0])
        raise AssertionError(
            f"{name}: {int((~ok).sum())} of {ok.size} dr values outside tolerance; first at {i}: "
            f"gpu={g[i]!r} oracle={ref64[i]!r} scale={abs_scale64[i]!r}")
    return float(np.max(err / np.maximum(abs_scale64, 1e-300))) if err.size else 0.0


def assert_close(name: str, gpu: torch.Tensor, ref64: np.ndarray, scale64: np.ndarray | None = None,
                 allow64: np.ndarray | None = None):
    if gpu.dtype == torch.bfloat16:
        return assert_bf16_close(name, gpu, ref64)
    return assert_f32_close(name, gpu, ref64, scale64, allow64=allow64)
