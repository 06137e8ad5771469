"""Comparison of MXFP8 outputs from the GPU with the fp64 oracle.

Exact inputs (the stand-alone quantiser): codes and scales must equal the
oracle's bit for bit, except the element bytes of blocks whose scale is NaN
(the format gives them no value).

Fused forward: the kernel quantises its own fp32 Y, which differs from the
exact Y by the fp32 chain's rounding.  A scale or code is a decision taken on
that fp32 value, so the check accepts exactly the results the exact Y could
give under a perturbation within the fp32 chain's error bound:

  |Y_fp32 - Y| <= rel * |Y| + abs, elementwise, with
    rel = 1e-5 (the fp32 bar of the activation itself), plus, for bf16 io, the
          first-order replacement of 1 - exp(-y) below y = 2^-11 (relative
          truncation y / 2) and the cancellation of 1 - exp(-y) above it
          (relative 2^-23 / y), for y = 2|G|/beta and, with linear_beta,
          y = 2|U|/linear_beta;
    abs = the subnormal-intermediate allowance of compare.py.

For each block the scale must lie between the scale of the smallest and of
the largest possible block maximum; given the GPU's scale, each element's code
must decode to a value between the codes of the interval's two ends (encoding
is monotone).  Blocks with a non-finite Y must carry the NaN scale, and so
must blocks where |Y| certainly exceeds fp32's range (the fp32 product is then
infinite); where the bound straddles fp32's largest value, the NaN scale and
the finite window are both accepted.
"""
from __future__ import annotations

import numpy as np
import torch

import oracle

BLOCK = 32
F32_REL = 1e-5
F32_MAX = float(np.finfo(np.float32).max)


def y_error_bound(gate_up64: np.ndarray, beta: float, linear_beta, io_bf16: bool) -> np.ndarray:
    """Relative bound on the fp32 Y of each element."""
    inter = gate_up64.shape[1] // 2
    rel = np.full((gate_up64.shape[0], inter), F32_REL)
    if io_bf16:
        terms = [2.0 * np.abs(gate_up64[:, :inter]) / beta]
        if linear_beta is not None:
            terms.append(2.0 * np.abs(gate_up64[:, inter:]) / linear_beta)
        with np.errstate(divide="ignore"):
            for y in terms:
                rel += np.where(y < 2.0 ** -11, 0.5 * y, 2.0 ** -23 / np.maximum(y, 2.0 ** -11))
    return rel


def _small_arg(y: np.ndarray) -> np.ndarray:
    """Relative error of the bf16-io kernels' 1 - exp(-y): the first-order
    replacement below y = 2^-11, cancellation above it."""
    with np.errstate(divide="ignore"):
        return np.where(y < 2.0 ** -11, 0.5 * y, 2.0 ** -23 / np.maximum(y, 2.0 ** -11))


def grad_error_bounds(gate_up64: np.ndarray, dgu64: np.ndarray, dg_scale64: np.ndarray, beta: float, linear_beta,
                      io_bf16: bool) -> tuple[np.ndarray, np.ndarray]:
    """Absolute bounds on the backward's fp32 dG and dU (before any output
    rounding).  fp32 io: the 1e-5 bar of the fp32 backward (dG relative to the
    sum of the magnitudes of dT_g/dG's two terms, dg_scale).  bf16 io adds the
    kernels' cheaper pieces: dG carries T_u and dU carries T_g, each with the
    small-argument error of its 1 - exp(-y) (y = 2|U|/linear_beta, 2|G|/beta).
    Near the gate's minimum the kernels take the exact dT_g/dG at the one bf16
    input nearest the root, and elsewhere the plain formula's rounding stays
    inside the 1e-5 dg_scale term."""
    inter = gate_up64.shape[1] // 2
    G, U = gate_up64[:, :inter], gate_up64[:, inter:]
    dG, dU = np.abs(dgu64[:, :inter]), np.abs(dgu64[:, inter:])
    eg = F32_REL * dg_scale64
    eu = F32_REL * dU
    if io_bf16:
        if linear_beta is not None:
            eg = eg + _small_arg(2.0 * np.abs(U) / linear_beta) * dG
        eu = eu + _small_arg(2.0 * np.abs(G) / beta) * dU
    return eg, eu


def _pad_blocks(a: np.ndarray, fill) -> np.ndarray:
    rows, cols = a.shape
    nblk = -(-cols // BLOCK)
    out = np.full((rows, nblk * BLOCK), fill, dtype=a.dtype)
    out[:, :cols] = a
    return out.reshape(rows, nblk, BLOCK)


def _host_u8(t: torch.Tensor) -> np.ndarray:
    return t.detach().cpu().contiguous().numpy().astype(np.uint8)


def assert_mx_exact(name: str, codes: torch.Tensor, scales: torch.Tensor, x64: np.ndarray, fmt: str,
                    mode: str):
    x64 = x64.reshape(-1, x64.shape[-1])
    want_c, want_s = oracle.mx_quantize(x64, fmt, mode)
    got_c = _host_u8(codes).reshape(want_c.shape)
    got_s = _host_u8(scales).reshape(want_s.shape)
    bad_s = np.argwhere(got_s != want_s)
    if bad_s.size:
        i, b = bad_s[0]
        blk = x64[i, b * BLOCK:(b + 1) * BLOCK]
        raise AssertionError(f"{name}: {bad_s.shape[0]} of {got_s.size} scales differ; first row {i} block {b}: "
                             f"gpu {got_s[i, b]} oracle {want_s[i, b]}, block max {np.nanmax(np.abs(blk))!r}")
    nan_blk = np.repeat(want_s == 255, BLOCK, axis=1)[:, :x64.shape[1]]
    bad = np.argwhere((got_c != want_c) & ~nan_blk)
    if bad.size:
        kinds = {}
        for i, j in bad[:2000]:
            key = ("zero sign" if (got_c[i, j] | want_c[i, j]) == 0x80 and (got_c[i, j] & 0x7F) == 0
                   else "other")
            kinds[key] = kinds.get(key, 0) + 1
        i, j = bad[0]
        X = 2.0 ** (int(want_s[i, j // BLOCK]) - 127)
        raise AssertionError(f"{name}: {bad.shape[0]} of {got_c.size} codes differ {kinds}; first at ({i}, {j}): "
                             f"x={x64[i, j]!r} x/X={x64[i, j] / X!r} gpu {got_c[i, j]:#04x} "
                             f"oracle {want_c[i, j]:#04x}")


def assert_mx_window(name: str, codes: torch.Tensor, scales: torch.Tensor, y64: np.ndarray, rel: np.ndarray,
                     abs64: np.ndarray | None, fmt: str, mode: str) -> dict:
    """Fused-forward check (see module doc).  Returns counts for the report."""
    rows, cols = y64.shape
    got_c = _host_u8(codes).reshape(rows, cols)
    got_s = _host_u8(scales).reshape(rows, -1)
    d = rel * np.abs(y64) + (0.0 if abs64 is None else abs64)
    lo, hi = y64 - d, y64 + d
    mag_hi = np.maximum(np.abs(lo), np.abs(hi))
    mag_lo = np.where((lo <= 0) & (hi >= 0), 0.0, np.minimum(np.abs(lo), np.abs(hi)))
    with np.errstate(invalid="ignore"):
        nonfinite = ~np.isfinite(y64) | (mag_lo > F32_MAX)
        maybe_inf = np.isfinite(y64) & (mag_hi > F32_MAX) & ~nonfinite
    bad_blk = _pad_blocks(nonfinite, False).any(axis=2)
    maybe_blk = _pad_blocks(maybe_inf, False).any(axis=2) & ~bad_blk
    amax_lo = np.where(bad_blk, 0.0, _pad_blocks(np.where(nonfinite, 0.0, mag_lo), 0.0).max(axis=2))
    amax_hi = np.where(bad_blk, 0.0, _pad_blocks(np.where(nonfinite, 0.0, mag_hi), 0.0).max(axis=2))
    s_lo = oracle.mx_scale_code_array(amax_lo, fmt, mode).astype(np.int32)
    s_hi = oracle.mx_scale_code_array(amax_hi, fmt, mode).astype(np.int32)
    gs = got_s.astype(np.int32)
    ok_s = np.where(bad_blk, gs == 255, ((gs >= s_lo) & (gs <= s_hi)) | (maybe_blk & (gs == 255)))
    bad_blk = bad_blk | (gs == 255)
    if not ok_s.all():
        i, b = np.argwhere(~ok_s)[0]
        raise AssertionError(f"{name}: {int((~ok_s).sum())} of {ok_s.size} scales outside their window; "
                             f"first row {i} block {b}: gpu {gs[i, b]} allowed [{s_lo[i, b]}, {s_hi[i, b]}] "
                             f"(block max {amax_lo[i, b]!r} .. {amax_hi[i, b]!r})")
    finite_blk = np.repeat(~bad_blk, BLOCK, axis=1)[:, :cols]
    X = np.repeat(np.ldexp(1.0, np.where(bad_blk, 0, gs - 127)), BLOCK, axis=1)[:, :cols]
    with np.errstate(invalid="ignore"):
        v_lo = oracle.fp8_decode_array(oracle.fp8_encode_array(np.where(finite_blk, lo / X, 0.0), fmt), fmt)
        v_hi = oracle.fp8_decode_array(oracle.fp8_encode_array(np.where(finite_blk, hi / X, 0.0), fmt), fmt)
        v = oracle.fp8_decode_array(got_c, fmt)
        ok = ~finite_blk | ((v >= v_lo) & (v <= v_hi))
    if not ok.all():
        i, j = np.argwhere(~ok)[0]
        raise AssertionError(f"{name}: {int((~ok).sum())} of {ok.size} codes outside their window; first at "
                             f"({i}, {j}): y={y64[i, j]!r} X={X[i, j]!r} gpu {got_c[i, j]:#04x} = {v[i, j]!r}, "
                             f"allowed [{v_lo[i, j]!r}, {v_hi[i, j]!r}]")
    unique = int(np.sum(finite_blk & (v_lo == v_hi)))
    return {"elements": int(finite_blk.sum()), "unique": unique, "nan_blocks": int(bad_blk.sum()),
            "scale_windows": int(np.sum(s_lo != s_hi))}
