"""The tolerance helpers of the MXFP8 grouped GEMM tests, on the CPU: the
exponent each fp8 code is aligned by agrees with its decoded value (oracle
mx_dequantize), and the group exponent sums bound every group's products."""
from __future__ import annotations

import numpy as np
import pytest

import oracle
from grouped_compare import _code_exponents, _group_exp_max, mx_exponent_sums


@pytest.mark.parametrize("fmt", ["e4m3", "e5m2"])
def test_code_exponents_match_decoded_values(fmt):
    codes = np.arange(256, dtype=np.uint8).reshape(8, 32)
    vals = oracle.mx_dequantize(codes, np.full((8, 1), 127, np.uint8), fmt).reshape(-1)
    e = _code_exponents(codes.reshape(-1), fmt)
    emin = -6 if fmt == "e4m3" else -14
    for c, v, ex in zip(range(256), vals, e):
        if not np.isfinite(v):
            continue
        if v == 0:
            assert ex == -np.inf, c
        elif abs(v) >= 2.0 ** emin:        # normal: 2^e <= |v| < 2^(e+1)
            assert 2.0 ** ex <= abs(v) < 2.0 ** (ex + 1), (c, v, ex)
        else:                              # subnormal: aligned at emin
            assert ex == emin and abs(v) < 2.0 ** ex, (c, v, ex)


def test_group_exponent_sums_bound_products():
    rng = np.random.default_rng(3)
    xc = rng.integers(0, 256, (5, 64)).astype(np.uint8)
    wc = rng.integers(0, 256, (1, 6, 64)).astype(np.uint8)
    xc[(xc & 0x7F) == 0x7F] = 0x38      # no NaN codes
    wc[(wc & 0x7F) == 0x7F] = 0x38
    xs = rng.integers(120, 130, (5, 2)).astype(np.uint8)
    ws = rng.integers(120, 130, (1, 6, 2)).astype(np.uint8)
    xv = oracle.mx_dequantize(xc, xs, "e4m3")
    wv = oracle.mx_dequantize(wc[0], ws[0], "e4m3")
    s = mx_exponent_sums(xc, xs, wc, ws, [0, 5], "e4m3")
    g = _group_exp_max(xc, xs, "e4m3")
    assert g.shape == (5, 8)
    # every product of group g is below 4 * 2^(Ex_g + Ew_g) (mantissas below 2)
    p = np.abs(xv[:, None, :] * wv[None, :, :]).reshape(5, 6, 8, 8).max(-1)
    xg, wg = g, _group_exp_max(wc[0], ws[0], "e4m3")
    assert np.all(p < 4 * xg[:, None, :] * wg[None, :, :] + 1e-300)
    assert np.allclose(s, xg @ wg.T)
