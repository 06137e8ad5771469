"""The MXFP8 comparison of mx_compare.py, on the CPU: results the oracle
itself produces pass it, and planted wrong codes or scales are caught.
(Checks the checker; no GPU and no HIP code involved.)"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
from mx_compare import assert_mx_exact, assert_mx_window, y_error_bound


def _y(seed=0, rows=8, cols=200):
    rng = np.random.default_rng(seed)
    return rng.normal(0, 1, (rows, cols)) * np.exp(rng.uniform(-10, 10, (rows, 1)))


@pytest.mark.parametrize("fmt,mode", [("e4m3", "floor"), ("e5m2", "ceil")])
def test_exact_accepts_oracle_and_catches_changes(fmt, mode):
    x = _y()
    c, s = oracle.mx_quantize(x, fmt, mode)
    assert_mx_exact("self", torch.from_numpy(c), torch.from_numpy(s), x, fmt, mode)
    c2 = c.copy()
    c2[3, 17] ^= 1
    with pytest.raises(AssertionError):
        assert_mx_exact("code", torch.from_numpy(c2), torch.from_numpy(s), x, fmt, mode)
    s2 = s.copy()
    s2[2, 1] += 1
    with pytest.raises(AssertionError):
        assert_mx_exact("scale", torch.from_numpy(c), torch.from_numpy(s2), x, fmt, mode)


@pytest.mark.parametrize("fmt,mode", [("e4m3", "floor"), ("e4m3", "ceil"), ("e5m2", "floor")])
def test_window_accepts_perturbed_and_catches_changes(fmt, mode):
    y = _y(1)
    rel = np.full(y.shape, 1e-5)
    # a quantisation of Y perturbed inside the bound passes
    rng = np.random.default_rng(2)
    yp = y * (1 + rng.uniform(-1e-5, 1e-5, y.shape))
    c, s = oracle.mx_quantize(yp, fmt, mode)
    st = assert_mx_window("perturbed", torch.from_numpy(c), torch.from_numpy(s), y, rel, None, fmt, mode)
    assert st["unique"] > 0.99 * st["elements"]
    # a code one step off where the window is a single code fails
    c0, s0 = oracle.mx_quantize(y, fmt, mode)
    c2 = c0.copy()
    c2[4, 33] = c2[4, 33] + 1 if (c2[4, 33] & 0x7F) < 0x70 else c2[4, 33] - 1
    with pytest.raises(AssertionError):
        assert_mx_window("code", torch.from_numpy(c2), torch.from_numpy(s0), y, rel, None, fmt, mode)
    # a scale one step off fails
    s2 = s0.copy()
    s2[5, 2] += 1
    with pytest.raises(AssertionError):
        assert_mx_window("scale", torch.from_numpy(c0), torch.from_numpy(s2), y, rel, None, fmt, mode)


def test_window_nonfinite_blocks():
    y = _y(3, rows=2, cols=64)
    y[0, 5] = np.nan
    y[1, 40] = 1e39           # beyond fp32: the fp32 product is infinite
    c, s = oracle.mx_quantize(np.where(np.abs(y) > 3.4e38, np.inf, y), "e4m3", "floor")
    assert s[0, 0] == 255 and s[1, 1] == 255
    assert_mx_window("nonfinite", torch.from_numpy(c), torch.from_numpy(s), y, np.full(y.shape, 1e-5), None,
                     "e4m3", "floor")
    s2 = s.copy()
    s2[0, 0] = 120
    with pytest.raises(AssertionError):
        assert_mx_window("nan scale", torch.from_numpy(c), torch.from_numpy(s2), y, np.full(y.shape, 1e-5),
                         None, "e4m3", "floor")


def test_error_bound_terms():
    gu = np.array([[0.0, 1e-4, 3.0, 0.0, 1e-4, 3.0]])
    r = y_error_bound(gu, 4.0, 25.0, io_bf16=True)
    # G = 1e-4: y = 5e-5 < 2^-11, first-order truncation y/2; U = 1e-4: y = 8e-6
    assert r[0, 1] == pytest.approx(1e-5 + 2.5e-5 + 4e-6)
    assert r[0, 2] == pytest.approx(1e-5 + 2.0 ** -23 / 1.5 + 2.0 ** -23 / 0.24)
    assert np.all(y_error_bound(gu, 4.0, 25.0, io_bf16=False) == 1e-5)
