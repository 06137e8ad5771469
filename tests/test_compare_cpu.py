"""The parity comparator (tests/compare.py) on hand-built cases.

Every GPU parity claim ("within 1 bf16 ulp", "1e-5 relative", "1e-4 of the
row sum's condition scale") is decided by these functions, so they are
checked here against values worked out by hand: bf16 bit patterns chosen
across signed zeros, sign changes, binade edges, subnormals, infinities and
NaN, and fp32 / dr errors just inside and just outside each bar.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import compare
from compare import (CANCEL_MIN, DR_REL, F32_MIN_NORMAL, F32_REL, SUBNORMAL_QUANTA, assert_bf16_close,
                     assert_dr_close, assert_f32_close, bf16_ulp_distance, subnormal_allowance)


@pytest.fixture(autouse=True)
def _keep_tally():
    """The hand-built cases here must not count in the session's dG tally."""
    saved = dict(compare.RELAXED_TALLY)
    yield
    compare.RELAXED_TALLY.update(saved)


def _bf16_from_bits(bits):
    return torch.tensor(np.array(bits, dtype=np.uint16).view(np.int16)).view(torch.bfloat16)


def _bits_value(bits):
    return float(np.array([bits << 16], dtype=np.uint32).view(np.float32)[0])


# (gpu bf16 bits, oracle value, expected ordinal distance)
DIST_CASES = [
    (0x0000, 0.0, 0),                    # +0 vs +0
    (0x8000, 0.0, 0),                    # -0 vs +0: the same point
    (0x0000, -0.0, 0),
    (0x3F80, 1.0, 0),                    # 1.0 exactly
    (0x3F81, 1.0, 1),                    # next bf16 above 1 (1 + 2^-7)
    (0x3F7F, 1.0, 1),                    # previous bf16 below 1 (1 - 2^-8): across the binade edge
    (0x3F7E, 1.0, 2),
    (0x4000, 1.9921875, 1),              # 2.0 vs the largest bf16 below 2
    (0x0001, 0.0, 1),                    # smallest positive subnormal vs 0
    (0x0001, -_bits_value(0x0001), 2),   # across zero: +min_sub vs -min_sub
    (0x8001, _bits_value(0x0001), 2),
    (0x0080, _bits_value(0x007F), 1),    # smallest normal vs largest subnormal
    (0x7F7F, _bits_value(0x7F7F), 0),    # largest finite
    (0x7F80, float("inf"), 0),           # +inf vs +inf
    (0x7F80, _bits_value(0x7F7F), 1),    # +inf is one step past the largest finite
    (0xBF80, -1.0, 0),
    (0xBF81, -1.0, 1),
]


@pytest.mark.parametrize("bits,ref,want", DIST_CASES, ids=[f"{b:#06x}-{r}" for b, r, _ in DIST_CASES])
def test_bf16_ordinal_distance(bits, ref, want):
    d = bf16_ulp_distance(_bf16_from_bits([bits]), np.array([ref], dtype=np.float64))
    assert int(d[0]) == want


def test_bf16_distance_rounds_the_oracle_once():
    """The oracle's fp64 value is rounded to nearest even before the distance:
    a value a hair above the midpoint of two bf16 neighbours belongs to the
    upper one, an exact midpoint to the even one."""
    lo, hi = _bits_value(0x3F80), _bits_value(0x3F81)          # 1, 1 + 2^-7
    mid = 0.5 * (lo + hi)
    g_lo, g_hi = _bf16_from_bits([0x3F80]), _bf16_from_bits([0x3F81])
    assert int(bf16_ulp_distance(g_hi, np.array([mid + 1e-12]))[0]) == 0
    assert int(bf16_ulp_distance(g_lo, np.array([mid + 1e-12]))[0]) == 1
    assert int(bf16_ulp_distance(g_lo, np.array([mid]))[0]) == 0      # tie to even (0x3F80)
    assert int(bf16_ulp_distance(g_hi, np.array([mid]))[0]) == 1


def test_bf16_distance_nan_never_passes():
    big = np.iinfo(np.int32).max
    assert int(bf16_ulp_distance(_bf16_from_bits([0x7FC0]), np.array([1.0]))[0]) == big
    assert int(bf16_ulp_distance(_bf16_from_bits([0x3F80]), np.array([np.nan]))[0]) == big
    with pytest.raises(AssertionError):
        assert_bf16_close("nan", _bf16_from_bits([0x7FC0]), np.array([np.nan]))


def test_bf16_bar_is_one_ulp():
    ref = np.array([1.0, 1.0])
    assert assert_bf16_close("ok", _bf16_from_bits([0x3F81, 0x3F7F]), ref) == 1
    with pytest.raises(AssertionError, match="more than 1 bf16 ulp"):
        assert_bf16_close("off by two", _bf16_from_bits([0x3F82, 0x3F80]), ref)


def test_f32_relative_bar():
    ref = np.array([1.0, -3.0, 1e-30])
    inside = ref * (1.0 + 0.99 * F32_REL)
    assert assert_f32_close("inside", torch.tensor(inside, dtype=torch.float32), ref) <= F32_REL
    for k in range(3):
        bad = ref.copy()
        bad[k] = ref[k] * (1.0 + 1.01 * F32_REL)
        with pytest.raises(AssertionError, match="outside"):
            assert_f32_close("outside", torch.tensor(bad, dtype=torch.float32).double().float(), ref)


def test_f32_bar_floor_at_smallest_normal():
    """A zero reference allows only 1e-5 of the smallest normal number."""
    ref = np.array([0.0, 0.0])
    tiny = F32_REL * F32_MIN_NORMAL
    g = torch.tensor([0.0, 2.0 ** -149], dtype=torch.float32)   # one subnormal quantum
    assert 2.0 ** -149 <= tiny
    assert_f32_close("floor", g, ref)
    with pytest.raises(AssertionError):
        assert_f32_close("above floor", torch.tensor([0.0, 1e-40], dtype=torch.float32), ref)
    # the subnormal allowance widens it by exactly the given absolute amount
    assert_f32_close("allowed", torch.tensor([0.0, 1e-40], dtype=torch.float32), ref,
                     allow64=np.array([0.0, 1e-40]))


def test_f32_dg_term_scale_only_where_the_terms_cancel():
    """dG: where the two terms' magnitudes sum to at least CANCEL_MIN x |dG|
    the bar is 1e-5 of that sum (and the element is counted as relaxed);
    elsewhere it stays 1e-5 of |dG| even when the term sum is larger."""
    ref = np.array([1e-3, 0.5])
    scale = np.array([1.0, 0.9])          # cancellation 1000x and 1.8x
    assert scale[0] >= CANCEL_MIN * ref[0] and scale[1] < CANCEL_MIN * ref[1]
    # element 0: 5e-6 absolute error, inside 1e-5 * 1.0 but outside 1e-5 * 1e-3
    g = torch.tensor([1e-3 + 5e-6, 0.5], dtype=torch.float64)
    st = assert_f32_close("dG", g, ref, scale)
    assert st["relaxed"] == 1 and st["max_rel"] <= F32_REL
    # element 1: 6e-6 absolute is outside 1e-5 * 0.5 even though 1e-5 * 0.9 would admit it
    g2 = torch.tensor([1e-3, 0.5 + 6e-6], dtype=torch.float64)
    with pytest.raises(AssertionError):
        assert_f32_close("dG", g2, ref, scale)
    # nothing relaxed when every element meets the plain bar
    assert assert_f32_close("dG", torch.tensor(ref), ref, scale)["relaxed"] == 0


def test_dr_bar():
    """|gpu - ref| <= 1e-4 * sum_j |go T_g T_u| + one ulp of the dtype of dr
    (fp32 here: 2^-24 |ref|)."""
    ref = np.array([0.0, 10.0])
    abs_scale = np.array([50.0, 20.0])
    tol = DR_REL * abs_scale + 2.0 ** -24 * np.abs(ref)
    g = torch.tensor(ref + 0.99 * tol, dtype=torch.float64)
    assert_dr_close("dr", g, ref, abs_scale)
    with pytest.raises(AssertionError, match="dr values outside"):
        assert_dr_close("dr", torch.tensor(ref + 1.01 * tol, dtype=torch.float64), ref, abs_scale)
    # a bf16 dr adds one bf16 ulp (2^-8 relative): 10.0 against 10.02 passes in
    # bf16 (tol 1e-4 + 2^-8 * 10.02 = 0.0392) and fails in fp32 (tol ~1e-4)
    ref2, sc2 = np.array([10.02]), np.array([1.0])
    assert_dr_close("bf16 dr", torch.tensor([10.0]).to(torch.bfloat16), ref2, sc2)
    with pytest.raises(AssertionError):
        assert_dr_close("fp32 dr", torch.tensor([10.0], dtype=torch.float32), ref2, sc2)
    with pytest.raises(AssertionError):   # the next bf16 value, 10.0625, is outside
        assert_dr_close("bf16 dr", torch.tensor([10.0625]).to(torch.bfloat16), np.array([10.0]), sc2)


def test_subnormal_allowance_values():
    """The backward: 64 subnormal quanta times the bound of the other
    factors, by hand; the forward: 2 quanta."""
    gate_up = np.array([[1.0, -2.0, 30.0, -4.0]])   # G = (1, -2), U = (30, -4)
    r = np.array([0.5])
    go = np.array([[2.0, -1.0]])
    a = subnormal_allowance(gate_up, r, go, 4.0, 25.0)
    tub = np.array([[25.0, 4.0]])                   # min(|U|, 25)
    np.testing.assert_allclose(a["y"], np.full((1, 2), 2 * 2.0 ** -149))   # the forward: 2 quanta flat
    np.testing.assert_allclose(a["dG"], SUBNORMAL_QUANTA * np.array([[2.0, 1.0]]) * 0.5 * (tub + 1.0 + 1.0))
    np.testing.assert_allclose(a["dU"], SUBNORMAL_QUANTA * np.array([[2.0, 1.0]]) * 0.5 * 5.0)
    np.testing.assert_allclose(a["dr"], SUBNORMAL_QUANTA * np.array([2.0 * 29.0 + 1.0 * 8.0]))
    b = subnormal_allowance(gate_up, r, None, 4.0, None)    # no grad_out: the forward's only
    np.testing.assert_allclose(b["y"], np.full((1, 2), 2 * 2.0 ** -149))
    assert set(b) == {"y"}
