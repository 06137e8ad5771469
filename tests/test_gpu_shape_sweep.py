"""Seeded random sweep of the elementwise entry points against the fp64 oracle.

Each case draws its own shape and options from one seed (printed before the
GPU work): io dtype, rows in 1..300, intermediate in 1..3000, beta (4, or
log-uniform in 0.5..50), linear_beta (25, None, or log-uniform in 1..100),
routing weights (fp32 per row, bf16 per row, one broadcast weight),
whether dr is requested, and whether gate_up starts one element past a
16-byte boundary (the element path).  Gate/up values are N(0, s) with s
log-uniform in 0.25..16, so some rows reach the saturated tails.  Every
case runs the forward and the backward at the bar of test_gpu_parity.py;
cases with at least 4096 values per output also run the MXFP8 forward and
backward at the bar of test_gpu_mx.py / test_gpu_bwd_mx.py, in a drawn
format and scale rule."""
from __future__ import annotations

import math

import numpy as np
import pytest
import torch

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
N_CASES = 160


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import ffn_gated_activation_amd  # noqa: F401


def draw_case(seed: int) -> dict:
    """Host-side description of one case (no tensors)."""
    rng = np.random.default_rng(seed)
    return {
        "io": torch.bfloat16 if rng.random() < 0.6 else torch.float32,
        "rows": int(rng.integers(1, 301)),
        "inter": int(rng.choice([rng.integers(1, 65), rng.integers(65, 3001), 8 * rng.integers(1, 375)])),
        "beta": 4.0 if rng.random() < 0.5 else float(math.exp(rng.uniform(math.log(0.5), math.log(50.0)))),
        "linear_beta": [25.0, None, float(math.exp(rng.uniform(0.0, math.log(100.0))))][int(rng.integers(0, 3))],
        "rw_mode": ["f32", "bf16", "broadcast"][int(rng.integers(0, 3))],
        "want_drw": bool(rng.random() < 0.7),
        "misaligned": bool(rng.random() < 0.25),
        "scale": float(math.exp(rng.uniform(math.log(0.25), math.log(16.0)))),
        "fmt": ["e4m3", "e5m2"][int(rng.integers(0, 2))],
        "mode": ["floor", "ceil"][int(rng.integers(0, 2))],
        "data_seed": int(rng.integers(0, 2 ** 31)),
    }


def make_tensors(c: dict):
    g = torch.Generator(device="cpu").manual_seed(c["data_seed"])
    rows, inter = c["rows"], c["inter"]
    gu = (c["scale"] * torch.randn(rows, 2 * inter, generator=g)).to(c["io"])
    go = torch.randn(rows, inter, generator=g).to(c["io"])
    if c["rw_mode"] == "broadcast":
        rw = torch.rand(1, generator=g) + 0.25
    else:
        rw = torch.rand(rows, 1, generator=g)
        if c["rw_mode"] == "bf16":
            rw = rw.to(torch.bfloat16)
    gu, go, rw = gu.to(DEV), go.to(DEV), rw.to(DEV)
    if c["misaligned"]:
        # one element past a 16-byte boundary: the element path
        base = torch.empty(gu.numel() + 1, dtype=gu.dtype, device=DEV)
        base[1:].copy_(gu.reshape(-1))
        gu = base[1:].view(rows, 2 * inter)
    return gu, rw, go


@pytest.mark.parametrize("seed", range(N_CASES))
def test_random_case(seed):
    from test_gpu_parity import run_and_check
    c = draw_case(1000 + seed)
    tag = (f"sweep[{seed}] {c['io']} {c['rows']}x{c['inter']} beta={c['beta']:.4g} lb={c['linear_beta']} "
           f"rw={c['rw_mode']} drw={c['want_drw']} misaligned={c['misaligned']} s={c['scale']:.3g}")
    print(f"[sweep] {tag}", flush=True)
    gu, rw, go = make_tensors(c)
    run_and_check(gu, rw, go, c["beta"], c["linear_beta"], c["want_drw"], tag=tag)
    if c["rows"] * c["inter"] >= 4096:
        from test_gpu_bwd_mx import _check as bwd_mx_check
        from test_gpu_mx import _fused_check
        _fused_check(gu, rw, c["beta"], c["linear_beta"], c["fmt"], c["mode"], tag=tag)
        bwd_mx_check(gu, rw, go, c["beta"], c["linear_beta"], c["fmt"], c["mode"], want_drw=c["want_drw"], tag=tag)


def test_sweep_draws_cover_the_options():
    """The drawn cases reach every option (a check of the generator on the
    host; it launches nothing)."""
    cs = [draw_case(1000 + s) for s in range(N_CASES)]
    assert {c["io"] for c in cs} == {torch.bfloat16, torch.float32}
    assert {c["rw_mode"] for c in cs} == {"f32", "bf16", "broadcast"}
    assert {c["misaligned"] for c in cs} == {True, False}
    assert any(c["linear_beta"] is None for c in cs) and any(c["beta"] != 4.0 for c in cs)
    assert any(c["inter"] % 8 for c in cs) and any(c["inter"] > 1000 for c in cs)
    assert sum(c["rows"] * c["inter"] >= 4096 for c in cs) >= N_CASES // 3
