"""Seeded random sweep of attention-residual mixing against the fp64 oracle.

Each case draws from one seed (printed before the GPU work): tokens in
1..900 (fewer when the values would pass ~42M), stored block sums 0..15
with or without the prefix (1 to 16 values per token in all), hidden either
a multiple of 8 up to 12288 or any width up to 3000 (the element path),
value, weight and output dtypes, and eps (1e-6, 0, or log-uniform in
1e-8..1).  Bar as test_gpu_attn_res.py."""
from __future__ import annotations

import math

import numpy as np
import pytest
import torch

pytestmark = pytest.mark.gpu
N_CASES = 60
DTS = [torch.bfloat16, torch.float32]


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import ffn_gated_activation_amd  # noqa: F401


def draw_case(seed: int) -> dict:
    rng = np.random.default_rng(seed)
    prefix = bool(rng.random() < 0.75)
    stored = int(rng.integers(0 if prefix else 1, 16))
    hidden = 8 * int(rng.integers(1, 1537)) if rng.random() < 0.7 else int(rng.integers(1, 3001))
    tokens = int(rng.integers(1, 901))
    tokens = max(1, min(tokens, (40 << 20) // ((stored + prefix) * hidden)))  # at most ~42M values a case
    return {
        "tokens": tokens,
        "stored": stored,
        "prefix": prefix,
        "hidden": hidden,
        "dt": DTS[int(rng.integers(0, 2))],
        "wdt": DTS[int(rng.integers(0, 2))],
        "odt": DTS[int(rng.integers(0, 2))],
        "eps": [1e-6, 0.0, float(math.exp(rng.uniform(math.log(1e-8), 0.0)))][int(rng.integers(0, 3))],
        "data_seed": int(rng.integers(0, 2 ** 31)),
    }


@pytest.mark.parametrize("seed", range(N_CASES))
def test_random_attn_res(seed):
    from test_gpu_attn_res import _check
    from ffn_gated_activation_amd.workloads import make_attn_res_inputs
    c = draw_case(4000 + seed)
    tag = (f"ares-sweep[{seed}] T{c['tokens']} m{c['stored']} prefix={c['prefix']} H{c['hidden']} "
           f"{c['dt']} w={c['wdt']} out={c['odt']} eps={c['eps']:.3g}")
    x = make_attn_res_inputs(c["tokens"], c["stored"], c["hidden"], c["prefix"], c["dt"], c["wdt"], device="cuda:0",
                             seed=c["data_seed"], eps=c["eps"])
    if c["stored"] == 0:
        x["blocks"] = None
    _check(x, c["odt"], tag=tag)


def test_attn_res_sweep_draws_cover_the_options():
    """Host-side check of the generator: it launches nothing."""
    cs = [draw_case(4000 + s) for s in range(N_CASES)]
    assert {c["prefix"] for c in cs} == {True, False}
    assert any(c["stored"] == 0 for c in cs) and any(c["stored"] + c["prefix"] >= 12 for c in cs)
    assert any(c["hidden"] % 8 for c in cs) and any(c["hidden"] > 8192 for c in cs)
    assert {c["dt"] for c in cs} == {c["odt"] for c in cs} == set(DTS)
    assert any(c["eps"] == 0.0 for c in cs)
