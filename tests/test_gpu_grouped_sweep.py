"""Seeded random sweep of the fused grouped GEMM + SiTU-GLU (bf16 and MXFP8
operands) against the fp64 oracle, every element.

Each case draws from one seed (printed before the GPU work): experts in
1..40, rows in 1..1200 split over the experts by a multinomial draw (so
some experts are empty and many tiles partial), hidden a multiple of 64
(bf16) or 128 (MXFP8) up to 1024, intermediate a multiple of 128 up to 512,
routing weights (per row uniform, per token softmax of 8 when rows allow,
or one broadcast weight), beta (4, or log-uniform in 0.5..50), linear_beta
(25, None, or log-uniform in 1..100), whether the projections are also
written, and for MXFP8 the element format.  Bars as test_gpu_grouped.py and
test_gpu_grouped_mx.py."""
from __future__ import annotations

import math

import numpy as np
import pytest
import torch

pytestmark = pytest.mark.gpu
N_CASES = 24


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import ffn_gated_activation_amd  # noqa: F401


def draw_case(seed: int, mx: bool) -> dict:
    rng = np.random.default_rng(seed)
    rows = int(rng.integers(1, 1201))
    modes = ["uniform", "one"] + (["top8"] if rows % 8 == 0 else [])
    step = 128 if mx else 64
    return {
        "rows": rows,
        "experts": int(rng.integers(1, 41)),
        "hidden": step * int(rng.integers(1, 1024 // step + 1)),
        "inter": 128 * int(rng.integers(1, 5)),
        "rw_mode": modes[int(rng.integers(0, len(modes)))],
        "beta": 4.0 if rng.random() < 0.5 else float(math.exp(rng.uniform(math.log(0.5), math.log(50.0)))),
        "linear_beta": [25.0, None, float(math.exp(rng.uniform(0.0, math.log(100.0))))][int(rng.integers(0, 3))],
        "want_gu": bool(rng.random() < 0.5),
        "fmt": ["e4m3", "e5m2"][int(rng.integers(0, 2))],
        "data_seed": int(rng.integers(0, 2 ** 31)),
    }


def _tag(c, mx):
    return (f"{'mx ' + c['fmt'] if mx else 'bf16'} rows {c['rows']} experts {c['experts']} hidden {c['hidden']} "
            f"inter {c['inter']} rw {c['rw_mode']} beta {c['beta']:.4g} lb {c['linear_beta']} gu {c['want_gu']}")


@pytest.mark.parametrize("seed", range(N_CASES))
def test_random_grouped_bf16(seed):
    from test_gpu_grouped import _check_all
    from ffn_gated_activation_amd.workloads import make_grouped_inputs
    c = draw_case(2000 + seed, mx=False)
    print(f"[grouped-sweep] {seed}: {_tag(c, False)}", flush=True)
    inp = make_grouped_inputs(c["rows"], c["experts"], c["hidden"], c["inter"], seed=c["data_seed"],
                              rw_mode=c["rw_mode"])
    _check_all(f"sweep {seed}", inp, c["beta"], c["linear_beta"], c["want_gu"])


@pytest.mark.parametrize("seed", range(N_CASES))
def test_random_grouped_mx(seed):
    from test_gpu_grouped_mx import _oracle, _run
    from ffn_gated_activation_amd.workloads import make_grouped_mx_inputs
    from grouped_compare import assert_gate_up_close, assert_grouped_close
    c = draw_case(3000 + seed, mx=True)
    print(f"[grouped-sweep] {seed}: {_tag(c, True)}", flush=True)
    inp = make_grouped_mx_inputs(c["rows"], c["experts"], c["hidden"], c["inter"], c["fmt"], seed=c["data_seed"],
                                 rw_mode=c["rw_mode"])
    res = _run(inp, c["beta"], c["linear_beta"], c["want_gu"])
    torch.cuda.synchronize()
    out, gu = res if c["want_gu"] else (res, None)
    ref, mx_exp = _oracle(inp, c["beta"], c["linear_beta"])
    ratio = assert_grouped_close(f"mx sweep {seed}", out, ref, c["hidden"], c["beta"], c["linear_beta"],
                                 mx_exp=mx_exp)
    if gu is not None:
        assert_gate_up_close(f"mx sweep {seed}", gu, ref, c["hidden"], mx_exp=mx_exp)
    print(f"[grouped-sweep] {seed}: max error / bound {ratio:.3g}", flush=True)


def test_grouped_sweep_draws_cover_the_options():
    """Host-side check of the generator: it launches nothing."""
    for mx, base in ((False, 2000), (True, 3000)):
        cs = [draw_case(base + s, mx) for s in range(N_CASES)]
        assert {c["rw_mode"] for c in cs} >= {"uniform", "one"}
        assert any(c["linear_beta"] is None for c in cs) and any(c["beta"] != 4.0 for c in cs)
        assert {c["want_gu"] for c in cs} == {True, False}
        assert any(c["rows"] < 256 for c in cs) and any(c["experts"] > 20 for c in cs)
        if mx:
            assert {c["fmt"] for c in cs} == {"e4m3", "e5m2"}
