"""The benchmark's parity gate, on the CPU.

bench.py reports no throughput for a step whose outputs disagree with the
oracle.  These checks feed its gate the oracle's own results, rounded to the
output dtype the way a correct kernel would store them, and then the same
results with one planted error in each output: the gate must pass the first
and fail every planted case.  Inputs are the seeded workload recipes at
their small sizes (fp32_small whole; top1_fwd rows, with the bf16 backward
run on them too)."""
from __future__ import annotations

import os
import sys

import numpy as np
import pytest
import torch

import oracle

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import bench  # noqa: E402
from ffn_gated_activation_amd.workloads import make_inputs  # noqa: E402


def _oracle_outputs(gu, rw, go, beta, lb, dtype):
    g64 = gu.double().numpy()
    r64 = rw.double().numpy().reshape(-1)
    y = oracle.forward(g64, r64, beta, lb)
    b = oracle.backward(g64, r64, go.double().numpy(), beta, lb, want_dr=True, want_scales=True)
    if dtype == torch.bfloat16:
        # the oracle's own fp64 -> bf16 rounding (round to nearest even)
        def rnd(a):
            bits = oracle.round_bf16_bits(a).astype(np.uint32) << 16
            return torch.from_numpy(bits.view(np.float32)).to(torch.bfloat16)
    else:
        def rnd(a):
            return torch.from_numpy(a.astype(np.float32))
    outs = {"y": rnd(y), "dgu": rnd(b["d_gate_up"]),
            "drw": torch.from_numpy(b["dr"].astype(np.float32)).reshape(-1, 1)}
    return outs, y, b


@pytest.mark.parametrize("name", ["fp32_small", "top1_fwd"])
def test_gate_passes_correct_outputs_and_fails_planted_errors(name):
    x = make_inputs(name, device="cpu", seed=0)
    gu, rw = x["gate_up"], x["routing_weights"]
    rows = 64 if name == "top1_fwd" else gu.shape[0]
    gu = gu[:rows].contiguous()
    rw = rw[:rows].contiguous() if rw.numel() > 1 else rw
    inter = gu.shape[1] // 2
    gen = torch.Generator().manual_seed(3)
    go = torch.randn(rows, inter, generator=gen).to(gu.dtype)
    outs, y, b = _oracle_outputs(gu, rw, go, x["beta"], x["linear_beta"], gu.dtype)
    idx = torch.arange(rows)
    gate = bench._parity if gu.dtype == torch.bfloat16 else bench._parity_f32
    ok = gate(outs, idx, inter, y, b, True, rows, rows)
    assert ok["pass"], ok

    # planted errors: two bf16 ulps (one would still be inside the bar) or
    # 3e-5 relative for fp32, in Y, in dG, in dU; dr off by 2e-4 of its scale
    i, j = rows // 3, inter // 5
    for key, col in (("y", j), ("dgu", j), ("dgu", inter + j)):
        bad = {k: v.clone() for k, v in outs.items()}
        t = bad[key][i, col:col + 1]
        if gu.dtype == torch.bfloat16:
            bits = t.view(torch.int16)
            t.copy_((bits + 2).view(torch.bfloat16))
        else:
            t.mul_(1 + 3e-5)
        res = gate(bad, idx, inter, y, b, True, rows, rows)
        assert not res["pass"], (key, col, res)
    bad = {k: v.clone() for k, v in outs.items()}
    bad["drw"][i] += float(2e-4 * b["dr_abs"][i])
    res = gate(bad, idx, inter, y, b, True, rows, rows)
    assert not res["pass"] and res["dr_within_bar"] is False, res
