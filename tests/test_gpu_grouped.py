"""Fused FC1 grouped GEMM + SiTU-GLU on the GPU against the fp64 oracle.

Every case compares the kernel's bf16 output (and, where asked, its bf16
projections) element by element with oracle.grouped_glu_forward, within the
bound derived in grouped_compare.py.  Small cases check every element; the
full routed-expert workload checks sampled rows of every expert, all
columns, in the launch configuration the benchmark times."""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
from ffn_gated_activation_amd import situ_glu_grouped_fwd
from ffn_gated_activation_amd.workloads import GROUPED, make_grouped_inputs
from grouped_compare import assert_gate_up_close, assert_grouped_close

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def _dev(inp):
    off = torch.tensor(inp["offsets"], dtype=torch.int32, device=DEV)
    return inp["x"].to(DEV), inp["weight"].to(DEV), off, inp["routing_weights"].to(DEV)


def _oracle_rows(inp, rows, beta, lb):
    """Oracle results of the given (sorted) rows, one expert at a time."""
    off = np.asarray(inp["offsets"])
    rows = np.asarray(rows)
    expert = np.searchsorted(off, rows, side="right") - 1
    rw = inp["routing_weights"].double().cpu().numpy().reshape(-1)
    parts = []
    for e in np.unique(expert):
        sel = rows[expert == e]
        xe = inp["x"][torch.from_numpy(sel)].double().cpu().numpy()
        we = inp["weight"][int(e):int(e) + 1].double().cpu().numpy()
        r = rw[sel] if rw.size > 1 else rw
        parts.append(oracle.grouped_glu_forward(xe, we, [0, len(sel)], r, beta, lb))
    return {k: np.concatenate([p[k] for p in parts]) for k in parts[0]}


def _check_all(name, inp, beta, lb, want_gu):
    x, w, off, rw = _dev(inp)
    print(f"[grouped] {name}: rows {x.shape[0]} hidden {x.shape[1]} experts {w.shape[0]} inter {w.shape[1] // 2}",
          flush=True)
    res = situ_glu_grouped_fwd(x, w, off, rw, beta, lb, want_gate_up=want_gu)
    torch.cuda.synchronize()
    out, gu = res if want_gu else (res, None)
    ref = oracle.grouped_glu_forward(inp["x"].double().numpy(), inp["weight"].double().numpy(), inp["offsets"],
                                     inp["routing_weights"].double().numpy(), beta, lb, threads=8)
    ratio = assert_grouped_close(name, out, ref, x.shape[1], beta, lb)
    if gu is not None:
        assert_gate_up_close(name, gu, ref, x.shape[1])
    print(f"[grouped] {name}: max error / bound {ratio:.3g}", flush=True)
    return out


CASES = [
    # name, rows, experts, counts, hidden, inter, rw_mode, beta, linear_beta, want_gate_up
    ("ragged_5_experts", 1000, 5, [300, 0, 1, 437, 262], 512, 256, "uniform", 4.0, 25.0, True),
    ("broadcast_no_lb", 777, 3, None, 256, 384, "one", 2.5, None, False),
    ("many_small_experts", 2000, 300, None, 128, 128, "top8", 4.0, 25.0, False),
    ("one_partial_tile", 64, 1, [64], 64, 128, "uniform", 4.0, 25.0, True),
    ("long_hidden", 304, 2, [129, 175], 7168, 256, "top8", 4.0, 25.0, True),
    ("first_expert_empty", 256, 4, [0, 0, 128, 128], 192, 128, "uniform", 1.5, 8.0, False),
]


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_grouped_matches_oracle(case):
    name, rows, experts, counts, hidden, inter, rw_mode, beta, lb, want_gu = case
    inp = make_grouped_inputs(rows, experts, hidden, inter, seed=11, counts=counts, rw_mode=rw_mode)
    _check_all(name, inp, beta, lb, want_gu)


def test_grouped_bf16_routing_weights():
    inp = make_grouped_inputs(512, 3, 256, 128, seed=5, rw_mode="uniform")
    inp["routing_weights"] = inp["routing_weights"].to(torch.bfloat16)
    _check_all("bf16_rw", inp, 4.0, 25.0, False)


def test_grouped_uncovered_rows_untouched():
    inp = make_grouped_inputs(300, 2, 128, 128, seed=3, counts=[150, 150], rw_mode="uniform")
    x, w, _, rw = _dev(inp)
    off = torch.tensor([5, 100, 250], dtype=torch.int32, device=DEV)
    out = torch.full((300, 128), 7.0, dtype=torch.bfloat16, device=DEV)
    situ_glu_grouped_fwd(x, w, off, rw, 4.0, 25.0, out=out)
    torch.cuda.synchronize()
    assert torch.all(out[:5] == 7.0) and torch.all(out[250:] == 7.0)
    rows = np.arange(5, 250)
    sub = dict(inp, offsets=[0, 5, 100, 250, 300])  # expert 0 = rows 5..99, expert 1 = 100..249
    sub["weight"] = torch.cat([inp["weight"][:1], inp["weight"], inp["weight"][:1]])
    ref = _oracle_rows(sub, rows, 4.0, 25.0)
    assert_grouped_close("uncovered", out, ref, 128, 4.0, 25.0, rows=torch.from_numpy(rows))


def test_grouped_max_experts():
    """SITU_GROUPED_MAX_EXPERTS experts, most with 0 to 2 rows: every
    workgroup scans all 4097 offsets to find its expert."""
    from ffn_gated_activation_amd._capi import SITU_GROUPED_MAX_EXPERTS
    inp = make_grouped_inputs(3000, SITU_GROUPED_MAX_EXPERTS, 64, 128, seed=23, rw_mode="uniform")
    _check_all("max_experts", inp, 4.0, 25.0, False)


def test_grouped_empty():
    x = torch.empty(0, 64, dtype=torch.bfloat16, device=DEV)
    w = torch.zeros(2, 256, 64, dtype=torch.bfloat16, device=DEV)
    off = torch.zeros(3, dtype=torch.int32, device=DEV)
    out = situ_glu_grouped_fwd(x, w, off, torch.ones(1, device=DEV))
    assert out.shape == (0, 128)


def test_grouped_full_workload_sampled():
    wl = GROUPED["grouped_fc1_top8"]
    inp = make_grouped_inputs(wl.rows, wl.experts, wl.hidden, wl.inter, device=DEV, seed=0)
    x, w, off, rw = inp["x"], inp["weight"], torch.tensor(inp["offsets"], dtype=torch.int32, device=DEV), \
        inp["routing_weights"]
    print(f"[grouped] full workload {wl.name}: counts {inp['counts']}", flush=True)
    out, gu = situ_glu_grouped_fwd(x, w, off, rw, wl.beta, wl.linear_beta, want_gate_up=True)
    out2 = situ_glu_grouped_fwd(x, w, off, rw, wl.beta, wl.linear_beta)
    torch.cuda.synchronize()
    assert torch.equal(out, out2), "results differ between two identical calls"
    # the first, second and last rows of every expert and 4 random rows of each
    rng = np.random.default_rng(0)
    o = inp["offsets"]
    rows = set()
    for e in range(wl.experts):
        if o[e + 1] > o[e]:
            rows.update({o[e], min(o[e] + 1, o[e + 1] - 1), o[e + 1] - 1})
            rows.update(rng.integers(o[e], o[e + 1], 4).tolist())
    rows = np.array(sorted(rows))
    cpu = {"x": x[torch.from_numpy(rows).to(DEV)].cpu(), "routing_weights": rw.cpu(), "weight": w,
           "offsets": o}
    # rows of the sample, renumbered: oracle per expert on the selected rows
    expert = np.searchsorted(np.asarray(o), rows, side="right") - 1
    parts, rwc = [], rw.double().cpu().numpy()
    for e in np.unique(expert):
        sel = np.nonzero(expert == e)[0]
        we = w[int(e):int(e) + 1].cpu().double().numpy()
        parts.append(oracle.grouped_glu_forward(cpu["x"][torch.from_numpy(sel)].double().numpy(), we,
                                                [0, len(sel)], rwc[rows[sel]], wl.beta, wl.linear_beta))
    ref = {k: np.concatenate([p[k] for p in parts]) for k in parts[0]}
    idx = torch.from_numpy(rows).to(DEV)
    ratio = assert_grouped_close("full", out[idx], ref, wl.hidden, wl.beta, wl.linear_beta)
    ratio_gu = assert_gate_up_close("full", gu[idx], ref, wl.hidden)
    print(f"[grouped] full: {len(rows)} sampled rows, max error / bound {ratio:.3g} (projections {ratio_gu:.3g})",
          flush=True)
