"""Fused FC1 grouped GEMM + SiTU-GLU on MXFP8 operands, on the GPU, against
the fp64 oracle.

Every case compares the kernel's bf16 output (and, where asked, its bf16
projections) element by element with oracle.grouped_glu_forward_mx, which
decodes the MX blocks (mx_dequantize) and takes the products exactly, within
the bound derived in grouped_compare.py for the scaled matrix cores.  Small
cases check every element; the full routed-expert workload checks sampled
rows of every expert, all columns, in the launch configuration the benchmark
times."""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
from ffn_gated_activation_amd import situ_glu_grouped_fwd_mxfp8
from ffn_gated_activation_amd.workloads import GROUPED_MX, make_grouped_mx_inputs
from grouped_compare import assert_gate_up_close, assert_grouped_close, mx_exponent_sums

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def _run(inp, beta, lb, want_gu=False, off=None, out=None):
    d = lambda t: t.to(DEV)  # noqa: E731
    if off is None:
        off = torch.tensor(inp["offsets"], dtype=torch.int32, device=DEV)
    return situ_glu_grouped_fwd_mxfp8(d(inp["x_codes"]), d(inp["x_scales"]), d(inp["weight_codes"]),
                                      d(inp["weight_scales"]), off, d(inp["routing_weights"]),
                                      inp["fp8_format"], beta, lb, want_gate_up=want_gu, out=out)


def _oracle(inp, beta, lb, rows=None):
    """Oracle results of all rows, or of the given (sorted) rows one expert
    at a time, with the exponent sums the tolerance of the scaled matrix
    cores needs (grouped_compare.mx_exponent_sums)."""
    cpu = lambda t: t.cpu().numpy()  # noqa: E731
    fmt = inp["fp8_format"]
    rw = inp["routing_weights"].double().cpu().numpy().reshape(-1)
    if rows is None:
        xc, xs, wc, ws = cpu(inp["x_codes"]), cpu(inp["x_scales"]), cpu(inp["weight_codes"]), \
            cpu(inp["weight_scales"])
        ref = oracle.grouped_glu_forward_mx(xc, xs, wc, ws, inp["offsets"], rw, fmt, beta, lb, threads=8)
        return ref, mx_exponent_sums(xc, xs, wc, ws, inp["offsets"], fmt)
    off = np.asarray(inp["offsets"])
    expert = np.searchsorted(off, rows, side="right") - 1
    parts, exps = [], []
    for e in np.unique(expert):
        sel = torch.from_numpy(rows[expert == e]).to(inp["x_codes"].device)
        r = rw[rows[expert == e]] if rw.size > 1 else rw
        xc, xs = cpu(inp["x_codes"][sel]), cpu(inp["x_scales"][sel])
        wc, ws = cpu(inp["weight_codes"][int(e):int(e) + 1]), cpu(inp["weight_scales"][int(e):int(e) + 1])
        parts.append(oracle.grouped_glu_forward_mx(xc, xs, wc, ws, [0, len(sel)], r, fmt, beta, lb))
        exps.append(mx_exponent_sums(xc, xs, wc, ws, [0, len(sel)], fmt))
    return {k: np.concatenate([p[k] for p in parts]) for k in parts[0]}, np.concatenate(exps)


CASES = [
    # name, rows, experts, counts, hidden, inter, fmt, rw_mode, beta, linear_beta, want_gate_up
    ("ragged_5_experts_e4m3", 1000, 5, [300, 0, 1, 437, 262], 512, 256, "e4m3", "uniform", 4.0, 25.0, True),
    ("ragged_5_experts_e5m2", 1000, 5, [300, 0, 1, 437, 262], 512, 256, "e5m2", "uniform", 4.0, 25.0, True),
    ("broadcast_no_lb", 777, 3, None, 256, 384, "e4m3", "one", 2.5, None, False),
    ("many_small_experts", 2000, 300, None, 128, 128, "e5m2", "top8", 4.0, 25.0, False),
    ("one_partial_tile", 64, 1, [64], 128, 128, "e4m3", "uniform", 4.0, 25.0, True),
    ("long_hidden_e4m3", 304, 2, [129, 175], 7168, 256, "e4m3", "top8", 4.0, 25.0, True),
    ("long_hidden_e5m2", 304, 2, [129, 175], 7168, 256, "e5m2", "top8", 4.0, 25.0, False),
    ("first_expert_empty", 256, 4, [0, 0, 128, 128], 384, 128, "e4m3", "uniform", 1.5, 8.0, False),
]


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_grouped_mx_matches_oracle(case):
    name, rows, experts, counts, hidden, inter, fmt, rw_mode, beta, lb, want_gu = case
    inp = make_grouped_mx_inputs(rows, experts, hidden, inter, fmt, seed=13, counts=counts, rw_mode=rw_mode)
    print(f"[grouped_mx] {name}: rows {rows} hidden {hidden} experts {experts} inter {inter} {fmt}", flush=True)
    res = _run(inp, beta, lb, want_gu)
    torch.cuda.synchronize()
    out, gu = res if want_gu else (res, None)
    ref, mx_exp = _oracle(inp, beta, lb)
    ratio = assert_grouped_close(name, out, ref, hidden, beta, lb, mx_exp=mx_exp)
    if gu is not None:
        assert_gate_up_close(name, gu, ref, hidden, mx_exp=mx_exp)
    print(f"[grouped_mx] {name}: max error / bound {ratio:.3g}", flush=True)


def test_grouped_mx_bf16_routing_weights_and_zero_codes():
    inp = make_grouped_mx_inputs(512, 3, 256, 128, "e4m3", seed=5, rw_mode="uniform")
    inp["routing_weights"] = inp["routing_weights"].to(torch.bfloat16)
    inp["x_codes"][7] = 0                       # an all-zero row
    inp["x_codes"][9, 32:64] = 0x80             # a block of negative zeros
    inp["weight_scales"][1, 5] = 90             # blocks scaled far apart (2^-37 and 2^13), products
    inp["x_scales"][11, 2] = 140                # still inside the fp32 normal range
    out = _run(inp, 4.0, 25.0)
    torch.cuda.synchronize()
    ref, mx_exp = _oracle(inp, 4.0, 25.0)
    assert_grouped_close("bf16_rw", out, ref, 256, 4.0, 25.0, mx_exp=mx_exp)


def test_grouped_mx_uncovered_rows_untouched():
    inp = make_grouped_mx_inputs(300, 2, 128, 128, "e4m3", seed=3, counts=[150, 150], rw_mode="uniform")
    off = torch.tensor([5, 100, 250], dtype=torch.int32, device=DEV)
    out = torch.full((300, 128), 7.0, dtype=torch.bfloat16, device=DEV)
    _run(inp, 4.0, 25.0, off=off, out=out)
    torch.cuda.synchronize()
    assert torch.all(out[:5] == 7.0) and torch.all(out[250:] == 7.0)
    rows = np.arange(5, 250)
    sub = dict(inp, offsets=[0, 5, 100, 250, 300])  # expert 0 = rows 5..99, expert 1 = 100..249
    sub["weight_codes"] = torch.cat([inp["weight_codes"][:1], inp["weight_codes"], inp["weight_codes"][:1]])
    sub["weight_scales"] = torch.cat([inp["weight_scales"][:1], inp["weight_scales"], inp["weight_scales"][:1]])
    ref, mx_exp = _oracle(sub, 4.0, 25.0, rows=rows)
    assert_grouped_close("uncovered", out, ref, 128, 4.0, 25.0, rows=torch.from_numpy(rows), mx_exp=mx_exp)


def test_grouped_mx_max_experts():
    from ffn_gated_activation_amd._capi import SITU_GROUPED_MAX_EXPERTS
    inp = make_grouped_mx_inputs(3000, SITU_GROUPED_MAX_EXPERTS, 128, 128, "e5m2", seed=29, rw_mode="uniform")
    out = _run(inp, 4.0, 25.0)
    torch.cuda.synchronize()
    ref, mx_exp = _oracle(inp, 4.0, 25.0)
    assert_grouped_close("max_experts", out, ref, 128, 4.0, 25.0, mx_exp=mx_exp)


def test_grouped_mx_empty():
    u8 = torch.uint8
    out = situ_glu_grouped_fwd_mxfp8(torch.empty(0, 128, dtype=u8, device=DEV), torch.empty(0, 4, dtype=u8,
                                     device=DEV), torch.zeros(2, 256, 128, dtype=u8, device=DEV),
                                     torch.zeros(2, 256, 4, dtype=u8, device=DEV),
                                     torch.zeros(3, dtype=torch.int32, device=DEV), torch.ones(1, device=DEV))
    assert out.shape == (0, 128)


def test_grouped_mx_full_workload_sampled():
    wl = GROUPED_MX["grouped_fc1_top8_mxfp8"]
    inp = make_grouped_mx_inputs(wl.rows, wl.experts, wl.hidden, wl.inter, "e4m3", device=DEV, seed=0)
    print(f"[grouped_mx] full workload {wl.name}: counts {inp['counts']}", flush=True)
    out, gu = _run(inp, wl.beta, wl.linear_beta, want_gu=True)
    out2 = _run(inp, wl.beta, wl.linear_beta)
    torch.cuda.synchronize()
    assert torch.equal(out, out2), "results differ between two identical calls"
    rng = np.random.default_rng(0)
    o = inp["offsets"]
    rows = set()
    for e in range(wl.experts):
        if o[e + 1] > o[e]:
            rows.update({o[e], min(o[e] + 1, o[e + 1] - 1), o[e + 1] - 1})
            rows.update(rng.integers(o[e], o[e + 1], 4).tolist())
    rows = np.array(sorted(rows))
    ref, mx_exp = _oracle(inp, wl.beta, wl.linear_beta, rows=rows)
    idx = torch.from_numpy(rows).to(DEV)
    ratio = assert_grouped_close("full", out[idx], ref, wl.hidden, wl.beta, wl.linear_beta, mx_exp=mx_exp)
    ratio_gu = assert_gate_up_close("full", gu[idx], ref, wl.hidden, mx_exp=mx_exp)
    print(f"[grouped_mx] full: {len(rows)} sampled rows, max error / bound {ratio:.3g} (projections "
          f"{ratio_gu:.3g})", flush=True)


def test_grouped_mx_nan_scale_does_not_leak():
    """hidden 640: 5 stages of 128 (an odd count: the loop adds a stage of
    zeros, whose scales come from an empty descriptor).  A NaN scale (byte
    255) at the start of x row 51 and of weight row 11, the bytes right after
    rows 50 and 10, must reach only that row's / that column's results."""
    hidden, inter = 640, 128
    inp = make_grouped_mx_inputs(300, 2, hidden, inter, "e4m3", seed=17, counts=[150, 150], rw_mode="uniform")
    inp["x_scales"][51, 0] = 255
    inp["weight_scales"][0, 11, 0] = 255
    out = _run(inp, 4.0, 25.0)
    torch.cuda.synchronize()
    ref, mx_exp = _oracle(inp, 4.0, 25.0)
    from grouped_compare import output_bound
    bound = output_bound(ref, hidden, 4.0, 25.0, mx_exp)
    y = out.double().cpu().numpy()
    keep = np.ones_like(y, dtype=bool)
    keep[51, :] = False
    keep[:150, 11] = False        # expert 0's gate column 11
    assert np.isfinite(ref["out"][keep]).all()
    err = np.abs(y - ref["out"])
    bad = keep & ~(err <= bound)
    assert not bad.any(), f"{int(bad.sum())} outputs outside the bound, first at {np.argwhere(bad)[0]}"


def test_grouped_mx_explicit_workspace():
    """A caller-provided workspace gives the same bits as the one allocated by
    the binding; one byte too small is rejected before any launch."""
    from ffn_gated_activation_amd import SituGluError, situ_glu_grouped_fwd_mxfp8_workspace_bytes
    rows, experts, hidden, inter = 700, 3, 384, 256
    inp = make_grouped_mx_inputs(rows, experts, hidden, inter, "e4m3", seed=31, rw_mode="uniform")
    need = situ_glu_grouped_fwd_mxfp8_workspace_bytes(rows, hidden, experts, inter)
    ref = _run(inp, 4.0, 25.0)
    d = lambda t: t.to(DEV)  # noqa: E731
    off = torch.tensor(inp["offsets"], dtype=torch.int32, device=DEV)
    args = (d(inp["x_codes"]), d(inp["x_scales"]), d(inp["weight_codes"]), d(inp["weight_scales"]), off,
            d(inp["routing_weights"]), "e4m3", 4.0, 25.0)
    wk = torch.full((need,), 0xA5, dtype=torch.uint8, device=DEV)     # stale contents must not matter
    out = situ_glu_grouped_fwd_mxfp8(*args, workspace=wk)
    torch.cuda.synchronize()
    assert torch.equal(out, ref)
    small = torch.empty(need - 1, dtype=torch.uint8, device=DEV)
    keep = torch.full((rows, inter), 3.0, dtype=torch.bfloat16, device=DEV)
    with pytest.raises(SituGluError):
        situ_glu_grouped_fwd_mxfp8(*args, out=keep, workspace=small)
    torch.cuda.synchronize()
    assert torch.all(keep == 3.0)
