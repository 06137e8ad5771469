"""GPU parity of the backward with MXFP8 d_gate_up (situ_glu_bwd_mxfp8)
against the fp64 oracle.

The kernel quantises its own fp32 dG and dU.  As for the fused forward
(mx_compare.py), every scale and code must be one the exact gradient could
give under a perturbation within the fp32 chain's bound, here
mx_compare.grad_error_bounds plus the subnormal allowance of compare.py; dG
and dU of a row are checked as two separate rows of blocks.  dr is checked as
for situ_glu_bwd.  Workload recipes at sizes the oracle finishes in seconds,
sampled rows at the full routed-expert size, ragged and misaligned rows, both
formats and scale rules, determinism."""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
from compare import assert_dr_close, subnormal_allowance
from mx_compare import assert_mx_window, grad_error_bounds
from ref import host_f64, sample_rows, threads

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
FORMATS = [("e4m3", "floor"), ("e4m3", "ceil"), ("e5m2", "floor"), ("e5m2", "ceil")]


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import ffn_gated_activation_amd  # noqa: F401


def _say(msg):
    print(msg, flush=True)


def _check(gate_up, rw, grad_out, beta, lb, fmt, mode, want_drw=True, rows=None, tag=""):
    from ffn_gated_activation_amd import situ_glu_bwd_mxfp8
    _say(f"[mx-bwd] {tag} gate_up={tuple(gate_up.shape)} {gate_up.dtype} rw={tuple(rw.shape)} {fmt}/{mode} "
         f"drw={want_drw}")
    codes, scales, drw = situ_glu_bwd_mxfp8(gate_up, rw, grad_out, beta, lb, want_drw, fmt, mode)
    torch.cuda.synchronize()
    inter = gate_up.shape[-1] // 2
    nblk = -(-inter // 32)
    gu = gate_up.reshape(-1, 2 * inter)
    go = grad_out.reshape(-1, inter)
    c = codes.reshape(-1, 2 * inter)
    s = scales.reshape(-1, 2 * nblk)
    r = rw.reshape(-1)
    broadcast = r.numel() == 1 and gu.shape[0] != 1
    if rows is not None:
        idx = torch.as_tensor(rows, device=gu.device)
        gu, go, c, s = (t.index_select(0, idx) for t in (gu, go, c, s))
        if not broadcast:
            r = r.index_select(0, idx.to(r.device))
    gu64, go64, r64 = host_f64(gu), host_f64(go), host_f64(r)
    b = oracle.backward(gu64, r64, go64, beta, lb, want_dr=want_drw, want_scales=True, threads=threads())
    dgu = b["d_gate_up"]
    eg, eu = grad_error_bounds(gu64, dgu, b["dg_scale"], beta, lb, gate_up.dtype == torch.bfloat16)
    al = subnormal_allowance(gu64, r64, go64, beta, lb)
    zero = np.zeros_like(eg)
    st_g = assert_mx_window(f"{tag} dG", c[:, :inter], s[:, :nblk], dgu[:, :inter], zero, eg + al["dG"], fmt, mode)
    st_u = assert_mx_window(f"{tag} dU", c[:, inter:], s[:, nblk:], dgu[:, inter:], zero, eu + al["dU"], fmt, mode)
    if want_drw:
        if broadcast:
            assert rows is None, "a broadcast dr needs every row"
            assert_dr_close(f"{tag} dr", drw.reshape(1), b["dr"], np.array([b["dr_abs"].sum()]),
                            allow64=np.array([al["dr"].sum()]))
        else:
            g = drw.reshape(-1)
            if rows is not None:
                g = g.index_select(0, torch.as_tensor(rows, device=g.device))
            assert_dr_close(f"{tag} dr", g, b["dr"], b["dr_abs"], allow64=al["dr"])
    else:
        assert drw is None
    _say(f"[mx-bwd] {tag} ok dG {st_g} dU {st_u}")
    for st in (st_g, st_u):
        assert st["unique"] >= 0.98 * st["elements"], st   # the windows stay narrow
    return codes, scales, drw


SMALL = [
    ("routed_top8", 64, 2048),
    ("fp32_small", 256, 512),
    ("stress_sat", 48, 2048),
    ("dense_ffn", 6, 18432),      # one broadcast weight, linear_beta None
    ("routed_top8", 16, 40),      # a short last block
    ("routed_top8", 8, 1000),     # 128-bit path, ragged strip
    ("fp32_small", 9, 1003),      # element path
    ("routed_top8", 8, 40000),    # several strips per wavefront
]


@pytest.mark.parametrize("fmt,mode", FORMATS)
@pytest.mark.parametrize("name,rows,inter", SMALL)
def test_bwd_mx_small(name, rows, inter, fmt, mode):
    from ffn_gated_activation_amd.workloads import make_inputs
    x = make_inputs(name, device=DEV, seed=13, rows=rows, inter=inter)
    go = x["grad_out"] if x["grad_out"] is not None else torch.randn(rows, inter, device=DEV).to(x["gate_up"].dtype)
    _check(x["gate_up"], x["routing_weights"], go, x["beta"], x["linear_beta"], fmt, mode,
           want_drw=x["want_drw"], tag=f"{name}[{rows}x{inter}]")


@pytest.mark.parametrize("fmt,mode", [("e4m3", "floor"), ("e5m2", "ceil")])
def test_bwd_mx_full_size_sampled(fmt, mode):
    from ffn_gated_activation_amd.workloads import make_inputs
    x = make_inputs("routed_top8", device=DEV, seed=0)
    rows = sample_rows(x["gate_up"].shape[0], k=60)
    _check(x["gate_up"], x["routing_weights"], x["grad_out"], x["beta"], x["linear_beta"], fmt, mode,
           rows=rows, tag="routed_top8 full, sampled rows")


def test_bwd_mx_broadcast_dr_and_bf16_weights():
    from ffn_gated_activation_amd.workloads import make_inputs
    x = make_inputs("routed_top8", device=DEV, seed=3, rows=304, inter=256)
    one = torch.tensor([0.7], device=DEV)
    _check(x["gate_up"], one, x["grad_out"], 4.0, 25.0, "e4m3", "floor", tag="broadcast weight")
    _check(x["gate_up"], x["routing_weights"].to(torch.bfloat16), x["grad_out"], 2.5, 8.0, "e5m2", "floor",
           tag="bf16 weights, b1 2.5")


def test_bwd_mx_misaligned_element_path():
    from ffn_gated_activation_amd.workloads import make_inputs
    x = make_inputs("routed_top8", device=DEV, seed=5, rows=16, inter=96)
    # offset views: 16-byte alignment lost, so the element path runs
    gu = torch.empty(16 * 192 + 1, dtype=torch.bfloat16, device=DEV)[1:].view(16, 192)
    gu.copy_(x["gate_up"])
    go = torch.empty(16 * 96 + 1, dtype=torch.bfloat16, device=DEV)[1:].view(16, 96)
    go.copy_(x["grad_out"])
    _check(gu, x["routing_weights"], go, 4.0, 25.0, "e4m3", "ceil", tag="misaligned")


def test_bwd_mx_deterministic_and_matches_bf16_dr():
    from ffn_gated_activation_amd import situ_glu_bwd, situ_glu_bwd_mxfp8
    from ffn_gated_activation_amd.workloads import make_inputs
    x = make_inputs("routed_top8", device=DEV, seed=7, rows=512, inter=2048)
    a = situ_glu_bwd_mxfp8(x["gate_up"], x["routing_weights"], x["grad_out"], 4.0, 25.0)
    b = situ_glu_bwd_mxfp8(x["gate_up"], x["routing_weights"], x["grad_out"], 4.0, 25.0)
    _, dr_bf16 = situ_glu_bwd(x["gate_up"], x["routing_weights"], x["grad_out"], 4.0, 25.0)
    torch.cuda.synchronize()
    assert all(torch.equal(p, q) for p, q in zip(a, b)), "results differ between two identical calls"
    # the same per-row reduction as the bf16 backward, both at the oracle's bar
    # (the bf16 backward's up branch may take its polynomial form, so the
    # last bits of the two sums can differ)
    ref = oracle.backward(host_f64(x["gate_up"]), host_f64(x["routing_weights"]), host_f64(x["grad_out"]), 4.0,
                          25.0, want_dr=True, want_scales=True, threads=threads())
    assert_dr_close("mx dr", a[2].reshape(-1), ref["dr"], ref["dr_abs"])
    assert_dr_close("bf16 dr", dr_bf16.reshape(-1), ref["dr"], ref["dr_abs"])


def test_bwd_mx_empty():
    from ffn_gated_activation_amd import situ_glu_bwd_mxfp8
    gu = torch.empty(0, 64, dtype=torch.bfloat16, device=DEV)
    rw = torch.empty(0, 1, device=DEV)
    go = torch.empty(0, 32, dtype=torch.bfloat16, device=DEV)
    c, s, d = situ_glu_bwd_mxfp8(gu, rw, go)
    assert c.shape == (0, 64) and s.shape == (0, 2) and d.shape == (0, 1)
