"""GPU parity on every element of the full-size workloads.

The whole forward and backward run once on the GPU at the workload's full
size, in the launch configuration the benchmark times; the outputs are then
compared with the fp64 oracle chunk by chunk (each row depends only on its
own inputs, so the oracle evaluates any block of rows on its own).  Same bar
as test_gpu_parity.py.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

from compare import assert_close, assert_dr_close
from ref import oracle_results

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
CHUNK_ELEMS = 1 << 23   # elements (rows x intermediate) per oracle chunk


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


@pytest.mark.parametrize("name", ["top1_fwd", "routed_top8", "stress_sat", "dense_ffn"])
def test_every_element_full_size(name):
    from ffn_gated_activation_amd import situ_glu_bwd, situ_glu_fwd
    from ffn_gated_activation_amd.workloads import make_inputs
    print(f"[full] {name}", flush=True)
    x = make_inputs(name, device=DEV, seed=0)
    gu, rw, go = x["gate_up"], x["routing_weights"], x["grad_out"]
    beta, lb, want = x["beta"], x["linear_beta"], x["want_drw"]
    y = situ_glu_fwd(gu, rw, beta, lb)
    dgu = drw = None
    if go is not None:
        dgu, drw = situ_glu_bwd(gu, rw, go, beta, lb, want_drw=want)
    torch.cuda.synchronize()
    rows, inter = y.shape
    step = max(1, CHUNK_ELEMS // inter)
    broadcast = rw.numel() == 1
    worst = {"y": 0, "dG": 0, "dU": 0, "dr": 0.0}
    for lo in range(0, rows, step):
        hi = min(rows, lo + step)
        rws = rw if broadcast else rw[lo:hi]
        gos = None if go is None else go[lo:hi]
        ref = oracle_results(gu[lo:hi], rws, gos, beta, lb, want and not broadcast,
                             backward=go is not None)
        tag = f"{name}[{lo}:{hi}]"
        worst["y"] = max(worst["y"], assert_close(f"{tag} Y", y[lo:hi], ref["y"]))
        if go is not None:
            d = dgu[lo:hi]
            worst["dG"] = max(worst["dG"], assert_close(f"{tag} dG", d[:, :inter], ref["dgu"][:, :inter],
                                                         ref["dg_scale"]))
            worst["dU"] = max(worst["dU"], assert_close(f"{tag} dU", d[:, inter:], ref["dgu"][:, inter:]))
            if want and not broadcast:
                worst["dr"] = max(worst["dr"], assert_dr_close(f"{tag} dr", drw[lo:hi].reshape(-1), ref["dr"],
                                                               ref["dr_abs"]))
    print(f"[full] {name} ok: max bf16 ulp Y {worst['y']} dG {worst['dG']} dU {worst['dU']}; "
          f"max dr error / scale {worst['dr']:.2e}", flush=True)
    del x, gu, rw, go, y, dgu, drw
    torch.cuda.empty_cache()


@pytest.mark.parametrize("inter", [2048, 18432])
def test_broadcast_dr_at_full_rows(inter):
    """One routing weight broadcast over all 16384 rows of the dense-FFN
    recipe, with its gradient (the sum over every row): the per-row partials
    of the row-mapped kernel and the fixed-order second pass over 16384 of
    them (sixteen strided passes per thread of its workgroup).  Every
    element of d_gate_up against the oracle, and the one dr at the parity
    bar (1e-4 of the sum of |go T_g T_u| over all rows, plus one ulp).
    inter = 18432 is the full dense-FFN shape."""
    from ffn_gated_activation_amd import situ_glu_bwd
    from ffn_gated_activation_amd.workloads import make_inputs
    print(f"[full] broadcast dr 16384 x {inter}", flush=True)
    x = make_inputs("dense_ffn", device=DEV, seed=0, inter=inter)
    gu, go = x["gate_up"], x["grad_out"]
    rw = torch.tensor([0.625], device=DEV)
    dgu, drw = situ_glu_bwd(gu, rw, go, 4.0, None, want_drw=True)
    torch.cuda.synchronize()
    rows = gu.shape[0]
    step = max(1, CHUNK_ELEMS // inter)
    total, total_abs, worst = 0.0, 0.0, 0
    for lo in range(0, rows, step):
        hi = min(rows, lo + step)
        # one broadcast weight over the chunk's rows: dr = the chunk's sum, dr_abs per row
        ref = oracle_results(gu[lo:hi], rw, go[lo:hi], 4.0, None, True)
        tag = f"bcast-dr[{lo}:{hi}]"
        worst = max(worst, assert_close(f"{tag} dG", dgu[lo:hi, :inter], ref["dgu"][:, :inter], ref["dg_scale"]))
        worst = max(worst, assert_close(f"{tag} dU", dgu[lo:hi, inter:], ref["dgu"][:, inter:]))
        total += float(ref["dr"][0])
        total_abs += float(np.sum(ref["dr_abs"]))
    err = assert_dr_close("bcast dr", drw.reshape(1), np.array([total]), np.array([total_abs]))
    print(f"[full] broadcast dr 16384 x {inter} ok: max bf16 ulp {worst}, dr {float(drw):.6g} vs {total:.6g}, "
          f"error / scale {err:.2e}", flush=True)

