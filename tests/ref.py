"""Run the fp64 oracle on torch inputs (test infrastructure).

Inputs are widened exactly (bf16 -> fp32 -> fp64 is exact) on the host; the
oracle sees the same values the GPU saw.  `rows` selects a subset of rows (the
oracle computes each row on its own, so a subset gives those rows' exact
results).
"""
from __future__ import annotations

import os

import numpy as np
import torch

import oracle


def host_f64(t: torch.Tensor) -> np.ndarray:
    return t.detach().to("cpu").to(torch.float64).numpy()


def threads() -> int:
    try:
        return max(1, min(16, len(os.sched_getaffinity(0))))
    except AttributeError:
        return max(1, min(16, os.cpu_count() or 1))


def oracle_results(gate_up: torch.Tensor, rw: torch.Tensor, grad_out: torch.Tensor | None, beta: float,
                   linear_beta, want_drw: bool, rows: np.ndarray | None = None, backward: bool = True):
    """fp64 oracle outputs for the selected rows of a (possibly GPU) problem."""
    inter = gate_up.shape[-1] // 2
    gu = gate_up.reshape(-1, 2 * inter)
    r = rw.reshape(-1)
    broadcast = r.numel() == 1 and gu.shape[0] != 1
    if rows is not None:
        idx = torch.as_tensor(rows, dtype=torch.long, device=gu.device)
        gu = gu.index_select(0, idx)
        if not broadcast:
            r = r.index_select(0, idx.to(r.device))
    gu64 = host_f64(gu)
    r64 = host_f64(r)
    out = {"y": oracle.forward(gu64, r64, beta, linear_beta, threads=threads())}
    if backward and grad_out is not None:
        go = grad_out.reshape(-1, inter)
        if rows is not None:
            go = go.index_select(0, idx.to(go.device))
        b = oracle.backward(gu64, r64, host_f64(go), beta, linear_beta, want_dr=want_drw,
                            want_scales=True, threads=threads())
        out.update(dgu=b["d_gate_up"], dr=b["dr"], dr_abs=b["dr_abs"], dg_scale=b["dg_scale"])
    return out


def sample_rows(n_rows: int, k: int = 48, seed: int = 1234) -> np.ndarray:
    """First, last and k seeded random rows, sorted and unique."""
    rng = np.random.default_rng(seed)
    pick = {0, 1, n_rows - 2, n_rows - 1}
    pick |= set(rng.integers(0, n_rows, size=k).tolist())
    return np.array(sorted(p for p in pick if 0 <= p < n_rows), dtype=np.int64)
