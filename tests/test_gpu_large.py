"""GPU parity past the 32-bit offsets: every entry point on tensors whose
byte (and, for bf16, element) offsets exceed 2^31 and 2^32.

The kernels address each row (token, row tile) from a 64-bit base and use
32-bit offsets only inside it; these cases put rows on both sides of the
2^31- and 2^32-byte marks of every input and output and compare them, with
the first, last and seeded random rows, against the fp64 oracle at the same
bar as the full-size sampled tests.  Each case frees its tensors before the
next (the largest holds about 30 GB of device memory)."""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
from ref import sample_rows

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import ffn_gated_activation_amd  # noqa: F401  (fails loudly if the library is not built)
    yield
    torch.cuda.empty_cache()


def _rows_around(n_rows: int, row_bytes: list[int], k: int = 24) -> np.ndarray:
    """First, last and k random rows, plus the rows on both sides of the
    2^31- and 2^32-byte marks of arrays with the given bytes per row."""
    pick = set(sample_rows(n_rows, k=k).tolist())
    for b in row_bytes:
        for mark in (1 << 31, 1 << 32):
            r = mark // b
            pick |= {r - 1, r, r + 1}
    return np.array(sorted(p for p in pick if 0 <= p < n_rows), dtype=np.int64)


def _free():
    torch.cuda.synchronize()
    torch.cuda.empty_cache()


@pytest.mark.parametrize("name,rows", [("routed_top8", (1 << 19) + 64), ("fp32_small", (1 << 18) + 8)])
def test_elementwise_past_32bit_offsets(name, rows):
    """bf16: gate_up [2^19 + 64, 4096] is 2^31 + 2^18 elements (4.3 GB);
    fp32: [2^18 + 8, 4096] is 4.3 GB.  Forward, backward and dr."""
    from test_gpu_parity import run_and_check
    from ffn_gated_activation_amd.workloads import make_inputs
    x = make_inputs(name, device=DEV, seed=5, rows=rows, inter=2048)
    gu = x["gate_up"]
    go = x["grad_out"] if x["grad_out"] is not None else torch.randn(rows, 2048, device=DEV).to(gu.dtype)
    es = gu.element_size()
    sel = _rows_around(rows, [4096 * es, 2048 * es])
    run_and_check(gu, x["routing_weights"], go, x["beta"], x["linear_beta"], True, rows=sel,
                  tag=f"{name} {rows}x2048 past 2^32 bytes")
    del x, gu, go
    _free()


def test_mx_forward_and_backward_past_32bit_offsets():
    """MXFP8 forward and backward on the bf16 routed recipe at
    [2^19 + 64, 4096] (gate_up 4.3 GB, backward codes 2^31 + 2^18 bytes)."""
    from test_gpu_bwd_mx import _check as bwd_check
    from test_gpu_mx import _fused_check
    from ffn_gated_activation_amd.workloads import make_inputs
    rows = (1 << 19) + 64
    x = make_inputs("routed_top8", device=DEV, seed=6, rows=rows, inter=2048)
    sel = _rows_around(rows, [8192, 4096, 2048])
    _fused_check(x["gate_up"], x["routing_weights"], x["beta"], x["linear_beta"], "e4m3", "floor", rows=sel,
                 tag="routed_top8 past 2^32 bytes")
    bwd_check(x["gate_up"], x["routing_weights"], x["grad_out"], x["beta"], x["linear_beta"], "e4m3", "floor",
              rows=sel, tag="routed_top8 past 2^32 bytes")
    del x
    _free()


def test_quantize_past_32bit_offsets():
    """Standalone MXFP8 quantisation of x [2^19 + 64, 4096] bf16: every
    sampled row's codes and scales equal the oracle's, bit for bit."""
    from ffn_gated_activation_amd import situ_glu_mx_quantize
    from mx_compare import assert_mx_exact
    from ref import host_f64
    rows, cols = (1 << 19) + 64, 4096
    g = torch.Generator(device=DEV)
    g.manual_seed(7)
    x = (3.0 * torch.randn(rows, cols, generator=g, device=DEV)).to(torch.bfloat16)
    codes, scales = situ_glu_mx_quantize(x, "e4m3", "floor")
    torch.cuda.synchronize()
    sel = _rows_around(rows, [cols * 2, cols])
    idx = torch.from_numpy(sel).to(DEV)
    assert_mx_exact("quantize large", codes.index_select(0, idx), scales.index_select(0, idx),
                    host_f64(x.index_select(0, idx)), "e4m3", "floor")
    print(f"[large] quantize: {len(sel)} rows bit-exact", flush=True)
    del x, codes, scales
    _free()


def test_attn_res_past_32bit_offsets():
    """Attention-residual mixing over blocks [40000, 8, 7168] bf16 (4.6 GB)
    plus the prefix; sampled tokens around the marks of the blocks array."""
    from test_gpu_attn_res import _check
    from ffn_gated_activation_amd.workloads import make_attn_res_inputs
    T, m, H = 40000, 8, 7168
    x = make_attn_res_inputs(T, m, H, True, device=DEV, seed=8, eps=1e-6)
    _check(x, tokens=_rows_around(T, [m * H * 2, H * 2], k=16), tag=f"attn_res {T}x{m}x{H} past 2^32 bytes")
    del x
    _free()


def _grouped_sample(offsets, n_rows, row_bytes, seed=0):
    o = np.asarray(offsets)
    rng = np.random.default_rng(seed)
    pick = set(_rows_around(n_rows, row_bytes, k=8).tolist())
    for e in range(len(o) - 1):
        if o[e + 1] > o[e]:
            pick |= {int(o[e]), int(o[e + 1]) - 1}
            pick |= set(rng.integers(o[e], o[e + 1], 2).tolist())
    return np.array(sorted(pick), dtype=np.int64)


def test_grouped_bf16_past_32bit_offsets():
    """Fused grouped GEMM + SiTU-GLU, x [2^20 + 256, 2048] bf16 (4.3 GB),
    4 experts, intermediate 2048: out 4.3 GB, projections 8.6 GB."""
    from ffn_gated_activation_amd import situ_glu_grouped_fwd
    from ffn_gated_activation_amd.workloads import make_grouped_inputs
    from grouped_compare import assert_gate_up_close, assert_grouped_close
    rows, experts, hidden, inter = (1 << 20) + 256, 4, 2048, 2048
    inp = make_grouped_inputs(rows, experts, hidden, inter, device=DEV, seed=9)
    x, w, rw = inp["x"], inp["weight"], inp["routing_weights"]
    off = torch.tensor(inp["offsets"], dtype=torch.int32, device=DEV)
    print(f"[large] grouped bf16: counts {inp['counts']}", flush=True)
    out, gu = situ_glu_grouped_fwd(x, w, off, rw, 4.0, 25.0, want_gate_up=True)
    torch.cuda.synchronize()
    sel = _grouped_sample(inp["offsets"], rows, [hidden * 2, inter * 2, inter * 4])
    expert = np.searchsorted(np.asarray(inp["offsets"]), sel, side="right") - 1
    rwc = rw.double().cpu().numpy()
    parts = []
    for e in np.unique(expert):
        s = sel[expert == e]
        xe = x.index_select(0, torch.from_numpy(s).to(DEV)).double().cpu().numpy()
        we = w[int(e):int(e) + 1].double().cpu().numpy()
        parts.append(oracle.grouped_glu_forward(xe, we, [0, len(s)], rwc[s], 4.0, 25.0))
    ref = {k: np.concatenate([p[k] for p in parts]) for k in parts[0]}
    idx = torch.from_numpy(sel).to(DEV)
    ratio = assert_grouped_close("grouped large", out.index_select(0, idx), ref, hidden, 4.0, 25.0)
    ratio_gu = assert_gate_up_close("grouped large", gu.index_select(0, idx), ref, hidden)
    print(f"[large] grouped bf16: {len(sel)} rows, max error / bound {ratio:.3g} (projections {ratio_gu:.3g})",
          flush=True)
    del inp, x, w, rw, off, out, gu
    _free()


def test_grouped_mx_past_32bit_offsets():
    """Fused grouped GEMM on MXFP8 operands, x codes [2^20 + 256, 4096]
    (4.3 GB), 4 experts, intermediate 2048: out 4.3 GB."""
    from test_gpu_grouped_mx import _oracle, _run
    from ffn_gated_activation_amd.workloads import make_grouped_mx_inputs
    from grouped_compare import assert_grouped_close
    rows, experts, hidden, inter = (1 << 20) + 256, 4, 4096, 2048
    inp = make_grouped_mx_inputs(rows, experts, hidden, inter, "e4m3", device=DEV, seed=10)
    print(f"[large] grouped mx: counts {inp['counts']}", flush=True)
    out = _run(inp, 4.0, 25.0)
    torch.cuda.synchronize()
    sel = _grouped_sample(inp["offsets"], rows, [hidden, inter * 2])
    ref, mx_exp = _oracle(inp, 4.0, 25.0, rows=sel)
    ratio = assert_grouped_close("grouped mx large", out.index_select(0, torch.from_numpy(sel).to(DEV)), ref,
                                 hidden, 4.0, 25.0, mx_exp=mx_exp)
    print(f"[large] grouped mx: {len(sel)} rows, max error / bound {ratio:.3g}", flush=True)
    del inp, out
    _free()
