"""GPU parity of the MXFP8 paths against the fp64 oracle.

* situ_glu_mx_quantize (exact inputs): bit-exact codes and scales, on every
  OCP E4M3 / E5M2 value, every rounding midpoint and its fp32 neighbours,
  saturation, scale-rule edges, fp32 subnormals, zeros, NaN / inf blocks and
  random rows over a wide range of magnitudes; fp32 and bf16 inputs; the
  128-bit path and the element path (ragged rows, misaligned buffers).
* situ_glu_fwd_mxfp8 (the fused forward): every scale and code within the
  window the fp32 Y's error bound allows (mx_compare.py), on the workloads'
  recipes at sizes the oracle finishes in seconds, on sampled rows at the
  full routed-expert size, and on an extreme-value grid; plus determinism.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
from compare import subnormal_allowance
from mx_compare import assert_mx_exact, assert_mx_window, y_error_bound
from ref import host_f64, sample_rows, threads

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
FORMATS = [("e4m3", "floor"), ("e4m3", "ceil"), ("e5m2", "floor"), ("e5m2", "ceil")]
MAXV = {"e4m3": 448.0, "e5m2": 57344.0}


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import ffn_gated_activation_amd  # noqa: F401


def _say(msg):
    print(msg, flush=True)


# ------------------------------------------------------------------ stand-alone quantiser

def _format_points(fmt: str) -> np.ndarray:
    """Every finite value of the format, the midpoints between neighbours and
    the fp32 numbers just above and below each (fp32 array)."""
    vals = oracle.fp8_decode_array(np.arange(256, dtype=np.uint8), fmt)
    vals = np.unique(vals[np.isfinite(vals) & (vals >= 0)])
    mids = (vals[1:] + vals[:-1]) / 2
    p = np.concatenate([vals, mids]).astype(np.float32)
    p = np.concatenate([p, np.nextafter(p, np.float32(np.inf)), np.nextafter(p, np.float32(0))])
    return np.concatenate([p, -p])


def _quant_rows(fmt: str, mode: str, seed: int) -> np.ndarray:
    """Rows of 32-value blocks (fp32) that pin the quantiser."""
    rng = np.random.default_rng(seed)
    mv = MAXV[fmt]
    pts = _format_points(fmt)
    pts = pts[np.abs(pts) <= mv]
    blocks = []
    # anchored blocks: value 0 = max_finite * 2^k fixes X = 2^k in both modes,
    # the other 31 are test points * 2^k
    for k in (-100, -20, -3, 0, 5, 60):
        order = rng.permutation(pts.size)
        for c in range(0, pts.size, 31):
            b = np.zeros(32, dtype=np.float64)
            b[0] = mv
            chunk = pts[order[c:c + 31]]
            b[1:1 + chunk.size] = chunk
            blocks.append(np.ldexp(b, k))
    # saturation (floor mode) and scale-rule edges: block maxima at 2^n,
    # just below, 1.75 * 2^n and its fp32 neighbours
    for n in (-126, -60, -1, 0, 1, 8, 9, 15, 16, 100, 127):
        for m in (1.0, np.nextafter(np.float32(1.0), np.float32(0)) * 2, 1.75,
                  float(np.nextafter(np.float32(1.75), np.float32(2))),
                  float(np.nextafter(np.float32(1.75), np.float32(0))), 1.99):
            a = np.ldexp(m, n)
            if a >= 3.4e38:
                continue
            b = rng.uniform(-1, 1, 32) * a
            b[rng.integers(32)] = a * (1 if rng.random() < 0.5 else -1)
            blocks.append(b)
    # random magnitudes, fp32 subnormals, zeros, signed zeros
    for e in rng.uniform(-140, 120, 200):
        blocks.append(rng.normal(0, 1, 32) * 2.0 ** e)
    blocks.append(np.ldexp(rng.integers(-2 ** 23, 2 ** 23, 32).astype(np.float64), -149))
    blocks.append(np.zeros(32))
    blocks.append(-np.zeros(32))
    x = np.concatenate(blocks).astype(np.float32)
    return x


def _nonfinite_block_rows() -> np.ndarray:
    b = np.ones((4, 32), dtype=np.float32)
    b[0, 3] = np.nan
    b[1, 7] = np.inf
    b[2, 31] = -np.inf
    b[3, :] = 2.0
    return b


def _run_quant(x: torch.Tensor, fmt, mode, tag):
    from ffn_gated_activation_amd import situ_glu_mx_quantize
    _say(f"[mx-quant] {tag} x={tuple(x.shape)} {x.dtype} {fmt}/{mode}")
    codes, scales = situ_glu_mx_quantize(x, fmt, mode)
    torch.cuda.synchronize()
    assert_mx_exact(tag, codes, scales, host_f64(x).reshape(-1, x.shape[-1]), fmt, mode)
    _say(f"[mx-quant] {tag} ok")


@pytest.mark.parametrize("fmt,mode", FORMATS)
@pytest.mark.parametrize("io", ["f32", "bf16"])
def test_quantize_exact_points(fmt, mode, io):
    x = _quant_rows(fmt, mode, seed=3)
    cols = 1024
    x = np.concatenate([x, np.zeros((-x.size) % cols, np.float32)]).reshape(-1, cols)
    t = torch.from_numpy(x).to(DEV)
    if io == "bf16":
        t = t.to(torch.bfloat16)
    _run_quant(t, fmt, mode, f"points {io}")


@pytest.mark.parametrize("fmt,mode", FORMATS)
def test_quantize_nonfinite_blocks(fmt, mode):
    t = torch.from_numpy(_nonfinite_block_rows()).to(DEV)
    _run_quant(t, fmt, mode, "nonfinite")


@pytest.mark.parametrize("cols", [40, 100, 1003, 2056, 32, 8])
@pytest.mark.parametrize("io", ["f32", "bf16"])
def test_quantize_ragged_rows(cols, io):
    g = torch.Generator(device="cpu").manual_seed(cols)
    x = torch.randn(37, cols, generator=g) * torch.exp2(torch.randint(-30, 30, (37, 1), generator=g).float())
    x = x.to(DEV)
    if io == "bf16":
        x = x.to(torch.bfloat16)
    for fmt, mode in FORMATS:
        _run_quant(x, fmt, mode, f"ragged cols={cols} {io}")


def test_quantize_misaligned_element_path():
    g = torch.Generator(device="cpu").manual_seed(5)
    base = torch.randn(16 * 512 + 1, generator=g).to(DEV)
    x = base[1:].view(16, 512)          # 4-byte aligned, not 16: element path
    _run_quant(x, "e4m3", "floor", "misaligned f32")
    codes_base = torch.empty(16 * 512 + 3, dtype=torch.uint8, device=DEV)
    codes = codes_base[3:].view(16, 512)  # codes not 4-byte aligned: element path
    from ffn_gated_activation_amd import situ_glu_mx_quantize
    c, s = situ_glu_mx_quantize(x, "e5m2", "ceil", codes=codes)
    torch.cuda.synchronize()
    assert_mx_exact("misaligned codes", c, s, host_f64(x), "e5m2", "ceil")


def test_quantize_empty():
    from ffn_gated_activation_amd import situ_glu_mx_quantize
    c, s = situ_glu_mx_quantize(torch.zeros(0, 64, device=DEV))
    assert c.shape == (0, 64) and s.shape == (0, 2)
    c, s = situ_glu_mx_quantize(torch.zeros(3, 0, device=DEV))
    assert c.shape == (3, 0) and s.shape == (3, 0)


# ------------------------------------------------------------------ fused forward

def _fused_check(gate_up, rw, beta, lb, fmt, mode, rows=None, tag=""):
    from ffn_gated_activation_amd import situ_glu_fwd_mxfp8
    _say(f"[mx-fwd] {tag} gate_up={tuple(gate_up.shape)} {gate_up.dtype} rw={tuple(rw.shape)} {fmt}/{mode}")
    codes, scales = situ_glu_fwd_mxfp8(gate_up, rw, beta, lb, fmt, mode)
    torch.cuda.synchronize()
    inter = gate_up.shape[-1] // 2
    gu = gate_up.reshape(-1, 2 * inter)
    r = rw.reshape(-1)
    c = codes.reshape(-1, inter)
    s = scales.reshape(gu.shape[0], -1)
    if rows is not None:
        idx = torch.as_tensor(rows, device=gu.device)
        gu, c, s = gu.index_select(0, idx), c.index_select(0, idx), s.index_select(0, idx)
        if r.numel() != 1:
            r = r.index_select(0, idx.to(r.device))
    gu64, r64 = host_f64(gu), host_f64(r)
    y64 = oracle.forward(gu64, r64, beta, lb, threads=threads())
    rel = y_error_bound(gu64, beta, lb, gate_up.dtype == torch.bfloat16)
    allow = subnormal_allowance(gu64, r64, None, beta, lb)["y"]
    st = assert_mx_window(tag, c, s, y64, rel, allow, fmt, mode)
    _say(f"[mx-fwd] {tag} ok {st}")
    assert st["unique"] >= 0.98 * st["elements"], st   # the windows stay narrow
    return codes, scales


SMALL = [
    ("routed_top8", 64, 2048),
    ("fp32_small", 256, 512),
    ("stress_sat", 48, 2048),
    ("top1_fwd", 40, 2048),
    ("dense_ffn", 6, 18432),
    ("routed_top8", 16, 40),      # a short last block
    ("routed_top8", 8, 1000),     # 128-bit path, ragged strip
    ("fp32_small", 9, 1003),      # element path
    ("routed_top8", 8, 40000),    # several strips per wavefront
    ("routed_top8", 8, 1800),     # four chunks per row, the last one partial (57 blocks)
    ("stress_sat", 3, 3848),      # two groups of four chunks per row, the last chunk partial
]


@pytest.mark.parametrize("fmt,mode", FORMATS)
@pytest.mark.parametrize("name,rows,inter", SMALL)
def test_fused_small(name, rows, inter, fmt, mode):
    from ffn_gated_activation_amd.workloads import make_inputs
    x = make_inputs(name, device=DEV, seed=11, rows=rows, inter=inter)
    _fused_check(x["gate_up"], x["routing_weights"], x["beta"], x["linear_beta"], fmt, mode,
                 tag=f"{name}[{rows}x{inter}]")


@pytest.mark.parametrize("fmt,mode", [("e4m3", "floor"), ("e5m2", "ceil")])
def test_fused_full_size_sampled(fmt, mode):
    from ffn_gated_activation_amd.workloads import make_inputs
    x = make_inputs("routed_top8", device=DEV, seed=0)
    rows = sample_rows(x["gate_up"].shape[0], k=60)
    _fused_check(x["gate_up"], x["routing_weights"], x["beta"], x["linear_beta"], fmt, mode, rows=rows,
                 tag="routed_top8 full")


def test_fused_extreme_grid():
    """Every pair from a grid of extreme G, U values (NaN, inf, huge, tiny,
    subnormal, zero), bf16 and fp32, with and without linear_beta."""
    vals = [0.0, -0.0, 1e-40, -1e-38, 1e-6, -3e-4, 0.5, -1.2187, 1.0, -2.0, 4.0, 30.0, -60.0, 100.0,
            -1e4, 3e38, -3e38, float("inf"), float("-inf"), float("nan")]
    G, U = np.meshgrid(np.array(vals), np.array(vals), indexing="ij")
    n = G.size
    inter = 64
    rows = -(-n // inter)
    g = np.zeros(rows * inter)
    u = np.zeros(rows * inter)
    g[:n], u[:n] = G.ravel(), U.ravel()
    gu = np.concatenate([g.reshape(rows, inter), u.reshape(rows, inter)], axis=1).astype(np.float32)
    for dt in (torch.float32, torch.bfloat16):
        t = torch.from_numpy(gu).to(DEV).to(dt)
        rw = torch.linspace(0.0, 2.0, rows, device=DEV).reshape(rows, 1)
        for lb in (25.0, None):
            for fmt, mode in FORMATS:
                _fused_check_lenient(t, rw, 4.0, lb, fmt, mode, tag=f"extreme {dt} lb={lb}")


def _fused_check_lenient(gate_up, rw, beta, lb, fmt, mode, tag):
    # the extreme grid holds NaN / inf blocks and elements in the subnormal
    # range: the window check applies, the uniqueness ratio does not
    from ffn_gated_activation_amd import situ_glu_fwd_mxfp8
    _say(f"[mx-fwd] {tag} {fmt}/{mode}")
    codes, scales = situ_glu_fwd_mxfp8(gate_up, rw, beta, lb, fmt, mode)
    torch.cuda.synchronize()
    gu64, r64 = host_f64(gate_up), host_f64(rw.reshape(-1))
    with np.errstate(invalid="ignore", over="ignore"):
        y64 = oracle.forward(gu64, r64, beta, lb)
    rel = y_error_bound(np.nan_to_num(gu64, nan=0.0, posinf=0.0, neginf=0.0), beta, lb,
                        gate_up.dtype == torch.bfloat16)
    with np.errstate(invalid="ignore", over="ignore"):
        allow = subnormal_allowance(np.nan_to_num(gu64, nan=0.0, posinf=3e38, neginf=-3e38), r64, None, beta,
                                    lb)["y"]
    st = assert_mx_window(tag, codes, scales, y64, rel, allow, fmt, mode)
    _say(f"[mx-fwd] {tag} ok {st}")


def test_fused_broadcast_and_bf16_weights():
    from ffn_gated_activation_amd.workloads import make_inputs
    x = make_inputs("routed_top8", device=DEV, seed=4, rows=32, inter=2048)
    _fused_check(x["gate_up"], torch.tensor([0.37], device=DEV), 4.0, 25.0, "e4m3", "floor", tag="broadcast r")
    _fused_check(x["gate_up"], x["routing_weights"].to(torch.bfloat16), 4.0, 25.0, "e4m3", "ceil",
                 tag="bf16 r")
    _fused_check(x["gate_up"], x["routing_weights"], 2.5, 10.0, "e4m3", "floor", tag="other betas")


def test_fused_misaligned_element_path():
    from ffn_gated_activation_amd.workloads import make_inputs
    x = make_inputs("routed_top8", device=DEV, seed=5, rows=16, inter=512)
    flat = torch.empty(16 * 1024 + 1, dtype=torch.bfloat16, device=DEV)
    gu = flat[1:].view(16, 1024)
    gu.copy_(x["gate_up"])
    assert gu.data_ptr() % 16 != 0
    _fused_check(gu, x["routing_weights"], 4.0, 25.0, "e4m3", "floor", tag="misaligned gate_up")


def test_fused_deterministic_and_row_independent():
    from ffn_gated_activation_amd import situ_glu_fwd_mxfp8
    from ffn_gated_activation_amd.workloads import make_inputs
    x = make_inputs("stress_sat", device=DEV, seed=2, rows=512, inter=2048)
    a = situ_glu_fwd_mxfp8(x["gate_up"], x["routing_weights"])
    b = situ_glu_fwd_mxfp8(x["gate_up"], x["routing_weights"])
    sub = situ_glu_fwd_mxfp8(x["gate_up"][100:200].contiguous(), x["routing_weights"][100:200].contiguous())
    torch.cuda.synchronize()
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])
    assert torch.equal(a[0][100:200], sub[0]) and torch.equal(a[1][100:200], sub[1])


def test_fused_empty():
    from ffn_gated_activation_amd import situ_glu_fwd_mxfp8
    c, s = situ_glu_fwd_mxfp8(torch.zeros(0, 64, device=DEV, dtype=torch.bfloat16),
                              torch.zeros(0, 1, device=DEV))
    assert c.shape == (0, 32) and s.shape == (0, 1)
