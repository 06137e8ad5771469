"""GPU properties that hold at any size, checked bit for bit.

  * run-to-run determinism (the stress workload's "rows processed in the same
    order" requirement: identical bits on every run);
  * row independence: a launch over a subset of rows gives the same bits as
    those rows of the full launch (the NeMo page's chunked forward is
    "bitwise-identical" to the unchunked one);
  * exact scalings: Y(2r) = 2 Y(r), dG(2r) = 2 dG(r), dU(2r) = 2 dU(r),
    dr(2r) = dr(r), dr(2 go) = 2 dr(go);  oddness Y(G, -U) = -Y(G, U) when
    linear_beta is set (T_u is odd);
  * bounds: no byte outside the declared output extents changes;
  * the native library is the code that runs (no fallback path exists).
"""
from __future__ import annotations

import pytest
import torch

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _inputs(name, **kw):
    from ffn_gated_activation_amd.workloads import make_inputs
    return make_inputs(name, device=DEV, **kw)


def _bits(t):
    return t.contiguous().view(torch.int16 if t.element_size() == 2 else torch.int32)


def _run(x, gate_up=None, rw=None, go=None):
    from ffn_gated_activation_amd import situ_glu_bwd, situ_glu_fwd
    gate_up = x["gate_up"] if gate_up is None else gate_up
    rw = x["routing_weights"] if rw is None else rw
    go = x["grad_out"] if go is None else go
    y = situ_glu_fwd(gate_up, rw, x["beta"], x["linear_beta"])
    dgu, drw = situ_glu_bwd(gate_up, rw, go, x["beta"], x["linear_beta"], want_drw=True)
    torch.cuda.synchronize()
    return y, dgu, drw


@pytest.mark.parametrize("name", ["stress_sat", "routed_top8", "fp32_small"])
def test_determinism(name):
    print(f"[props] determinism {name}", flush=True)
    x = _inputs(name, seed=0)
    a = _run(x)
    b = _run(x)
    for u, v in zip(a, b):
        assert torch.equal(_bits(u), _bits(v))


def test_row_subset_bitwise():
    print("[props] row subsets", flush=True)
    x = _inputs("stress_sat", rows=4096, seed=1)
    full = _run(x)
    for lo, hi in ((0, 1), (5, 6), (17, 1000), (4000, 4096), (1, 4095)):
        sub = _run(x, gate_up=x["gate_up"][lo:hi], rw=x["routing_weights"][lo:hi], go=x["grad_out"][lo:hi])
        for f, s in zip(full, sub):
            assert torch.equal(_bits(f[lo:hi]), _bits(s)), (lo, hi)


def test_exact_scalings():
    print("[props] scalings", flush=True)
    x = _inputs("routed_top8", rows=1024, seed=2)
    y, dgu, drw = _run(x)
    y2, dgu2, drw2 = _run(x, rw=x["routing_weights"] * 2)
    assert torch.equal(_bits(y2), _bits((y.float() * 2).to(y.dtype)))
    assert torch.equal(_bits(dgu2), _bits((dgu.float() * 2).to(dgu.dtype)))
    assert torch.equal(_bits(drw2), _bits(drw))
    _, _, drw3 = _run(x, go=(x["grad_out"].float() * 2).to(x["grad_out"].dtype))
    assert torch.equal(_bits(drw3), _bits(drw * 2))
    inter = x["gate_up"].shape[1] // 2
    flipped = x["gate_up"].clone()
    flipped[:, inter:] = -flipped[:, inter:]
    yn, _, _ = _run(x, gate_up=flipped)
    assert torch.equal(_bits(yn), _bits(-y))


def test_output_bounds_canaries():
    """Outputs written through the C ABI into the middle of larger buffers."""
    import ctypes

    from ffn_gated_activation_amd import _capi
    print("[props] canaries", flush=True)
    lib = _capi.load()
    pad = 4096
    for name, rows, inter in (("routed_top8", 96, 2048), ("stress_sat", 13, 1001), ("fp32_small", 7, 36)):
        x = _inputs(name, rows=rows, inter=inter, seed=3)
        gu, rw, go = x["gate_up"], x["routing_weights"], x["grad_out"]
        dt = gu.dtype
        io = _capi.SITU_DTYPE_BF16 if dt == torch.bfloat16 else _capi.SITU_DTYPE_F32
        n_out, n_dgu = rows * inter, rows * 2 * inter
        canary = torch.full((pad + n_out + pad,), -7.0, dtype=dt, device=DEV)
        ref_c = canary.clone()
        s = torch.cuda.current_stream().cuda_stream
        lb = ctypes.pointer(ctypes.c_double(25.0))
        _capi.check(lib.situ_glu_fwd(gu.data_ptr(), io, rows, inter, rw.data_ptr(), _capi.SITU_DTYPE_F32,
                                     rows, 4.0, lb, canary[pad:].data_ptr(), s))
        d = torch.full((pad + n_dgu + pad,), 5.0, dtype=dt, device=DEV)
        ref_d = d.clone()
        dr = torch.full((pad + rows + pad,), 3.0, device=DEV)
        ref_r = dr.clone()
        _capi.check(lib.situ_glu_bwd(gu.data_ptr(), io, rows, inter, rw.data_ptr(), _capi.SITU_DTYPE_F32,
                                     rows, 4.0, lb, go.data_ptr(), d[pad:].data_ptr(), dr[pad:].data_ptr(),
                                     None, 0, s))
        torch.cuda.synchronize()
        assert torch.equal(canary[:pad], ref_c[:pad]) and torch.equal(canary[pad + n_out:], ref_c[pad + n_out:])
        assert torch.equal(d[:pad], ref_d[:pad]) and torch.equal(d[pad + n_dgu:], ref_d[pad + n_dgu:])
        assert torch.equal(dr[:pad], ref_r[:pad]) and torch.equal(dr[pad + rows:], ref_r[pad + rows:])
        # and every declared output element was written
        assert not torch.any(canary[pad:pad + n_out] == -7.0) or name == "stress_sat"


def test_native_library_is_loaded():
    from ffn_gated_activation_amd import _capi
    _capi.load()
    with open("/proc/self/maps") as f:
        maps = f.read()
    assert "libsitu_glu.so" in maps
