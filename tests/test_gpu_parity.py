"""GPU parity: the HIP kernels (through the C ABI) against the fp64 oracle.

Element by element at sizes the oracle finishes in seconds (several
wavefront tiles and ragged tails), and on sampled rows at the full workload
sizes in the same launch configuration the benchmark times.  Tolerances are
in compare.py (1 bf16 ulp; 1e-5 relative on fp32 io; 1e-4 of the row sum's
condition scale for dr).
"""
from __future__ import annotations

import math

import numpy as np
import pytest
import torch

from compare import assert_close, assert_dr_close, subnormal_allowance
from ref import host_f64, oracle_results, sample_rows

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import ffn_gated_activation_amd  # noqa: F401  (fails loudly if the library is not built)


def _say(msg):
    print(msg, flush=True)


def run_and_check(gate_up, rw, grad_out, beta, linear_beta, want_drw, rows=None, tag=""):
    """Run fwd (+bwd) on the GPU and compare the selected rows with the oracle."""
    from ffn_gated_activation_amd import situ_glu_bwd, situ_glu_fwd
    _say(f"[parity] {tag} gate_up={tuple(gate_up.shape)} {gate_up.dtype} rw={tuple(rw.shape)} "
         f"beta={beta} linear_beta={linear_beta} drw={want_drw}")
    y = situ_glu_fwd(gate_up, rw, beta, linear_beta)
    dgu = drw = None
    if grad_out is not None:
        dgu, drw = situ_glu_bwd(gate_up, rw, grad_out, beta, linear_beta, want_drw=want_drw)
    torch.cuda.synchronize()
    ref = oracle_results(gate_up, rw, grad_out, beta, linear_beta, want_drw, rows=rows,
                         backward=grad_out is not None)
    inter = gate_up.shape[-1] // 2
    sel = (lambda t: t.reshape(-1, t.shape[-1])) if rows is None else \
        (lambda t: t.reshape(-1, t.shape[-1]).index_select(0, torch.as_tensor(rows, device=t.device)))
    al = {}
    if gate_up.dtype == torch.float32:
        r64 = host_f64(rw.reshape(-1))
        if r64.size != 1 and rows is not None:
            r64 = r64[rows]
        al = subnormal_allowance(host_f64(sel(gate_up)), r64, None if grad_out is None else host_f64(sel(grad_out)),
                                 beta, linear_beta)
    stats = {"y": assert_close(f"{tag} Y", sel(y), ref["y"], allow64=al.get("y"))}
    if grad_out is not None:
        d = sel(dgu)
        stats["dG"] = assert_close(f"{tag} dG", d[:, :inter], ref["dgu"][:, :inter], ref["dg_scale"],
                                   allow64=al.get("dG"))
        stats["dU"] = assert_close(f"{tag} dU", d[:, inter:], ref["dgu"][:, inter:], allow64=al.get("dU"))
        if want_drw:
            broadcast = rw.numel() == 1 and gate_up.reshape(-1, 2 * inter).shape[0] != 1
            if broadcast:
                assert rows is None, "a broadcast dr needs every row"
                stats["dr"] = assert_dr_close(f"{tag} dr", drw.reshape(1), ref["dr"],
                                              np.array([ref["dr_abs"].sum()]),
                                              allow64=None if "dr" not in al else np.array([al["dr"].sum()]))
            else:
                g = drw.reshape(-1)
                if rows is not None:
                    g = g.index_select(0, torch.as_tensor(rows, device=g.device))
                stats["dr"] = assert_dr_close(f"{tag} dr", g, ref["dr"], ref["dr_abs"], allow64=al.get("dr"))
        else:
            assert drw is None
    _say(f"[parity] {tag} ok {stats}")
    return stats


def inputs(name, device=DEV, **kw):
    from ffn_gated_activation_amd.workloads import make_inputs
    return make_inputs(name, device=device, **kw)


# ---------------------------------------------------------------- small, element by element

SMALL = [
    # (workload, rows, inter) -- same recipes, sizes the oracle finishes in seconds
    ("fp32_small", None, None),
    ("top1_fwd", 96, None),
    ("top1_fwd", 40, 2056),      # 257 vectors per half row: a partial second unrolled pass
    ("dense_ffn", 12, None),
    ("routed_top8", 512, None),
    ("stress_sat", 256, None),
    ("stress_sat", 33, 520),     # 65 vectors per half row
    ("routed_top8", 24, 24),     # 3 vectors per half row: most lanes idle
    ("fp32_small", 37, 516),     # fp32 vector path with a ragged lane tail
    ("routed_top8", 8, 40000),   # more strips than wavefronts per row: each walks several
    ("fp32_small", 16, 4096),    # fp32 rows of several strips (LDS merge of dr)
    ("stress_sat", 5, 65536),    # the longest rows: 16 wavefronts, 8192 vectors per half
]


@pytest.mark.parametrize("name,rows,inter", SMALL, ids=[f"{n}-{r}-{i}" for n, r, i in SMALL])
def test_small_workloads(name, rows, inter):
    x = inputs(name, rows=rows, inter=inter, seed=3)
    run_and_check(x["gate_up"], x["routing_weights"], x["grad_out"], x["beta"], x["linear_beta"],
                  x["want_drw"], tag=f"{name}[{rows},{inter}]")


@pytest.mark.parametrize("linear_beta", [25.0, 3.0, 0.5])
@pytest.mark.parametrize("beta", [4.0, 2.5])
def test_up_branch_polynomial_range(beta, linear_beta):
    """bf16 io with a linear beta: a wavefront's chunk (512 values of a row)
    whose |U| all lie within linear_beta / 4 takes the polynomial
    tanh(U / linear_beta), a chunk with any |U| beyond takes the exponential
    form.  U log-uniform over 1e-40 .. the bound with random signs, plus the
    bound itself, zero, -0 and subnormals; in odd rows the first chunk also
    holds the next bf16 value above the bound (that chunk takes the
    exponential form, the second chunk the polynomial).  Every element
    against the oracle, forward and backward with the routing-weight
    gradient."""
    rows, inter = 64, 1024
    gen = torch.Generator(device="cpu").manual_seed(11)
    bound = 0.25 * linear_beta
    mag = torch.exp(torch.empty(rows, inter).uniform_(math.log(1e-40), math.log(bound), generator=gen))
    u = torch.where(torch.rand(rows, inter, generator=gen) < 0.5, -mag, mag)
    u[:, 0], u[:, 1], u[:, 2], u[:, 3], u[:, 4] = bound, -bound, 0.0, -0.0, 3e-39
    u[:, 512], u[:, 513] = bound, -bound
    above = float((np.array([bound], dtype=np.float32).view(np.uint32) + (1 << 16)).view(np.float32)[0])
    u[1::2, 5] = above
    g = 2.0 * torch.randn(rows, inter, generator=gen)
    gate_up = torch.cat([g, u], dim=1).to(torch.bfloat16)
    assert float(gate_up[:, inter:].float().abs().max()) == above
    assert float(gate_up[0, inter:].float().abs().max()) == bound
    rw = torch.rand(rows, 1, generator=gen)
    go = torch.randn(rows, inter, generator=gen).to(torch.bfloat16)
    run_and_check(gate_up.to(DEV), rw.to(DEV), go.to(DEV), beta, linear_beta, True,
                  tag=f"poly-range[b={beta},lb={linear_beta}]")


def test_dense_ffn_broadcast_dr_small():
    """One broadcast weight with its gradient (sum over every row)."""
    x = inputs("dense_ffn", rows=20, inter=1000, seed=5)
    rw = torch.tensor([0.75], device=DEV)
    run_and_check(x["gate_up"], rw, x["grad_out"], 4.0, None, True, tag="broadcast-dr")
    run_and_check(x["gate_up"], rw, x["grad_out"], 4.0, 25.0, True, tag="broadcast-dr-lb")


# ---------------------------------------------------------------- full size, sampled rows

FULL = ["fp32_small", "top1_fwd", "dense_ffn", "routed_top8", "stress_sat"]


@pytest.mark.parametrize("name", FULL)
def test_full_size_sampled(name):
    x = inputs(name, seed=0)
    n = x["gate_up"].shape[0]
    rows = None if n <= 256 else sample_rows(n, k=40)
    run_and_check(x["gate_up"], x["routing_weights"], x["grad_out"], x["beta"], x["linear_beta"],
                  x["want_drw"], rows=rows, tag=f"{name}[full]")
    del x
    torch.cuda.empty_cache()


# ---------------------------------------------------------------- edge cases

def _grid_values():
    gstar = -1.2187557268720125
    g = [0.0, -0.0, 1e-30, -1e-30, 1e-6, -1e-6, 2.0 ** -9, -(2.0 ** -9), 0.015, -0.015, 0.5, -0.5,
         1.0, -1.0, gstar, -1.21875, -1.2109375, -1.2265625, -1.25, -1.1875, 10.0, -10.0, 30.0, -30.0,
         60.0, -60.0, 88.0, -88.0, 100.0, -100.0, 150.0, -150.0, 1000.0, -1000.0, 3e38, -3e38]
    u = [0.0, 1e-6, -1e-6, 0.1, -0.1, 1.0, -1.0, 3.0, 60.0, -60.0, 1000.0, -1000.0, 1e4, -1e4]
    return g, u


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
@pytest.mark.parametrize("linear_beta", [25.0, None])
def test_extreme_value_grid(dtype, linear_beta):
    g, u = _grid_values()
    G = torch.tensor(g, dtype=torch.float64).repeat_interleave(len(u))
    U = torch.tensor(u, dtype=torch.float64).repeat(len(g))
    n = G.numel()
    inter = 8
    pad = (-n) % inter
    G = torch.cat([G, torch.zeros(pad, dtype=torch.float64)]).reshape(-1, inter)
    U = torch.cat([U, torch.zeros(pad, dtype=torch.float64)]).reshape(-1, inter)
    gate_up = torch.cat([G, U], dim=1).to(dtype).to(DEV)
    rows = gate_up.shape[0]
    gen = torch.Generator().manual_seed(2)
    go = torch.randn(rows, inter, generator=gen).to(dtype).to(DEV)
    rw = torch.rand(rows, 1, generator=gen).to(DEV)
    run_and_check(gate_up, rw, go, 4.0, linear_beta, True, tag=f"grid-{dtype}-{linear_beta}")


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_gate_minimum_neighbourhood(dtype):
    """Every representable G near the root of dT_g/dG, where its terms cancel."""
    gstar = -1.2187557268720125
    if dtype == torch.bfloat16:
        base = torch.tensor(gstar).to(torch.bfloat16).view(torch.int16).item()
        bits = torch.arange(base - 40, base + 41, dtype=torch.int16)
        G = bits.view(torch.bfloat16).to(torch.float64)
    else:
        G = torch.linspace(gstar - 0.05, gstar + 0.05, 4001, dtype=torch.float64)
        base = torch.tensor(gstar, dtype=torch.float32).view(torch.int32).item()
        G = torch.cat([G, torch.arange(base - 200, base + 201, dtype=torch.int32).view(torch.float32).double()])
    inter = 8
    pad = (-G.numel()) % inter
    G = torch.cat([G, torch.full((pad,), gstar, dtype=torch.float64)]).reshape(-1, inter)
    rows = G.shape[0]
    gen = torch.Generator().manual_seed(4)
    U = torch.randn(rows, inter, generator=gen, dtype=torch.float64) * 2
    gate_up = torch.cat([G, U], dim=1).to(dtype).to(DEV)
    go = torch.randn(rows, inter, generator=gen).to(dtype).to(DEV)
    rw = torch.rand(rows, 1, generator=gen).to(DEV)
    run_and_check(gate_up, rw, go, 4.0, 25.0, True, tag=f"root-{dtype}")


@pytest.mark.parametrize("beta,linear_beta", [(3.0, 25.0), (1.0, 7.5), (0.5, None), (100.0, 1.0),
                                              (4.0, 1.0), (2.0, 25.0)])
def test_other_betas(beta, linear_beta):
    x = inputs("routed_top8", rows=64, inter=520, seed=7)
    gu = (x["gate_up"].float() * 2).to(torch.bfloat16)
    run_and_check(gu, x["routing_weights"], x["grad_out"], beta, linear_beta, True,
                  tag=f"beta={beta},lb={linear_beta}")


@pytest.mark.parametrize("beta", [3.0, 0.5, 100.0])
def test_other_betas_root_neighbourhood(beta):
    """The root window for a beta other than 4 (built on the host by bisection
    and a Taylor series): all bf16 values near the oracle's root."""
    import oracle
    lo, hi = -60.0, -1e-3   # dT_g/dG < 0 far left, > 0 near 0
    for _ in range(200):
        mid = 0.5 * (lo + hi)
        if oracle.gate_grad(mid, beta) < 0:
            lo = mid
        else:
            hi = mid
    base = torch.tensor(lo).to(torch.bfloat16).view(torch.int16).item()
    G = torch.arange(base - 24, base + 24, dtype=torch.int16).view(torch.bfloat16).double().reshape(-1, 8)
    rows = G.shape[0]
    gen = torch.Generator().manual_seed(8)
    U = torch.randn(rows, 8, generator=gen, dtype=torch.float64)
    gate_up = torch.cat([G, U], 1).to(torch.bfloat16).to(DEV)
    go = torch.randn(rows, 8, generator=gen).to(torch.bfloat16).to(DEV)
    rw = torch.rand(rows, 1, generator=gen).to(DEV)
    run_and_check(gate_up, rw, go, beta, 25.0, True, tag=f"root-beta={beta}")


@pytest.mark.parametrize("inter", [1, 3, 7, 9, 13, 100, 1001])
@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_ragged_intermediate(inter, dtype):
    """I not a multiple of the 128-bit vector: the element path."""
    gen = torch.Generator().manual_seed(inter)
    rows = 11
    gate_up = (torch.randn(rows, 2 * inter, generator=gen) * 3).to(dtype).to(DEV)
    go = torch.randn(rows, inter, generator=gen).to(dtype).to(DEV)
    rw = torch.rand(rows, 1, generator=gen).to(DEV)
    run_and_check(gate_up, rw, go, 4.0, 25.0, True, tag=f"ragged-{inter}-{dtype}")


def test_misaligned_buffers():
    """16-byte-misaligned storage (element aligned) takes the element path."""
    gen = torch.Generator().manual_seed(12)
    rows, inter = 19, 64
    big = (torch.randn(rows * 2 * inter + 1, generator=gen) * 2).to(torch.bfloat16).to(DEV)
    gate_up = big[1:].view(rows, 2 * inter)
    assert gate_up.data_ptr() % 16 != 0
    gob = torch.randn(rows * inter + 3, generator=gen).to(torch.bfloat16).to(DEV)
    go = gob[3:].view(rows, inter)
    rw = torch.rand(rows, 1, generator=gen).to(DEV)
    run_and_check(gate_up, rw, go, 4.0, 25.0, True, tag="misaligned")


def test_leading_dims_and_single_row():
    gen = torch.Generator().manual_seed(13)
    gate_up = torch.randn(2, 3, 5, 2 * 16, generator=gen).to(torch.bfloat16).to(DEV)
    rw = torch.rand(2, 3, 5, 1, generator=gen).to(DEV)
    go = torch.randn(2, 3, 5, 16, generator=gen).to(torch.bfloat16).to(DEV)
    run_and_check(gate_up, rw, go, 4.0, 25.0, True, tag="leading-dims")
    one = torch.randn(1, 2 * 40, generator=gen).to(torch.bfloat16).to(DEV)
    run_and_check(one, torch.tensor([0.3], device=DEV), torch.randn(1, 40, generator=gen).to(torch.bfloat16).to(DEV),
                  4.0, 25.0, True, tag="one-row")


def test_routing_weight_variants():
    """bf16 routing weights (and their bf16 gradient), zero and negative weights."""
    x = inputs("routed_top8", rows=64, inter=256, seed=9)
    rw = x["routing_weights"].clone()
    rw[0] = 0.0
    rw[1] = -0.75
    rw[2] = 3.5
    run_and_check(x["gate_up"], rw, x["grad_out"], 4.0, 25.0, True, tag="rw-signs")
    run_and_check(x["gate_up"], rw.to(torch.bfloat16), x["grad_out"], 4.0, 25.0, True, tag="rw-bf16")
    rwb = torch.tensor([0.625], device=DEV, dtype=torch.bfloat16)
    run_and_check(x["gate_up"], rwb, x["grad_out"], 4.0, 25.0, True, tag="rw-bf16-broadcast")


def test_empty_inputs():
    from ffn_gated_activation_amd import situ_glu_bwd, situ_glu_fwd
    for rows, inter in ((0, 8), (5, 0), (0, 0)):
        gu = torch.empty(rows, 2 * inter, dtype=torch.bfloat16, device=DEV)
        rw = torch.rand(rows, 1, device=DEV) if rows else torch.ones(1, device=DEV)
        go = torch.empty(rows, inter, dtype=torch.bfloat16, device=DEV)
        y = situ_glu_fwd(gu, rw)
        assert y.shape == (rows, inter)
        dgu, drw = situ_glu_bwd(gu, rw, go, want_drw=True)
        torch.cuda.synchronize()
        assert dgu.shape == gu.shape
        assert torch.count_nonzero(drw).item() == 0   # an empty sum
