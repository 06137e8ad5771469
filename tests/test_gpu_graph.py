"""The hot path under HIP graph capture.

The library launches kernels only (no allocation, memset or
synchronisation), so a forward and a backward can be recorded once and
replayed.  Each case records both, then replays the graph several times
with new inputs written eagerly between the replays.  Every replay must
equal, bit for bit, eager calls on the same inputs.  The cases cover:
- row-aligned weights with d_routing_weights;
- one broadcast weight with its workspace and second (reduce) launch;
- fp32 io;
- the MXFP8 forward.
"""
import pytest
import torch

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import ffn_gated_activation_amd  # noqa: F401


def _bits(t):
    return t.contiguous().view(torch.uint8)


CASES = [
    # name, rows, I, dtype, broadcast weight, linear_beta, MXFP8 forward too
    ("bf16_rows_dr", 300, 1024, torch.bfloat16, False, 25.0, True),
    ("bf16_broadcast_dr", 257, 2048, torch.bfloat16, True, None, False),
    ("f32_rows_dr", 130, 520, torch.float32, False, 25.0, False),
]


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_graph_replays_match_eager(case):
    from ffn_gated_activation_amd import (situ_glu_bwd, situ_glu_bwd_workspace_bytes, situ_glu_fwd,
                                          situ_glu_fwd_mxfp8)
    name, rows, inter, dt, one, lb, mx = case
    print(f"[graph] {name}: rows {rows} I {inter} {dt} broadcast {one} lb {lb} mx {mx}", flush=True)
    gen = torch.Generator(device=DEV).manual_seed(31)
    gu = torch.empty(rows, 2 * inter, dtype=dt, device=DEV)
    rw = torch.empty(1 if one else rows, 1, dtype=torch.float32, device=DEV)
    go = torch.empty(rows, inter, dtype=dt, device=DEV)

    def fill():
        gu.copy_((2.0 * torch.randn(rows, 2 * inter, generator=gen, device=DEV)).to(dt))
        rw.copy_(torch.rand(rw.shape, generator=gen, device=DEV) + 0.25)
        go.copy_(torch.randn(rows, inter, generator=gen, device=DEV).to(dt))

    y = torch.empty(rows, inter, dtype=dt, device=DEV)
    dgu = torch.empty_like(gu)
    drw = torch.empty_like(rw)
    need = situ_glu_bwd_workspace_bytes(rows, inter, rw.shape[0])
    ws = torch.empty(max(need, 1), dtype=torch.uint8, device=DEV)
    codes = torch.empty(rows, inter, dtype=torch.uint8, device=DEV)
    scales = torch.empty(rows, (inter + 31) // 32, dtype=torch.uint8, device=DEV)

    def step():
        situ_glu_fwd(gu, rw, 4.0, lb, out=y)
        situ_glu_bwd(gu, rw, go, 4.0, lb, True, d_gate_up=dgu, d_routing_weights=drw, workspace=ws)
        if mx:
            situ_glu_fwd_mxfp8(gu, rw, 4.0, lb, codes=codes, scales=scales)

    fill()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        for _ in range(2):
            step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    for rep in range(4):
        fill()                                   # eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = [y.clone(), dgu.clone(), drw.clone()] + ([codes.clone(), scales.clone()] if mx else [])
        ref = [situ_glu_fwd(gu, rw, 4.0, lb)]
        ref += list(situ_glu_bwd(gu, rw, go, 4.0, lb, True))
        if mx:
            ref += list(situ_glu_fwd_mxfp8(gu, rw, 4.0, lb))
        torch.cuda.synchronize()
        for i, (a, b) in enumerate(zip(got, ref)):
            assert torch.equal(_bits(a), _bits(b)), f"{name}: replay {rep}, output {i} differs from eager"
    del g
