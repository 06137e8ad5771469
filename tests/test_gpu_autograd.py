"""The autograd drop-in (NeMo page "kimi_k3.situ", `_WeightedSiTUFunction`,
`_weighted_situ`): gradients through autograd equal the C ABI's backward bit
for bit, the routing-weight gradient is skipped when not needed, and a small
MoE-style FFN (FC1 -> weighted SiTU-GLU -> FC2) trains through it with
gradients of the activation matching the fp64 oracle."""
from __future__ import annotations

import numpy as np
import pytest
import torch

from compare import assert_close, assert_dr_close
from ref import oracle_results

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _bits(t):
    return t.contiguous().view(torch.int16 if t.element_size() == 2 else torch.int32)


@pytest.mark.parametrize("lb", [25.0, None])
def test_autograd_matches_c_abi(lb):
    from ffn_gated_activation_amd import situ_glu_bwd, situ_glu_fwd, weighted_situ
    gen = torch.Generator(device=DEV).manual_seed(21)
    gu = torch.randn(3, 40, 2 * 264, generator=gen, device=DEV).to(torch.bfloat16).requires_grad_()
    rw = torch.rand(3, 40, 1, generator=gen, device=DEV).requires_grad_()
    go = torch.randn(3, 40, 264, generator=gen, device=DEV).to(torch.bfloat16)
    y = weighted_situ(gu, rw, 4.0, lb)
    y.backward(go)
    y2 = situ_glu_fwd(gu.detach(), rw.detach(), 4.0, lb)
    d2, r2 = situ_glu_bwd(gu.detach(), rw.detach(), go, 4.0, lb, want_drw=True)
    torch.cuda.synchronize()
    assert torch.equal(_bits(y.detach()), _bits(y2))
    assert torch.equal(_bits(gu.grad), _bits(d2))
    assert torch.equal(_bits(rw.grad), _bits(r2))


def test_autograd_without_routing_grad_and_broadcast_weight():
    from ffn_gated_activation_amd import weighted_situ
    gen = torch.Generator(device=DEV).manual_seed(22)
    gu = torch.randn(64, 2 * 128, generator=gen, device=DEV).to(torch.bfloat16).requires_grad_()
    rw = torch.rand(64, 1, generator=gen, device=DEV)            # no grad wanted
    y = weighted_situ(gu, rw)
    y.float().sum().backward()
    assert gu.grad is not None and rw.grad is None
    one = torch.tensor([0.5], device=DEV, requires_grad=True)      # one weight for all rows
    gu2 = gu.detach().clone().requires_grad_()
    go = torch.randn(64, 128, generator=gen, device=DEV).to(torch.bfloat16)
    weighted_situ(gu2, one, 4.0, None).backward(go)
    ref = oracle_results(gu2.detach(), one.detach(), go, 4.0, None, True)
    assert_close("broadcast dG", gu2.grad[:, :128], ref["dgu"][:, :128], ref["dg_scale"])
    assert_close("broadcast dU", gu2.grad[:, 128:], ref["dgu"][:, 128:])
    assert_dr_close("broadcast dr", one.grad.reshape(1), ref["dr"], np.array([ref["dr_abs"].sum()]))


def test_other_broadcast_shapes_raise():
    from ffn_gated_activation_amd import weighted_situ
    gu = torch.zeros(4, 16, device=DEV, dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        weighted_situ(gu, torch.ones(4, 8, device=DEV))


def test_moe_ffn_trains_through_it():
    """FC1 -> weighted SiTU-GLU -> FC2 on routed rows; the activation's
    gradient seen by FC1 matches the oracle, and a few SGD steps lower the loss."""
    from ffn_gated_activation_amd import weighted_situ
    torch.manual_seed(0)
    tokens, k, hidden, inter = 64, 4, 256, 512
    fc1 = torch.nn.Linear(hidden, 2 * inter, bias=False, device=DEV, dtype=torch.bfloat16)
    fc2 = torch.nn.Linear(inter, hidden, bias=False, device=DEV, dtype=torch.bfloat16)
    x = torch.randn(tokens * k, hidden, device=DEV, dtype=torch.bfloat16)
    logits = torch.randn(tokens, k, device=DEV)
    target = torch.randn(tokens * k, hidden, device=DEV, dtype=torch.bfloat16)
    opt = torch.optim.SGD(list(fc1.parameters()) + list(fc2.parameters()), lr=0.5)
    losses = []
    for it in range(5):
        rw = torch.softmax(logits, dim=1).reshape(tokens * k, 1)
        gate_up = fc1(x)
        gate_up.retain_grad()
        h = weighted_situ(gate_up, rw)
        h.retain_grad()
        loss = torch.nn.functional.mse_loss(fc2(h).float(), target.float())
        opt.zero_grad()
        loss.backward()
        if it == 0:
            ref = oracle_results(gate_up.detach(), rw.detach(), h.grad.detach(), 4.0, 25.0, False)
            assert_close("ffn dG", gate_up.grad[:, :inter], ref["dgu"][:, :inter], ref["dg_scale"])
            assert_close("ffn dU", gate_up.grad[:, inter:], ref["dgu"][:, inter:])
        opt.step()
        losses.append(float(loss))
    assert losses[-1] < losses[0], losses
