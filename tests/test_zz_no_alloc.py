"""The allocation-free backward (situ_glu_bwd_noalloc) against situ_glu_bwd.

Both are called through the C ABI (ctypes) on the same inputs; the
allocation-free one keeps the broadcast weight's per-row partials in the
library's scratch array instead of a caller workspace and runs the same
kernels, so every output must match bit for bit.  Two calls in a row, the
second on fewer rows, show that what the first call left in the scratch
array does not reach the second.  The broadcast routing-weight gradient is
also checked against the fp64 oracle at the parity bar.
"""
from __future__ import annotations

import ctypes

import pytest
import torch

import oracle
from compare import assert_dr_close
from ref import host_f64

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


@pytest.fixture(scope="module")
def lib():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from ffn_gated_activation_amd import _capi
    return _capi


def _say(msg):
    print(msg, flush=True)


def _call(capi, noalloc, gu, rw, go, lb, want):
    lib = capi.load()
    rows, two_i = gu.shape
    inter = two_i // 2
    io = capi.SITU_DTYPE_BF16 if gu.dtype == torch.bfloat16 else capi.SITU_DTYPE_F32
    dgu = torch.full_like(gu, 7.0)
    drw = torch.full_like(rw, 7.0) if want else None
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    lbp = capi.lb_ptr(lb)
    args = [gu.data_ptr(), io, rows, inter, rw.data_ptr(), capi.SITU_DTYPE_F32, rw.numel(), 4.0, lbp,
            go.data_ptr(), dgu.data_ptr(), drw.data_ptr() if want else None]
    if noalloc:
        rc = lib.situ_glu_bwd_noalloc(*args, stream)
    else:
        need = lib.situ_glu_bwd_workspace_bytes(rows, inter, rw.numel()) if want else 0
        ws = torch.empty(max(need, 1), dtype=torch.uint8, device=DEV)
        rc = lib.situ_glu_bwd(*args, ws.data_ptr() if need else None, need, stream)
    capi.check(rc, lib)
    torch.cuda.synchronize()
    return dgu, drw


CASES = [
    # (rows, inter, dtype, broadcast weight, linear beta, seed)
    (3000, 1024, torch.bfloat16, True, 25.0, 1),
    (500, 1024, torch.bfloat16, True, 25.0, 2),      # fewer rows than the call before
    (4097, 2056, torch.bfloat16, True, None, 3),     # a 16-byte last chunk per half row, no linear beta
    (64, 4096, torch.float32, True, 25.0, 4),
    (700, 512, torch.bfloat16, False, 25.0, 5),      # one weight per row: no scratch at all
]


@pytest.mark.parametrize("rows,inter,dtype,broadcast,lb,seed", CASES,
                         ids=[f"{r}x{i}-{str(d)[6:]}-{'bcast' if b else 'row'}-lb{lb}" for r, i, d, b, lb, _ in CASES])
def test_noalloc_matches_workspace_backward(lib, rows, inter, dtype, broadcast, lb, seed):
    gen = torch.Generator(device="cpu").manual_seed(seed)
    gu = (2.0 * torch.randn(rows, 2 * inter, generator=gen)).to(dtype).to(DEV)
    go = torch.randn(rows, inter, generator=gen).to(dtype).to(DEV)
    rw = (torch.tensor([0.75]) if broadcast else torch.rand(rows, 1, generator=gen)).to(DEV)
    _say(f"[noalloc] rows={rows} inter={inter} {dtype} broadcast={broadcast} lb={lb}")
    for want in (True, False):
        d0, r0 = _call(lib, False, gu, rw, go, lb, want)
        d1, r1 = _call(lib, True, gu, rw, go, lb, want)
        assert torch.equal(d0.view(torch.int16 if dtype == torch.bfloat16 else torch.int32),
                           d1.view(torch.int16 if dtype == torch.bfloat16 else torch.int32)), "d_gate_up differs"
        if want:
            assert torch.equal(r0.view(torch.int32), r1.view(torch.int32)), (r0.flatten()[:4], r1.flatten()[:4])
            if broadcast:
                ref = oracle.backward(host_f64(gu), host_f64(rw), host_f64(go), 4.0, lb, want_dr=True,
                                      want_scales=False, threads=8)
                assert_dr_close("noalloc dr", r1.reshape(1), ref["dr"], ref["dr_abs"].sum(keepdims=True))
    _say(f"[noalloc] rows={rows} ok")
