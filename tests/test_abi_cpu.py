"""The C-ABI library on a host without a GPU: it loads, exports every symbol
include/situ_glu.h declares, and rejects invalid arguments before any device
work (so these calls never reach the HIP runtime).  Also the host-side
root-window constants against the oracle."""
from __future__ import annotations

import ctypes
import math
import os
import re

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "situ_glu.h")


@pytest.fixture(scope="module")
def capi():
    from ffn_gated_activation_amd import _capi
    if not os.path.exists(_capi.LIB_PATH):
        from ffn_gated_activation_amd.build import build_library
        build_library()
    return _capi


@pytest.fixture(scope="module")
def lib(capi):
    return capi.load()


def _declared():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^\S[^\n(]*?\b(situ_glu_\w+)\s*\(", text, re.M)))


def test_exports_every_declared_symbol(lib, capi):
    names = _declared()
    assert set(names) == set(capi.EXPORTED), names
    for n in names:
        assert hasattr(lib, n), n
    assert lib.situ_glu_abi_version() == capi.ABI_VERSION == 8


def test_header_compiles_as_c(tmp_path):
    src = tmp_path / "t.c"
    src.write_text('#include "situ_glu.h"\nint main(void){return SITU_OK;}\n')
    import subprocess
    subprocess.run(["gcc", "-std=c99", "-Wall", "-Werror", "-I", os.path.dirname(HEADER), "-c", str(src),
                    "-o", str(tmp_path / "t.o")], check=True)


FAKE = 0x10000  # never dereferenced: every call below fails validation first


def _fwd(lib, **kw):
    a = dict(gate_up=FAKE, io=1, rows=4, inter=8, rw=FAKE + 4096, rwd=0, rw_rows=4, beta=4.0, lb=25.0,
             out=FAKE + 8192)
    a.update(kw)
    lb = None if a["lb"] is None else ctypes.pointer(ctypes.c_double(a["lb"]))
    return lib.situ_glu_fwd(a["gate_up"], a["io"], a["rows"], a["inter"], a["rw"], a["rwd"], a["rw_rows"],
                            a["beta"], lb, a["out"], None)


def _bwd(lib, **kw):
    a = dict(gate_up=FAKE, io=1, rows=4, inter=8, rw=FAKE + 4096, rwd=0, rw_rows=4, beta=4.0, lb=25.0,
             go=FAKE + 8192, dgu=FAKE + 16384, drw=FAKE + 32768, ws=None, wsb=0)
    a.update(kw)
    lb = None if a["lb"] is None else ctypes.pointer(ctypes.c_double(a["lb"]))
    return lib.situ_glu_bwd(a["gate_up"], a["io"], a["rows"], a["inter"], a["rw"], a["rwd"], a["rw_rows"],
                            a["beta"], lb, a["go"], a["dgu"], a["drw"], a["ws"], a["wsb"], None)


BAD_FWD = [
    dict(io=2), dict(io=-1), dict(rwd=7), dict(beta=0.0), dict(beta=-1.0), dict(beta=math.inf),
    dict(beta=math.nan), dict(lb=0.0), dict(lb=-3.0), dict(lb=math.inf), dict(lb=math.nan),
    dict(rows=-1), dict(inter=-2), dict(rw_rows=3), dict(rw_rows=0), dict(gate_up=None),
    dict(rw=None), dict(out=None), dict(gate_up=FAKE + 1), dict(rw=FAKE + 4098), dict(out=FAKE + 8193),
    dict(out=FAKE + 16), dict(out=FAKE + 4096 - 2),   # overlaps gate_up / routing weights
]


@pytest.mark.parametrize("kw", BAD_FWD, ids=[str(k) for k in BAD_FWD])
def test_fwd_rejects(lib, capi, kw):
    rc = _fwd(lib, **kw)
    assert rc == capi.SITU_ERR_INVALID_ARG, (kw, rc)
    assert capi.last_error(lib) != ""


BAD_BWD = [
    dict(io=3), dict(beta=-2.0), dict(lb=math.nan), dict(rw_rows=2), dict(go=None), dict(dgu=None),
    dict(dgu=FAKE + 8192 + 8),                       # overlaps grad_out
    dict(drw=FAKE + 16384 + 32),                     # overlaps d_gate_up
    dict(drw=FAKE + 4096),                           # overlaps routing weights
    dict(rw_rows=1),                                 # broadcast dr needs a workspace
    dict(rw_rows=1, ws=FAKE + 65536, wsb=8),         # too small (4 rows x 4 bytes)
    dict(rw_rows=1, ws=FAKE + 65538, wsb=64),        # misaligned workspace
    dict(drw=FAKE + 32769),                          # misaligned d_routing_weights
]


@pytest.mark.parametrize("kw", BAD_BWD, ids=[str(k) for k in BAD_BWD])
def test_bwd_rejects(lib, capi, kw):
    rc = _bwd(lib, **kw)
    assert rc == capi.SITU_ERR_INVALID_ARG, (kw, rc)
    assert capi.last_error(lib) != ""


def _bwd_noalloc(lib, **kw):
    a = dict(gate_up=FAKE, io=1, rows=4, inter=8, rw=FAKE + 4096, rwd=0, rw_rows=4, beta=4.0, lb=25.0,
             go=FAKE + 8192, dgu=FAKE + 16384, drw=FAKE + 32768)
    a.update(kw)
    lb = None if a["lb"] is None else ctypes.pointer(ctypes.c_double(a["lb"]))
    return lib.situ_glu_bwd_noalloc(a["gate_up"], a["io"], a["rows"], a["inter"], a["rw"], a["rwd"],
                                    a["rw_rows"], a["beta"], lb, a["go"], a["dgu"], a["drw"], None)


BAD_BWD_NOALLOC = [k for k in BAD_BWD if "ws" not in k and k != dict(rw_rows=1)]


@pytest.mark.parametrize("kw", BAD_BWD_NOALLOC, ids=[str(k) for k in BAD_BWD_NOALLOC])
def test_bwd_noalloc_rejects(lib, capi, kw):
    """The allocation-free backward validates its arguments as situ_glu_bwd
    does, before any device work."""
    rc = _bwd_noalloc(lib, **kw)
    assert rc == capi.SITU_ERR_INVALID_ARG, (kw, rc)
    assert capi.last_error(lib) != ""


def test_bwd_noalloc_scratch_limit(lib, capi):
    """One broadcast weight with its gradient keeps one fp32 partial per row in
    the library's scratch: more rows than SITU_NOALLOC_MAX_ROWS are
    unsupported (refused before any device work); a per-row weight needs no
    scratch at any row count."""
    big = capi.SITU_NOALLOC_MAX_ROWS + 1
    assert _bwd_noalloc(lib, rows=big, rw_rows=1) == capi.SITU_ERR_UNSUPPORTED
    assert "SITU_NOALLOC_MAX_ROWS" in capi.last_error(lib)
    # no d_routing_weights: no scratch, so validation goes on to the other checks
    assert _bwd_noalloc(lib, rows=big, rw_rows=1, drw=None, go=None) == capi.SITU_ERR_INVALID_ARG


def test_beta_is_a_double(lib, capi):
    """beta and linear_beta cross the boundary as C doubles, the type of the
    pages' Python float arguments (a deliberate widening of a C float):
    values beyond float's range are finite, positive and accepted (an empty
    call checks them and launches nothing); infinities are rejected."""
    assert _fwd(lib, rows=0, rw_rows=0, beta=1e39, lb=1e39) == capi.SITU_OK
    assert _fwd(lib, rows=0, rw_rows=0, beta=math.inf) == capi.SITU_ERR_INVALID_ARG
    out = (ctypes.c_float * 8)()
    # a beta that differs from 4 below float's resolution is a different beta (not the b1 = 4 path)
    assert lib.situ_glu_gate_window(4.0 + 1e-12, out) == capi.SITU_OK


def test_pointers_must_be_element_aligned(lib, capi):
    """Any element-aligned address is accepted (16-byte alignment selects the
    128-bit path, anything else the element path); an address that is not a
    multiple of the element size is rejected, a deliberate narrowing: no
    tensor of that dtype can start there."""
    assert _fwd(lib, gate_up=FAKE + 1) == capi.SITU_ERR_INVALID_ARG
    assert "aligned" in capi.last_error(lib)
    assert _fwd(lib, io=0, gate_up=FAKE + 2) == capi.SITU_ERR_INVALID_ARG      # fp32 at a 2-byte address
    assert _bwd(lib, go=FAKE + 8193) == capi.SITU_ERR_INVALID_ARG
    assert "aligned" in capi.last_error(lib)
    assert _bwd(lib, rw=FAKE + 4097) == capi.SITU_ERR_INVALID_ARG


def _bwd_mx(lib, **kw):
    # gate_up 4 x 2 x 40 bf16 = 640 bytes at FAKE; rw at FAKE + 4096; grad_out 320 bytes at FAKE + 8192;
    # d_codes 4 x 80 = 320 bytes at FAKE + 16384; d_scales 4 x 4 = 16 bytes at FAKE + 20480;
    # d_routing_weights at FAKE + 32768
    a = dict(gate_up=FAKE, io=1, rows=4, inter=40, rw=FAKE + 4096, rwd=0, rw_rows=4, beta=4.0, lb=25.0,
             go=FAKE + 8192, fmt=0, mode=0, codes=FAKE + 16384, scales=FAKE + 20480, drw=FAKE + 32768, ws=None,
             wsb=0)
    a.update(kw)
    lb = None if a["lb"] is None else ctypes.pointer(ctypes.c_double(a["lb"]))
    return lib.situ_glu_bwd_mxfp8(a["gate_up"], a["io"], a["rows"], a["inter"], a["rw"], a["rwd"], a["rw_rows"],
                                  a["beta"], lb, a["go"], a["fmt"], a["mode"], a["codes"], a["scales"], a["drw"],
                                  a["ws"], a["wsb"], None)


BAD_BWD_MX = [
    dict(io=3), dict(fmt=2), dict(mode=5), dict(beta=-2.0), dict(lb=math.nan), dict(rw_rows=2), dict(go=None),
    dict(codes=None), dict(scales=None),
    dict(codes=FAKE + 8192 + 16),                    # overlaps grad_out
    dict(scales=FAKE + 16384 + 300),                 # overlaps d_codes
    dict(drw=FAKE + 20480 + 8),                      # overlaps d_scales
    dict(codes=FAKE + 600),                          # overlaps gate_up
    dict(rw_rows=1),                                 # broadcast dr needs a workspace
    dict(rw_rows=1, ws=FAKE + 65536, wsb=8),         # too small (4 rows x 4 bytes)
    dict(rw_rows=1, ws=FAKE + 20480, wsb=64),        # workspace overlaps d_scales
    dict(drw=FAKE + 32769),                          # misaligned d_routing_weights
]


@pytest.mark.parametrize("kw", BAD_BWD_MX, ids=[str(k) for k in BAD_BWD_MX])
def test_bwd_mx_rejects(lib, capi, kw):
    rc = _bwd_mx(lib, **kw)
    assert rc == capi.SITU_ERR_INVALID_ARG, (kw, rc)
    assert capi.last_error(lib) != ""


def test_bwd_mx_empty_and_unsupported(lib, capi):
    assert _bwd_mx(lib, rows=0, rw_rows=0, gate_up=None, go=None, codes=None, scales=None, drw=None) == capi.SITU_OK
    assert _bwd_mx(lib, inter=0, codes=None, scales=None, drw=None) == capi.SITU_OK
    assert _bwd_mx(lib, inter=1 << 30, rows=1, rw_rows=1) == capi.SITU_ERR_UNSUPPORTED
    assert _bwd_mx(lib, rows=1 << 31, rw_rows=1) == capi.SITU_ERR_UNSUPPORTED


def _fwd_mx(lib, **kw):
    a = dict(gate_up=FAKE, io=1, rows=4, inter=40, rw=FAKE + 4096, rwd=0, rw_rows=4, beta=4.0, lb=25.0,
             fmt=0, mode=0, codes=FAKE + 8192, scales=FAKE + 16384)
    a.update(kw)
    lb = None if a["lb"] is None else ctypes.pointer(ctypes.c_double(a["lb"]))
    return lib.situ_glu_fwd_mxfp8(a["gate_up"], a["io"], a["rows"], a["inter"], a["rw"], a["rwd"],
                                  a["rw_rows"], a["beta"], lb, a["fmt"], a["mode"], a["codes"], a["scales"],
                                  None)


def _quant(lib, **kw):
    a = dict(x=FAKE, io=0, rows=4, cols=40, fmt=0, mode=0, codes=FAKE + 8192, scales=FAKE + 16384)
    a.update(kw)
    return lib.situ_glu_mx_quantize(a["x"], a["io"], a["rows"], a["cols"], a["fmt"], a["mode"], a["codes"],
                                    a["scales"], None)


# codes: 4 x 40 bytes at FAKE + 8192; scales: 4 x 2 bytes at FAKE + 16384
BAD_FWD_MX = [
    dict(io=2), dict(beta=0.0), dict(lb=-1.0), dict(rw_rows=2), dict(fmt=2), dict(fmt=-1), dict(mode=2),
    dict(codes=None), dict(scales=None), dict(gate_up=None),
    dict(codes=FAKE + 100),                          # overlaps gate_up (4 x 80 x 2 bytes)
    dict(scales=FAKE + 4096 + 2),                    # overlaps routing weights
    dict(scales=FAKE + 8192 + 150),                  # overlaps codes
]
BAD_QUANT = [
    dict(io=5), dict(fmt=3), dict(mode=-1), dict(rows=-1), dict(cols=-1), dict(x=None), dict(codes=None),
    dict(scales=None), dict(x=FAKE + 2),             # fp32 x must be 4-byte aligned
    dict(codes=FAKE + 600),                          # overlaps x (4 x 40 x 4 bytes)
    dict(scales=FAKE + 8192 + 159),                  # overlaps codes
]


@pytest.mark.parametrize("kw", BAD_FWD_MX, ids=[str(k) for k in BAD_FWD_MX])
def test_fwd_mxfp8_rejects(lib, capi, kw):
    assert _fwd_mx(lib, **kw) == capi.SITU_ERR_INVALID_ARG, kw
    assert capi.last_error(lib) != ""


@pytest.mark.parametrize("kw", BAD_QUANT, ids=[str(k) for k in BAD_QUANT])
def test_mx_quantize_rejects(lib, capi, kw):
    assert _quant(lib, **kw) == capi.SITU_ERR_INVALID_ARG, kw
    assert capi.last_error(lib) != ""


def _ares(lib, **kw):
    a = dict(blocks=FAKE, tokens=4, m=3, hidden=64, prefix=FAKE + 8192, io=1, w=FAKE + 16384, p=FAKE + 16512,
             wd=1, eps=1e-6, out=FAKE + 32768, od=1)
    a.update(kw)
    return lib.situ_glu_attn_res_fwd(a["blocks"], a["tokens"], a["m"], a["hidden"], a["prefix"], a["io"], a["w"],
                                     a["p"], a["wd"], a["eps"], a["out"], a["od"], None)


# blocks 4 x 3 x 64 x 2 = 1536 bytes at FAKE; prefix 512 bytes at FAKE + 8192;
# weights 128 bytes each; out 512 bytes at FAKE + 32768
BAD_ARES = [
    dict(io=2), dict(wd=-1), dict(od=3), dict(eps=-1e-6), dict(eps=math.nan), dict(eps=math.inf),
    dict(tokens=-1), dict(m=-1), dict(hidden=-4), dict(m=16), dict(m=0, prefix=None), dict(blocks=None),
    dict(w=None), dict(p=None), dict(out=None), dict(blocks=FAKE + 1), dict(prefix=FAKE + 8193),
    dict(w=FAKE + 16385), dict(out=FAKE + 32769, od=0),
    dict(out=FAKE + 1000),                             # overlaps blocks
    dict(out=FAKE + 8192 + 256),                       # overlaps prefix
    dict(out=FAKE + 16384 - 100),                      # overlaps norm_weight
]


@pytest.mark.parametrize("kw", BAD_ARES, ids=[str(k) for k in BAD_ARES])
def test_attn_res_rejects(lib, capi, kw):
    assert _ares(lib, **kw) == capi.SITU_ERR_INVALID_ARG, kw
    assert capi.last_error(lib) != ""


def _grouped(lib, **kw):
    lb = ctypes.c_double(25.0)
    a = dict(x=FAKE, io=1, rows=4, hidden=64, w=FAKE + 4096, experts=2, inter=128, off=FAKE + 70000,
             rw=FAKE + 70016, rwd=0, rw_rows=4, beta=4.0, lb=ctypes.byref(lb), out=FAKE + 73728,
             gu=FAKE + 81920)
    a.update(kw)
    return lib.situ_glu_grouped_fwd(a["x"], a["io"], a["rows"], a["hidden"], a["w"], a["experts"], a["inter"],
                                    a["off"], a["rw"], a["rwd"], a["rw_rows"], a["beta"], a["lb"], a["out"],
                                    a["gu"], None)


# x 4 x 64 x 2 = 512 bytes at FAKE; weight 2 x 256 x 64 x 2 = 65536 bytes at
# FAKE + 4096; offsets 12 bytes at FAKE + 70000; routing weights 16 bytes at
# FAKE + 70016; out 1024 bytes at FAKE + 73728; gate_up 2048 bytes at FAKE + 81920
BAD_GROUPED = [
    dict(rwd=3), dict(beta=0.0), dict(beta=math.nan), dict(rows=-1), dict(hidden=-64), dict(experts=-1),
    dict(experts=0), dict(rw_rows=3), dict(x=None), dict(w=None), dict(off=None), dict(rw=None), dict(out=None),
    dict(x=FAKE + 8), dict(w=FAKE + 4104), dict(out=FAKE + 73736), dict(gu=FAKE + 81928), dict(off=FAKE + 70002),
    dict(out=FAKE + 256),                              # overlaps x
    dict(gu=FAKE + 60000),                             # overlaps the weight
    dict(out=FAKE + 81920 - 512),                      # overlaps gate_up_out
    dict(out=FAKE + 70016 - 1008),                     # overlaps the offsets and routing weights
    dict(experts=4097),
]


@pytest.mark.parametrize("kw", BAD_GROUPED, ids=[str(k) for k in BAD_GROUPED])
def test_grouped_rejects(lib, capi, kw):
    assert _grouped(lib, **kw) == capi.SITU_ERR_INVALID_ARG, kw
    assert capi.last_error(lib) != ""


def test_grouped_empty_and_unsupported(lib, capi):
    assert _grouped(lib, rows=0, rw_rows=0, x=None, out=None, gu=None) == capi.SITU_OK
    assert _grouped(lib, inter=0, out=None, gu=None) == capi.SITU_OK
    assert _grouped(lib, io=0) == capi.SITU_ERR_UNSUPPORTED           # fp32 x
    assert _grouped(lib, hidden=96) == capi.SITU_ERR_UNSUPPORTED      # not a multiple of 64
    assert _grouped(lib, hidden=32) == capi.SITU_ERR_UNSUPPORTED
    assert _grouped(lib, inter=192) == capi.SITU_ERR_UNSUPPORTED      # not a multiple of 128
    assert _grouped(lib, hidden=capi.SITU_GROUPED_MAX_HIDDEN + 64) == capi.SITU_ERR_UNSUPPORTED
    assert _grouped(lib, rows=1 << 31, rw_rows=1) == capi.SITU_ERR_UNSUPPORTED
    # a launch grid beyond 2^31 - 1 workgroups
    assert _grouped(lib, rows=(1 << 31) - 1, rw_rows=1, inter=1 << 20) == capi.SITU_ERR_UNSUPPORTED


def test_grouped_python_layer_rejects():
    import torch

    from ffn_gated_activation_amd import situ_glu_grouped_fwd
    with pytest.raises(ValueError):
        situ_glu_grouped_fwd(torch.zeros(4, 64, dtype=torch.bfloat16), torch.zeros(2, 256, 64, dtype=torch.bfloat16),
                             torch.zeros(3, dtype=torch.int32), torch.ones(4))
    with pytest.raises((TypeError, ValueError)):
        situ_glu_grouped_fwd(torch.zeros(4, 64), torch.zeros(2, 256, 64), torch.zeros(3, dtype=torch.int32),
                             torch.ones(4))


def _grouped_mx(lib, **kw):
    lb = ctypes.c_double(25.0)
    a = dict(x=FAKE, xs=FAKE + 1024, rows=4, hidden=128, w=FAKE + 4096, ws=FAKE + 69632, experts=2, inter=128,
             fmt=0, off=FAKE + 71680, rw=FAKE + 71696, rwd=0, rw_rows=4, beta=4.0, lb=ctypes.byref(lb),
             out=FAKE + 73728, gu=FAKE + 81920, wk=FAKE + 86016, wkb=4096)
    a.update(kw)
    return lib.situ_glu_grouped_fwd_mxfp8(a["x"], a["xs"], a["rows"], a["hidden"], a["w"], a["ws"], a["experts"],
                                          a["inter"], a["fmt"], a["off"], a["rw"], a["rwd"], a["rw_rows"],
                                          a["beta"], a["lb"], a["out"], a["gu"], a["wk"], a["wkb"], None)


# x codes 4 x 128 bytes at FAKE; x scales 16 bytes at FAKE + 1024; weight codes
# 2 x 256 x 128 = 65536 bytes at FAKE + 4096; weight scales 2048 bytes at
# FAKE + 69632; offsets 12 bytes at FAKE + 71680; routing weights 16 bytes at
# FAKE + 71696; out 1024 bytes at FAKE + 73728; gate_up 2048 bytes at FAKE + 81920;
# workspace (needs 256 + 2304 bytes) at FAKE + 86016
BAD_GROUPED_MX = [
    dict(wk=None), dict(wkb=2559), dict(wk=FAKE + 86024),   # workspace NULL, too small, misaligned
    dict(wk=FAKE + 81920 + 1024),                            # workspace overlaps gate_up_out
    dict(wk=FAKE + 69632),                                   # workspace overlaps the weight scales
    dict(fmt=2), dict(fmt=-1), dict(rwd=3), dict(beta=0.0), dict(rows=-1), dict(experts=0), dict(rw_rows=3),
    dict(x=None), dict(xs=None), dict(w=None), dict(ws=None), dict(off=None), dict(out=None),
    dict(x=FAKE + 8), dict(w=FAKE + 4104), dict(xs=FAKE + 1026), dict(ws=FAKE + 69634), dict(out=FAKE + 73736),
    dict(out=FAKE + 70656),                            # overlaps the weight scales
    dict(gu=FAKE + 1024),                              # overlaps the x scales
    dict(out=FAKE + 81920 - 512),                      # overlaps gate_up_out
    dict(experts=4097),
]


@pytest.mark.parametrize("kw", BAD_GROUPED_MX, ids=[str(k) for k in BAD_GROUPED_MX])
def test_grouped_mx_rejects(lib, capi, kw):
    assert _grouped_mx(lib, **kw) == capi.SITU_ERR_INVALID_ARG, kw
    assert capi.last_error(lib) != ""


def test_grouped_mx_empty_and_unsupported(lib, capi):
    assert _grouped_mx(lib, rows=0, rw_rows=0, x=None, xs=None, out=None, gu=None) == capi.SITU_OK
    assert _grouped_mx(lib, inter=0, out=None, gu=None) == capi.SITU_OK
    assert _grouped_mx(lib, hidden=64) == capi.SITU_ERR_UNSUPPORTED      # not a multiple of 128
    assert _grouped_mx(lib, hidden=192) == capi.SITU_ERR_UNSUPPORTED
    assert _grouped_mx(lib, inter=192) == capi.SITU_ERR_UNSUPPORTED
    assert _grouped_mx(lib, rows=(1 << 31) - 1, rw_rows=1, inter=1 << 20) == capi.SITU_ERR_UNSUPPORTED
    # rows * hidden / 128 must stay below 2^30 (the stage-major scale offsets)
    assert _grouped_mx(lib, rows=1 << 24, rw_rows=1, hidden=128 * 64) == capi.SITU_ERR_UNSUPPORTED
    # the workspace may be NULL on an empty call
    assert _grouped_mx(lib, rows=0, rw_rows=0, x=None, xs=None, out=None, gu=None, wk=None, wkb=0) == capi.SITU_OK


def test_grouped_mx_workspace_bytes(lib, capi):
    f = lib.situ_glu_grouped_fwd_mxfp8_workspace_bytes
    # hidden / 128 slices of (R rounded up to 32, plus 32) dwords per array, each array rounded up to 256 bytes
    assert f(4, 128, 2, 128) == 256 + 2304
    assert f(65536, 7168, 16, 2048) == 2 * 56 * (65536 + 32) * 4
    assert f(0, 7168, 16, 2048) == 56 * 32 * 4 + 56 * (65536 + 32) * 4
    assert f(-1, 128, 1, 128) == 0 and f(4, 128, capi.SITU_GROUPED_MAX_EXPERTS + 1, 128) == 0


def test_grouped_mx_python_layer_rejects():
    import torch

    from ffn_gated_activation_amd import situ_glu_grouped_fwd_mxfp8
    u8 = torch.uint8
    good = dict(x_codes=torch.zeros(4, 128, dtype=u8), x_scales=torch.zeros(4, 4, dtype=u8),
                weight_codes=torch.zeros(2, 256, 128, dtype=u8), weight_scales=torch.zeros(2, 256, 4, dtype=u8),
                group_offsets=torch.zeros(3, dtype=torch.int32), routing_weights=torch.ones(4))
    for bad in (dict(x_codes=torch.zeros(4, 128)),                      # float codes
                dict(x_scales=torch.zeros(4, 4, dtype=torch.int32)),    # wrong scale dtype
                dict(x_scales=torch.zeros(4, 3, dtype=u8)),             # wrong scale shape
                dict(weight_codes=torch.zeros(2, 256, 96, dtype=u8)),   # hidden mismatch
                dict(fp8_format="e3m4")):
        with pytest.raises((TypeError, ValueError)):
            situ_glu_grouped_fwd_mxfp8(**{**good, **bad})
    with pytest.raises((TypeError, ValueError)):  # e5m2 float8 codes under the e4m3 format
        situ_glu_grouped_fwd_mxfp8(**{**good, "x_codes": torch.zeros(4, 128, dtype=torch.float8_e5m2)})


def test_attn_res_empty_and_unsupported(lib, capi):
    assert _ares(lib, tokens=0, blocks=None, prefix=None, out=None) == capi.SITU_OK
    assert _ares(lib, hidden=0, blocks=None, prefix=None, out=None) == capi.SITU_OK
    assert _ares(lib, hidden=1 << 30) == capi.SITU_ERR_UNSUPPORTED
    assert _ares(lib, tokens=1 << 31) == capi.SITU_ERR_UNSUPPORTED
    assert _ares(lib, m=15, prefix=None, tokens=0) == capi.SITU_OK


def test_mx_empty_and_unsupported(lib, capi):
    # empty calls succeed without touching any pointer
    assert _fwd_mx(lib, rows=0, rw_rows=0, codes=None, scales=None) == capi.SITU_OK
    assert _fwd_mx(lib, inter=0, codes=None, scales=None) == capi.SITU_OK
    assert _quant(lib, rows=0, x=None, codes=None, scales=None) == capi.SITU_OK
    assert _quant(lib, cols=0, x=None, codes=None, scales=None) == capi.SITU_OK
    assert _quant(lib, cols=1 << 30, rows=1) == capi.SITU_ERR_UNSUPPORTED
    assert _quant(lib, rows=1 << 31) == capi.SITU_ERR_UNSUPPORTED
    assert _fwd_mx(lib, inter=1 << 30, rows=1, rw_rows=1) == capi.SITU_ERR_UNSUPPORTED


def test_unsupported_sizes(lib, capi):
    assert _fwd(lib, inter=1 << 30, rows=1, rw_rows=1) == capi.SITU_ERR_UNSUPPORTED
    assert _fwd(lib, rows=1 << 31, rw_rows=1) == capi.SITU_ERR_UNSUPPORTED


def test_workspace_bytes(lib):
    f = lib.situ_glu_bwd_workspace_bytes
    assert f(16384, 18432, 1) == 16384 * 4
    assert f(65536, 2048, 65536) == 0
    assert f(1, 8, 1) == 0
    assert f(-1, 8, 1) == 0


def test_python_layer_rejects_cpu_tensors():
    import torch

    from ffn_gated_activation_amd import situ_glu_fwd
    with pytest.raises(ValueError):
        situ_glu_fwd(torch.zeros(2, 8), torch.ones(2, 1))


def test_tensors_of_one_call_share_a_device():
    """Every tensor of a call must sit on one GPU (the call then runs with that
    GPU current); checked on stand-ins, as the CPU has no GPU tensors."""
    from ffn_gated_activation_amd.situ_glu import _check_device

    class OnGpu:
        is_cuda = True

        def __init__(self, dev):
            self.device = dev

    _check_device(OnGpu("cuda:0"), None, OnGpu("cuda:0"))
    with pytest.raises(ValueError, match="same device"):
        _check_device(OnGpu("cuda:0"), OnGpu("cuda:1"))


def test_forward_only_entry_points_refuse_grad():
    """The entry points without a backward refuse tensors that need one
    (grad mode on, an input requiring grad) rather than returning an output
    cut off from the graph; under no_grad they go on to the device check."""
    import torch

    import ffn_gated_activation_amd as m
    gu = torch.zeros(2, 64, requires_grad=True)
    rw = torch.ones(2, 1)
    calls = [
        lambda: m.situ_glu_fwd(gu, rw),
        lambda: m.situ_glu_fwd_mxfp8(gu, rw),
        lambda: m.situ_glu_mx_quantize(gu),
        lambda: m.situ_glu_attn_res_fwd(torch.zeros(2, 3, 64), None, gu[0], torch.ones(64), 1e-6),
        lambda: m.situ_glu_grouped_fwd(torch.zeros(4, 64), torch.zeros(1, 128, 64), torch.tensor([0, 4]),
                                       torch.ones(4, 1, requires_grad=True)),
        lambda: m.situ_glu_grouped_fwd_mxfp8(None, None, None, None, torch.tensor([0, 4]),
                                             torch.ones(4, 1, requires_grad=True)),
    ]
    for call in calls:
        with pytest.raises(RuntimeError, match="has no backward"):
            call()
    with torch.no_grad():
        with pytest.raises(ValueError, match="GPU only"):
            m.situ_glu_fwd(gu, rw)
    # the differentiable form is weighted_situ (its forward runs with grad mode off inside autograd)
    with pytest.raises(ValueError, match="GPU only"):
        m.weighted_situ(gu, rw)


def _bf16_neighbours(x: float, n: int) -> np.ndarray:
    """The 2n+1 bf16 values around the bf16 value x (bit patterns +-n)."""
    b = int(np.float32(x).view(np.uint32)) >> 16
    bits = np.arange(b - n, b + n + 1, dtype=np.uint32) << 16
    return bits.view(np.float32).astype(np.float64)


def test_gate_window_constants(capi, lib):
    """The root window the kernels use agrees with the oracle: G*_f32 is the
    float nearest the oracle's root and the degree-7 polynomial (fp32 io)
    matches the oracle's dT_g/dG inside its window to 1e-6 relative
    (evaluated in double); just outside the window the two terms cancel by at
    most 20x, so that the plain fp32 difference stays well inside 1e-5 there.  bf16 io: out[6] is the bf16 value nearest the root, out[7] the
    oracle's dT_g/dG there to fp32 rounding, and at every other bf16 value
    within 64 values of it the plain formula's two terms cancel by at most a
    factor 600 (so its fp32 rounding stays ~1e-4 of a bf16 ulp)."""
    import oracle
    out = (ctypes.c_float * 12)()
    for beta in (4.0, 3.0, 1.0, 0.5, 2.0, 42.88545377783707, 100.0, 1e4):
        assert lib.situ_glu_gate_window(beta, out) == 0
        ghi, hw = float(out[0]), float(out[1])
        cs = [float(out[2 + k]) for k in range(8)]
        gsub, tsub = float(out[10]), float(out[11])
        lo, hi = -80.0, -1e-4
        for _ in range(200):
            mid = 0.5 * (lo + hi)
            if oracle.gate_grad(mid, beta) < 0:
                lo = mid
            else:
                hi = mid
        root = 0.5 * (lo + hi)
        assert abs(np.float32(root) - ghi) <= abs(np.spacing(np.float32(root))), (beta, root, ghi)
        assert 0 < hw <= 1 / 8 and hw <= abs(ghi) / 4
        c1 = cs[1]
        for d in np.linspace(-hw, hw, 41):
            g = ghi + d
            p = sum(c * d ** k for k, c in enumerate(cs))
            t = oracle.gate_grad(g, beta)
            scale = abs(c1 * (g - root)) + 1e-300
            # coefficients are rounded to fp32: allow their rounding too
            tol = 1e-6 * scale + 6e-8 * sum(abs(c * d ** k) for k, c in enumerate(cs))
            assert abs(p - t) <= tol, (beta, d, p, t)
        if beta >= 2.0:
            assert hw >= 0.1, (beta, hw)
            for g in (ghi - hw * 1.0001, ghi + hw * 1.0001):
                s = 1.0 / (1.0 + np.exp(-g))
                t1 = s / np.cosh(g / beta) ** 2
                t2 = beta * np.tanh(-g / beta) * s * (1.0 - s)
                assert (t1 + t2) / abs(t1 - t2) <= 20.0, (beta, g, (t1 + t2) / abs(t1 - t2))
        # bf16 io: the substituted value and its neighbours
        near = _bf16_neighbours(gsub, 64)
        assert np.all(np.abs(near - root) >= abs(gsub - root)), (beta, gsub, root)
        t = oracle.gate_grad(gsub, beta)
        assert abs(tsub - t) <= 2.0 ** -23 * abs(t) + 1e-45, (beta, tsub, t)
        for g in near:
            if g == gsub or g >= 0:
                continue
            # G < 0: T_g' = sigmoid sech^2(G/b) - b tanh(|G|/b) sigmoid sigmoid(-G), terms of opposite sign
            s = 1.0 / (1.0 + np.exp(-g))
            t1 = s / np.cosh(g / beta) ** 2
            t2 = beta * np.tanh(-g / beta) * s * (1.0 - s)
            assert (t1 + t2) / abs(t1 - t2) <= 600.0, (beta, g, (t1 + t2) / abs(t1 - t2))
    assert lib.situ_glu_gate_window(-1.0, out) == capi.SITU_ERR_INVALID_ARG


def test_split_covers_every_chunk(lib, capi):
    """The 128-bit path's work split (situ_glu_split): the chunk-index
    division by chunks per row is exact for every chunk index of the
    workloads' shapes and for sampled indices up to 2^31 at many other
    divisors; the flat grid covers every chunk once; the row mapping gives
    each row at most 16 wavefronts that cover its chunks, and the slot
    division is exact for every slot of a workgroup; the MXFP8 forward gives
    a wavefront a row's aligned group of four chunks where it can."""
    out = (ctypes.c_int64 * 10)()
    rng = np.random.default_rng(0)
    shapes = [(256, 512, capi.SITU_DTYPE_F32), (8192, 2048, capi.SITU_DTYPE_BF16),
              (16384, 18432, capi.SITU_DTYPE_BF16), (65536, 2048, capi.SITU_DTYPE_BF16),
              (131072, 2048, capi.SITU_DTYPE_BF16), (7, 8, capi.SITU_DTYPE_BF16), (3, 4, capi.SITU_DTYPE_F32),
              (5, 520, capi.SITU_DTYPE_BF16), (1000, 65536 + 8, capi.SITU_DTYPE_BF16),
              (2, 1 << 20, capi.SITU_DTYPE_F32), (3, (1 << 28) - 8, capi.SITU_DTYPE_BF16)]
    for rows, inter, dt in shapes:
        es = 4 if dt == capi.SITU_DTYPE_F32 else 2
        for lbg in (0, 1):
            for direction in (0, 1, 2, 3):
                assert lib.situ_glu_split(dt, rows, inter, lbg, direction, out) == 0, capi.last_error(lib)
                cpr, total, k, wpr, grid, block, magic, shift, wmagic, half = [int(v) for v in out]
                assert half == inter * es and cpr == -(-half // 1024) and total == rows * cpr
                if cpr > 1:
                    x = np.arange(total, dtype=np.uint64) if total <= 1 << 22 else \
                        rng.integers(0, total, 1 << 20, dtype=np.uint64)
                    q = (x * np.uint64(magic)) >> np.uint64(32 + shift)
                    assert np.array_equal(q, x // np.uint64(cpr)), (rows, inter, direction)
                assert 64 <= block <= 1024 and block % 64 == 0
                if direction == 3 and es == 2 and cpr % 4 == 0:
                    # a wavefront's four chunks are one aligned group of a row
                    assert k == 4 and total % 4 == 0
                if direction != 2:
                    assert wpr == 0 and block <= 256
                    waves = grid * (block // 64)
                    assert waves * k >= total and (waves - block // 64) * k < total
                else:
                    assert 1 <= wpr <= 16 and wpr * k >= cpr and (wpr - 1) * k < cpr
                    rpb = block // 64 // wpr
                    assert rpb >= 1 and rpb * wpr == block // 64
                    assert grid * rpb >= rows and (grid - 1) * rpb < rows
                    for slot in range(16):
                        assert (slot * wmagic) >> 8 == slot // wpr
    # the division at other divisors, up to the largest chunk index 2^31 - 1
    for cpr in list(range(2, 300)) + [int(v) for v in rng.integers(300, 1 << 20, 200)]:
        inter = cpr * 512
        rows = max(1, ((1 << 31) - 1) // cpr)
        assert lib.situ_glu_split(capi.SITU_DTYPE_BF16, rows, inter, 1, 0, out) == 0, capi.last_error(lib)
        magic, shift = int(out[6]), int(out[7])
        x = np.concatenate([rng.integers(0, rows * cpr, 4096, dtype=np.uint64),
                            np.array([0, cpr - 1, cpr, rows * cpr - 1], dtype=np.uint64),
                            (np.arange(1, 64, dtype=np.uint64) * np.uint64(cpr)) - np.uint64(1)])
        q = (x * np.uint64(magic)) >> np.uint64(32 + shift)
        assert np.array_equal(q, x // np.uint64(cpr)), cpr
    # rejected: element-path sizes, bad direction, too many chunks
    assert lib.situ_glu_split(capi.SITU_DTYPE_BF16, 4, 12, 1, 0, out) == capi.SITU_ERR_INVALID_ARG
    assert lib.situ_glu_split(capi.SITU_DTYPE_BF16, 4, 16, 1, 4, out) == capi.SITU_ERR_INVALID_ARG
    assert lib.situ_glu_split(7, 4, 16, 1, 0, out) == capi.SITU_ERR_INVALID_ARG
    assert lib.situ_glu_split(capi.SITU_DTYPE_BF16, 4, 16, 1, 0, None) == capi.SITU_ERR_INVALID_ARG
    assert lib.situ_glu_split(capi.SITU_DTYPE_BF16, (1 << 31) - 1, 1024, 1, 0, out) == capi.SITU_ERR_UNSUPPORTED


def test_mx_python_layer_rejects():
    import torch

    from ffn_gated_activation_amd import situ_glu_fwd_mxfp8, situ_glu_mx_quantize
    with pytest.raises(ValueError):
        situ_glu_fwd_mxfp8(torch.zeros(2, 64), torch.ones(2, 1))
    with pytest.raises(ValueError):
        situ_glu_mx_quantize(torch.zeros(2, 64))


def test_attn_res_python_layer_rejects():
    import torch

    from ffn_gated_activation_amd import situ_glu_attn_res_fwd
    with pytest.raises(ValueError):
        situ_glu_attn_res_fwd(torch.zeros(2, 3, 8), torch.zeros(2, 8), torch.ones(8), torch.ones(8), 1e-6)


def test_autograd_rejects_cpu_tensors():
    import torch

    from ffn_gated_activation_amd import weighted_situ
    with pytest.raises(ValueError):
        weighted_situ(torch.zeros(2, 8, requires_grad=True), torch.ones(2, 1))


def test_stream_probe_library_validates_before_launch():
    """The benchmark's bandwidth probe (its own library, outside the C ABI
    above): exported, and every malformed call is rejected with 1 before
    any launch; a zero-byte call launches nothing."""
    from ffn_gated_activation_amd.build import PROBE_LIB, build_probe
    if not os.path.exists(PROBE_LIB):
        build_probe()
    p = ctypes.CDLL(PROBE_LIB)
    f = p.situ_stream_probe
    f.argtypes = [ctypes.POINTER(ctypes.c_void_p), ctypes.c_int, ctypes.POINTER(ctypes.c_void_p), ctypes.c_int,
                  ctypes.c_int64, ctypes.c_void_p]
    f.restype = ctypes.c_int
    fake = 1 << 20
    ins = (ctypes.c_void_p * 4)(fake, fake + 4096, fake + 8192, fake + 12288)
    outs = (ctypes.c_void_p * 2)(fake + 16384, fake + 20480)
    assert f(ins, 2, outs, 1, 0, None) == 0
    for n_in, n_out, nbytes in ((0, 1, 16), (5, 1, 16), (2, 0, 16), (2, 3, 16), (2, 1, 8), (2, 1, -16),
                                (2, 1, (1 << 40) + 16)):
        assert f(ins, n_in, outs, n_out, nbytes, None) == 1, (n_in, n_out, nbytes)
    bad = (ctypes.c_void_p * 2)(fake + 8, fake)
    assert f(bad, 2, outs, 1, 16, None) == 1
    assert f(ins, 2, (ctypes.c_void_p * 1)(0), 1, 16, None) == 1
    assert f(None, 2, outs, 1, 16, None) == 1
