"""ctypes binding of libsitu_glu.so (declared in include/situ_glu.h).

Argument marshalling only.  PyTorch is imported first so that the HIP runtime
it carries is the one the library binds to (both use the soname
libamdhip64.so.7); torch then owns every device allocation and stream.
"""
from __future__ import annotations

import ctypes
import os

import torch  # noqa: F401  (loads the process's HIP runtime before the library)

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libsitu_glu.so")

SITU_OK = 0
SITU_ERR_INVALID_ARG = 1
SITU_ERR_UNSUPPORTED = 2
SITU_ERR_DEVICE = 3
SITU_DTYPE_F32 = 0
SITU_DTYPE_BF16 = 1
SITU_FP8_E4M3 = 0
SITU_FP8_E5M2 = 1
SITU_MX_SCALE_FLOOR = 0
SITU_MX_SCALE_CEIL = 1
SITU_MX_BLOCK = 32
SITU_GROUPED_MAX_EXPERTS = 4096
SITU_GROUPED_MAX_HIDDEN = 1 << 20
SITU_GROUPED_MAX_INTERMEDIATE = 1 << 20
SITU_NOALLOC_MAX_ROWS = 262144
ABI_VERSION = 8

# every symbol include/situ_glu.h declares
EXPORTED = ("situ_glu_fwd", "situ_glu_bwd", "situ_glu_bwd_workspace_bytes",
            "situ_glu_last_error", "situ_glu_abi_version", "situ_glu_gate_window",
            "situ_glu_fwd_mxfp8", "situ_glu_mx_quantize", "situ_glu_attn_res_fwd",
            "situ_glu_grouped_fwd", "situ_glu_grouped_fwd_mxfp8",
            "situ_glu_grouped_fwd_mxfp8_workspace_bytes", "situ_glu_bwd_mxfp8", "situ_glu_split",
            "situ_glu_bwd_noalloc")


class SituGluError(RuntimeError):
    def __init__(self, code: int, message: str):
        super().__init__(f"situ_glu error {code}: {message}")
        self.code = code


_lib = None


def _bind(lib):
    vp, i64, i32, dbl = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_double
    dblp = ctypes.POINTER(ctypes.c_double)
    lib.situ_glu_fwd.restype = i32
    lib.situ_glu_fwd.argtypes = [vp, i32, i64, i64, vp, i32, i64, dbl, dblp, vp, vp]
    lib.situ_glu_bwd.restype = i32
    lib.situ_glu_bwd.argtypes = [vp, i32, i64, i64, vp, i32, i64, dbl, dblp, vp, vp, vp, vp,
                                 ctypes.c_size_t, vp]
    lib.situ_glu_bwd_noalloc.restype = i32
    lib.situ_glu_bwd_noalloc.argtypes = [vp, i32, i64, i64, vp, i32, i64, dbl, dblp, vp, vp, vp, vp]
    lib.situ_glu_bwd_workspace_bytes.restype = ctypes.c_size_t
    lib.situ_glu_bwd_workspace_bytes.argtypes = [i64, i64, i64]
    lib.situ_glu_last_error.restype = ctypes.c_char_p
    lib.situ_glu_last_error.argtypes = []
    lib.situ_glu_abi_version.restype = i32
    lib.situ_glu_abi_version.argtypes = []
    lib.situ_glu_gate_window.restype = i32
    lib.situ_glu_gate_window.argtypes = [dbl, ctypes.POINTER(ctypes.c_float)]
    lib.situ_glu_split.restype = i32
    lib.situ_glu_split.argtypes = [i32, i64, i64, i32, i32, ctypes.POINTER(ctypes.c_int64)]
    lib.situ_glu_fwd_mxfp8.restype = i32
    lib.situ_glu_fwd_mxfp8.argtypes = [vp, i32, i64, i64, vp, i32, i64, dbl, dblp, i32, i32, vp, vp, vp]
    lib.situ_glu_bwd_mxfp8.restype = i32
    lib.situ_glu_bwd_mxfp8.argtypes = [vp, i32, i64, i64, vp, i32, i64, dbl, dblp, vp, i32, i32, vp, vp, vp, vp,
                                       ctypes.c_size_t, vp]
    lib.situ_glu_mx_quantize.restype = i32
    lib.situ_glu_mx_quantize.argtypes = [vp, i32, i64, i64, i32, i32, vp, vp, vp]
    lib.situ_glu_attn_res_fwd.restype = i32
    lib.situ_glu_attn_res_fwd.argtypes = [vp, i64, i64, i64, vp, i32, vp, vp, i32, dbl, vp, i32, vp]
    lib.situ_glu_grouped_fwd.restype = i32
    lib.situ_glu_grouped_fwd.argtypes = [vp, i32, i64, i64, vp, i64, i64, vp, vp, i32, i64, dbl, dblp, vp, vp,
                                         vp]
    lib.situ_glu_grouped_fwd_mxfp8.restype = i32
    lib.situ_glu_grouped_fwd_mxfp8.argtypes = [vp, vp, i64, i64, vp, vp, i64, i64, i32, vp, vp, i32, i64, dbl,
                                                dblp, vp, vp, vp, ctypes.c_size_t, vp]
    lib.situ_glu_grouped_fwd_mxfp8_workspace_bytes.restype = ctypes.c_size_t
    lib.situ_glu_grouped_fwd_mxfp8_workspace_bytes.argtypes = [i64, i64, i64, i64]
    return lib


def load(path: str | None = None):
    """Load the built library; fail loudly if it has not been built."""
    global _lib
    if path is not None:
        return _bind(ctypes.CDLL(path))
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(
                f"{LIB_PATH} is not built; run `python -m ffn_gated_activation_amd.build` "
                "(or __graft_entry__.build()) first")
        _lib = _bind(ctypes.CDLL(LIB_PATH))
        v = _lib.situ_glu_abi_version()
        if v != ABI_VERSION:
            raise RuntimeError(f"libsitu_glu ABI version {v}, expected {ABI_VERSION}")
    return _lib


def last_error(lib=None) -> str:
    return (lib or load()).situ_glu_last_error().decode()


def check(rc: int, lib=None):
    if rc != SITU_OK:
        raise SituGluError(rc, last_error(lib))


def lb_ptr(linear_beta):
    """Host pointer to linear_beta, or NULL for None."""
    if linear_beta is None:
        return None
    return ctypes.pointer(ctypes.c_double(float(linear_beta)))
