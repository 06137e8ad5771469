"""Weighted SiTU-GLU for AMD Instinct MI355X (gfx950).

Hand-written HIP kernels behind a C ABI (include/situ_glu.h, built into
libsitu_glu.so by ``python -m ffn_gated_activation_amd.build``) and a thin
ctypes binding with the same names.  PyTorch provides device memory and
streams only.
"""
from .situ_glu import (  # noqa: F401
    apply_attn_res,
    attn_res_core,
    situ_glu_abi_version,
    situ_glu_attn_res_fwd,
    situ_glu_bwd,
    situ_glu_bwd_mxfp8,
    situ_glu_bwd_workspace_bytes,
    situ_glu_fwd,
    situ_glu_fwd_mxfp8,
    situ_glu_gate_window,
    situ_glu_grouped_fwd,
    situ_glu_grouped_fwd_mxfp8,
    situ_glu_grouped_fwd_mxfp8_workspace_bytes,
    situ_glu_last_error,
    situ_glu_mx_quantize,
    situ_glu_split,
)
from ._capi import SituGluError  # noqa: F401
from .autograd import WeightedSiTUFunction, weighted_situ  # noqa: F401

__all__ = ["situ_glu_fwd", "situ_glu_bwd", "situ_glu_bwd_mxfp8", "situ_glu_bwd_workspace_bytes", "situ_glu_last_error",
           "situ_glu_abi_version", "situ_glu_gate_window", "situ_glu_fwd_mxfp8", "situ_glu_mx_quantize",
           "situ_glu_attn_res_fwd", "attn_res_core", "apply_attn_res", "situ_glu_grouped_fwd",
           "situ_glu_grouped_fwd_mxfp8",
           "situ_glu_grouped_fwd_mxfp8_workspace_bytes", "situ_glu_split", "SituGluError", "WeightedSiTUFunction", "weighted_situ"]
