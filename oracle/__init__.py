"""Plain fp64 CPU oracle for the weighted SiTU-GLU (test infrastructure).

TEST INFRASTRUCTURE ONLY: the test suite, the smoke check and the CPU-baseline
leg of ``bench.py`` may import this package; the product path never does.  The
arithmetic lives in ``situ_oracle.c`` (the activation and its gradients),
``mx_oracle.c`` (MXFP8 block quantisation) and ``attn_res_oracle.c``
(attention-residual mixing), plain C in double precision with libm, sharing
nothing with the HIP library.  This module only compiles them
with gcc, loads them with ctypes and marshals numpy arrays; the one
exception is ``grouped_glu_forward`` (FC1 of routed experts followed by the
activation), whose projections are a numpy float64 matrix product per expert
feeding the C activation; ``mx_dequantize`` / ``grouped_glu_forward_mx``
decode MX block-scaled operands (the C decoder, times 2^(scale - 127) per
32-value block) before the same products.

Definitions followed (see the header of ``situ_oracle.c``):
  * Megatron-LM PR "[Dev] Add SiTU-GLU through Transformer Engine", section
    "Activation": T_g = b1*tanh(G/b1)*sigmoid(G), T_u = b2*tanh(U/b2),
    Y = T_g*T_u.
  * NeMo AutoModel "kimi_k3.situ" page, ``_situ_fwd_core`` (result
    situ(g)*up(u0)*w), ``_situ_bwd_core`` (analytic dG, dU and the optional
    routing-weight reduction), ``_WeightedSiTUFunction.forward`` (gate first,
    up second in the last axis).
  * The same Megatron-LM PR, section "Design" (routed experts run FC1 as a
    grouped GEMM; a SiTU-capable cuDNN frontend fuses that grouped GEMM with
    the scaled SiTU-GLU): the projections of every expert's rows by that
    expert's FC1 weight, then the weighted activation of them.

Row blocks can be spread over threads because every row is independent; the
per-row arithmetic and its order are the C code's, unchanged.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import threading
from concurrent.futures import ThreadPoolExecutor

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "situ_oracle.c")
_MX_SRC = os.path.join(_HERE, "mx_oracle.c")
_ARES_SRC = os.path.join(_HERE, "attn_res_oracle.c")
_LIB = os.path.join(_HERE, "libsitu_oracle.so")
_lock = threading.Lock()
_lib = None

_dp = ctypes.POINTER(ctypes.c_double)


def build(src: str = _SRC, out: str = _LIB, mx_src: str = _MX_SRC, ares_src: str = _ARES_SRC) -> str:
    """Compile the oracle with gcc (no fast-math: IEEE double semantics)."""
    tmp = out + ".tmp%d" % os.getpid()
    cmd = ["gcc", "-O2", "-fPIC", "-shared", "-std=c11", "-fno-fast-math",
           "-ffp-contract=off", "-Wall", "-Wextra", "-o", tmp, src, mx_src, ares_src, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, out)
    return out


def _bind(lib):
    i64 = ctypes.c_int64
    lib.situ_oracle_gate.restype = ctypes.c_double
    lib.situ_oracle_gate.argtypes = [ctypes.c_double, ctypes.c_double]
    lib.situ_oracle_gate_grad.restype = ctypes.c_double
    lib.situ_oracle_gate_grad.argtypes = [ctypes.c_double, ctypes.c_double]
    lib.situ_oracle_up.restype = ctypes.c_double
    lib.situ_oracle_up.argtypes = [ctypes.c_double, ctypes.c_int, ctypes.c_double]
    lib.situ_oracle_up_grad.restype = ctypes.c_double
    lib.situ_oracle_up_grad.argtypes = [ctypes.c_double, ctypes.c_int, ctypes.c_double]
    lib.situ_oracle_forward.restype = None
    lib.situ_oracle_forward.argtypes = [i64, i64, _dp, _dp, i64, ctypes.c_double,
                                        ctypes.c_int, ctypes.c_double, _dp]
    lib.situ_oracle_backward.restype = None
    lib.situ_oracle_backward.argtypes = [i64, i64, _dp, _dp, i64, ctypes.c_double,
                                         ctypes.c_int, ctypes.c_double, _dp, _dp,
                                         _dp, _dp, _dp]
    lib.situ_oracle_bf16_bits.restype = ctypes.c_uint16
    lib.situ_oracle_bf16_bits.argtypes = [ctypes.c_double]
    lib.situ_oracle_bf16_bits_array.restype = None
    lib.situ_oracle_bf16_bits_array.argtypes = [i64, _dp, ctypes.POINTER(ctypes.c_uint16)]
    lib.situ_oracle_f32_array.restype = None
    lib.situ_oracle_f32_array.argtypes = [i64, _dp, ctypes.POINTER(ctypes.c_float)]
    u8p = ctypes.POINTER(ctypes.c_uint8)
    lib.mx_oracle_fp8_decode.restype = ctypes.c_double
    lib.mx_oracle_fp8_decode.argtypes = [ctypes.c_uint8, ctypes.c_int]
    lib.mx_oracle_fp8_encode.restype = ctypes.c_uint8
    lib.mx_oracle_fp8_encode.argtypes = [ctypes.c_double, ctypes.c_int]
    lib.mx_oracle_scale_code.restype = ctypes.c_int
    lib.mx_oracle_scale_code.argtypes = [ctypes.c_double, ctypes.c_int, ctypes.c_int]
    lib.mx_oracle_quantize_block.restype = None
    lib.mx_oracle_quantize_block.argtypes = [_dp, ctypes.c_int, ctypes.c_int, ctypes.c_int, u8p, u8p]
    lib.mx_oracle_quantize_rows.restype = None
    lib.mx_oracle_quantize_rows.argtypes = [i64, i64, _dp, ctypes.c_int, ctypes.c_int, u8p, u8p]
    lib.mx_oracle_fp8_encode_array.restype = None
    lib.mx_oracle_fp8_encode_array.argtypes = [i64, _dp, ctypes.c_int, u8p]
    lib.mx_oracle_fp8_decode_array.restype = None
    lib.mx_oracle_fp8_decode_array.argtypes = [i64, u8p, ctypes.c_int, _dp]
    lib.mx_oracle_scale_code_array.restype = None
    lib.mx_oracle_scale_code_array.argtypes = [i64, _dp, ctypes.c_int, ctypes.c_int, u8p]
    lib.ares_oracle_forward.restype = None
    lib.ares_oracle_forward.argtypes = [i64, i64, ctypes.c_int, i64, _dp, _dp, _dp, _dp, ctypes.c_double,
                                        _dp, _dp, _dp, _dp, _dp]
    return lib


def load(path: str | None = None):
    """Load the compiled oracle, compiling it first only if it is not built."""
    global _lib
    if path is not None:
        return _bind(ctypes.CDLL(path))
    with _lock:
        if _lib is None:
            if not os.path.exists(_LIB):
                build()
            _lib = _bind(ctypes.CDLL(_LIB))
        return _lib


def _ptr(a: np.ndarray, ctype=ctypes.c_double):
    return a.ctypes.data_as(ctypes.POINTER(ctype))


def _as_f64(a) -> np.ndarray:
    return np.ascontiguousarray(np.asarray(a, dtype=np.float64))


def _lb_args(linear_beta):
    return (0, 0.0) if linear_beta is None else (1, float(linear_beta))


def _blocks(rows: int, threads: int):
    threads = max(1, min(int(threads), rows))
    step = -(-rows // threads)
    return [(s, min(rows, s + step)) for s in range(0, rows, step)]


def gate(g: float, beta: float = 4.0, lib=None) -> float:
    return (lib or load()).situ_oracle_gate(float(g), float(beta))


def gate_grad(g: float, beta: float = 4.0, lib=None) -> float:
    return (lib or load()).situ_oracle_gate_grad(float(g), float(beta))


def up(u: float, linear_beta=25.0, lib=None) -> float:
    has, b = _lb_args(linear_beta)
    return (lib or load()).situ_oracle_up(float(u), has, b)


def up_grad(u: float, linear_beta=25.0, lib=None) -> float:
    has, b = _lb_args(linear_beta)
    return (lib or load()).situ_oracle_up_grad(float(u), has, b)


def forward(gate_up, rw, beta: float = 4.0, linear_beta=25.0, threads: int = 1,
            lib=None) -> np.ndarray:
    """Y[rows, I] in fp64.  gate_up: [rows, 2I]; rw: [rows] or [1]."""
    lib = lib or load()
    gu = _as_f64(gate_up)
    rows, two_i = gu.shape
    inter = two_i // 2
    r = _as_f64(rw).reshape(-1)
    rw_rows = r.shape[0]
    assert rw_rows in (rows, 1), "routing weights must be per row or one scalar"
    y = np.empty((rows, inter), dtype=np.float64)
    has, b2 = _lb_args(linear_beta)

    def run(lo, hi):
        rr = r if rw_rows == 1 else r[lo:hi]
        lib.situ_oracle_forward(hi - lo, inter, _ptr(gu[lo:hi]), _ptr(rr),
                                1 if rw_rows == 1 else hi - lo, float(beta),
                                has, b2, _ptr(y[lo:hi]))

    _run_blocks(run, rows, threads)
    return y


def backward(gate_up, rw, grad_out, beta: float = 4.0, linear_beta=25.0,
             want_dr: bool = True, want_scales: bool = True, threads: int = 1,
             lib=None) -> dict:
    """Analytic backward in fp64.

    Returns a dict with ``d_gate_up`` [rows, 2I], ``dr`` ([rows], [1] or None),
    ``dr_abs`` [rows] and ``dg_scale`` [rows, I] (None unless want_scales).
    """
    lib = lib or load()
    gu = _as_f64(gate_up)
    rows, two_i = gu.shape
    inter = two_i // 2
    r = _as_f64(rw).reshape(-1)
    rw_rows = r.shape[0]
    assert rw_rows in (rows, 1), "routing weights must be per row or one scalar"
    go = _as_f64(grad_out)
    assert go.shape == (rows, inter)
    dgu = np.empty_like(gu)
    scalar = rw_rows == 1 and rows != 1
    dr_rows = np.zeros(rows, dtype=np.float64) if want_dr else None
    dr_abs = np.empty(rows, dtype=np.float64)
    dgs = np.empty((rows, inter), dtype=np.float64) if want_scales else None
    has, b2 = _lb_args(linear_beta)
    null = _dp()
    # Row sums are always taken row by row (the one broadcast weight is
    # repeated per row); for a broadcast weight they are added below in row
    # order, which is the order the C code's own broadcast mode uses.
    r_rows = np.ascontiguousarray(np.broadcast_to(r, (rows,)))

    def run(lo, hi):
        n = hi - lo
        lib.situ_oracle_backward(
            n, inter, _ptr(gu[lo:hi]), _ptr(r_rows[lo:hi]), n, float(beta),
            has, b2, _ptr(go[lo:hi]), _ptr(dgu[lo:hi]),
            _ptr(dr_rows[lo:hi]) if want_dr else null, _ptr(dr_abs[lo:hi]),
            _ptr(dgs[lo:hi]) if want_scales else null)

    _run_blocks(run, rows, threads)
    dr = None
    if want_dr:
        if scalar:
            total = 0.0
            for v in dr_rows:
                total += float(v)
            dr = np.array([total], dtype=np.float64)
        else:
            dr = dr_rows
    return {"d_gate_up": dgu, "dr": dr, "dr_abs": dr_abs, "dg_scale": dgs}


def _run_blocks(fn, rows: int, threads: int):
    if rows == 0:
        return
    blocks = _blocks(rows, threads)
    if len(blocks) == 1:
        fn(*blocks[0])
        return
    with ThreadPoolExecutor(max_workers=len(blocks)) as ex:
        list(ex.map(lambda b: fn(*b), blocks))


def round_bf16_bits(x, lib=None) -> np.ndarray:
    """fp64 -> bfloat16 bit patterns (uint16), round to nearest even."""
    lib = lib or load()
    a = _as_f64(x)
    out = np.empty(a.shape, dtype=np.uint16)
    lib.situ_oracle_bf16_bits_array(a.size, _ptr(a), _ptr(out, ctypes.c_uint16))
    return out


def round_f32(x, lib=None) -> np.ndarray:
    """fp64 -> fp32, round to nearest even."""
    lib = lib or load()
    a = _as_f64(x)
    out = np.empty(a.shape, dtype=np.float32)
    lib.situ_oracle_f32_array(a.size, _ptr(a), _ptr(out, ctypes.c_float))
    return out


# ----------------------------------------------------------------- MXFP8

FP8_FORMATS = {"e4m3": 0, "e5m2": 1}
MX_SCALE_MODES = {"floor": 0, "ceil": 1}
MX_BLOCK = 32


def _fmt(fmt) -> int:
    return FP8_FORMATS[fmt] if isinstance(fmt, str) else int(fmt)


def _mode(mode) -> int:
    return MX_SCALE_MODES[mode] if isinstance(mode, str) else int(mode)


def fp8_decode(code: int, fmt="e4m3", lib=None) -> float:
    """Value of an OFP8 code (E4M3 or E5M2)."""
    return (lib or load()).mx_oracle_fp8_decode(int(code), _fmt(fmt))


def fp8_encode(x: float, fmt="e4m3", lib=None) -> int:
    """Nearest OFP8 code, ties to even, saturating at the largest finite value."""
    return int((lib or load()).mx_oracle_fp8_encode(float(x), _fmt(fmt)))


def mx_scale_code(amax: float, fmt="e4m3", mode="floor", lib=None) -> int:
    """E8M0 scale code of a block with largest magnitude amax."""
    return int((lib or load()).mx_oracle_scale_code(float(amax), _fmt(fmt), _mode(mode)))


def mx_quantize(x, fmt="e4m3", mode="floor", threads: int = 1, lib=None):
    """Blocks of 32 along each row of x [rows, cols] (fp64): (codes uint8
    [rows, cols], scales uint8 [rows, ceil(cols / 32)])."""
    lib = lib or load()
    a = _as_f64(x)
    if a.ndim == 1:
        a = a.reshape(1, -1)
    rows, cols = a.shape
    nblk = -(-cols // MX_BLOCK)
    codes = np.empty((rows, cols), dtype=np.uint8)
    scales = np.empty((rows, nblk), dtype=np.uint8)
    u8 = ctypes.c_uint8

    def run(lo, hi):
        lib.mx_oracle_quantize_rows(hi - lo, cols, _ptr(a[lo:hi]), _fmt(fmt), _mode(mode),
                                    _ptr(codes[lo:hi], u8), _ptr(scales[lo:hi], u8))

    _run_blocks(run, rows, threads)
    return codes, scales


def fp8_encode_array(x, fmt="e4m3", lib=None) -> np.ndarray:
    """fp8_encode over an array (uint8 codes, same shape)."""
    lib = lib or load()
    a = _as_f64(x)
    out = np.empty(a.shape, dtype=np.uint8)
    lib.mx_oracle_fp8_encode_array(a.size, _ptr(a), _fmt(fmt), _ptr(out, ctypes.c_uint8))
    return out


def fp8_decode_array(codes, fmt="e4m3", lib=None) -> np.ndarray:
    """fp8_decode over an array of codes (float64, same shape)."""
    lib = lib or load()
    c = np.ascontiguousarray(np.asarray(codes, dtype=np.uint8))
    out = np.empty(c.shape, dtype=np.float64)
    lib.mx_oracle_fp8_decode_array(c.size, _ptr(c, ctypes.c_uint8), _fmt(fmt), _ptr(out))
    return out


def mx_scale_code_array(amax, fmt="e4m3", mode="floor", lib=None) -> np.ndarray:
    """mx_scale_code over an array of block maxima (uint8 codes)."""
    lib = lib or load()
    a = _as_f64(amax)
    out = np.empty(a.shape, dtype=np.uint8)
    lib.mx_oracle_scale_code_array(a.size, _ptr(a), _fmt(fmt), _mode(mode), _ptr(out, ctypes.c_uint8))
    return out


# ----------------------------------------------------------------- attention-residual mixing

ARES_MAX_BLOCKS = 64


def attn_res_forward(blocks, prefix, norm_w, proj_w, eps: float, threads: int = 1, lib=None) -> dict:
    """fp64 attention-residual mixing.

    blocks [T, m, H]; prefix [T, H] or None (values = blocks followed by the
    prefix along the block axis).  Returns out [T, H], logits / probs /
    absdot [T, NB] and scale [T, H] (see attn_res_oracle.c)."""
    lib = lib or load()
    bl = _as_f64(blocks)
    T, m, H = bl.shape
    has = prefix is not None
    pf = _as_f64(prefix).reshape(T, H) if has else np.zeros((max(T, 1), max(H, 1)))
    nb = m + (1 if has else 0)
    assert 1 <= nb <= ARES_MAX_BLOCKS
    w = _as_f64(norm_w).reshape(H)
    p = _as_f64(proj_w).reshape(H)
    out = np.empty((T, H))
    logits = np.empty((T, nb))
    probs = np.empty((T, nb))
    absdot = np.empty((T, nb))
    scale = np.empty((T, H))

    def run(lo, hi):
        lib.ares_oracle_forward(hi - lo, m, int(has), H, _ptr(bl[lo:hi]), _ptr(pf[lo:hi] if has else pf),
                                _ptr(w), _ptr(p), float(eps), _ptr(out[lo:hi]), _ptr(logits[lo:hi]),
                                _ptr(probs[lo:hi]), _ptr(absdot[lo:hi]), _ptr(scale[lo:hi]))

    _run_blocks(run, T, threads)
    return {"out": out, "logits": logits, "probs": probs, "absdot": absdot, "scale": scale}


# ----------------------------------------------------------------- grouped FC1 + SiTU-GLU

def grouped_glu_forward(x, w, m_offsets, rw, beta: float = 4.0, linear_beta=25.0, threads: int = 1,
                        want_terms: bool = True, lib=None) -> dict:
    """fp64 fused FC1 + weighted SiTU-GLU of routed experts.

    x [M, K] (rows grouped by expert: expert e owns rows m_offsets[e] ..
    m_offsets[e+1]); w [E, 2I, K] (expert e's FC1 weight, gate rows first);
    rw [M] (or one weight).  For every expert the projections are
    gate_up = x_e w_e^T (a float64 matrix product), and the output is the
    weighted SiTU-GLU of those exact projections (the C oracle's forward).

    Returns out [M, I], gate_up [M, 2I], and (want_terms) the magnitudes a
    tolerance needs: sG / sU = sum_k |x_k w_k| of every gate / up projection,
    the partial derivatives dY/dG, dY/dU of the output, and the factors
    T_g, T_g', T_u, T_u' and r of every output element."""
    lib = lib or load()
    X = _as_f64(x)
    W = _as_f64(w)
    E, two_i, K = W.shape
    inter = two_i // 2
    M = X.shape[0]
    off = [int(v) for v in m_offsets]
    assert len(off) == E + 1 and off[0] == 0 and off[-1] == M
    gu = np.zeros((M, two_i))
    s = np.zeros((M, two_i)) if want_terms else None
    for e in range(E):
        a, b = off[e], off[e + 1]
        if b > a:
            gu[a:b] = X[a:b] @ W[e].T
            if want_terms:
                s[a:b] = np.abs(X[a:b]) @ np.abs(W[e]).T
    r = _as_f64(rw).reshape(-1)
    out = forward(gu, r, beta, linear_beta, threads=threads, lib=lib)
    res = {"out": out, "gate_up": gu}
    if want_terms:
        g, u = gu[:, :inter], gu[:, inter:]
        rr = np.broadcast_to(r.reshape(-1, 1), (M, 1)) if r.size == M else np.full((M, 1), r[0])
        vg = np.vectorize(lambda v: gate(v, beta, lib=lib))
        vgp = np.vectorize(lambda v: gate_grad(v, beta, lib=lib))
        vu = np.vectorize(lambda v: up(v, linear_beta, lib=lib))
        vup = np.vectorize(lambda v: up_grad(v, linear_beta, lib=lib))
        tg, tu = vg(g), vu(u)
        tgp, tup = vgp(g), vup(u)
        res.update(sG=s[:, :inter], sU=s[:, inter:], dY_dG=rr * vgp(g) * tu, dY_dU=rr * tg * vup(u),
                   Tg=tg, Tg_prime=tgp, Tu=tu, Tu_prime=tup, r=np.broadcast_to(rr, (M, inter)))
    return res


def mx_dequantize(codes, scales, fmt="e4m3", lib=None) -> np.ndarray:
    """MX block-scaled values: x = decode(code) * 2^(scale - 127), one scale
    byte per 32 consecutive values of a row (the last block of a row may be
    shorter); scale byte 255 (the E8M0 NaN) makes its block NaN."""
    lib = lib or load()
    c = np.asarray(codes, dtype=np.uint8)
    rows, cols = c.shape
    s = np.asarray(scales, dtype=np.uint8).reshape(rows, -1)
    assert s.shape[1] == -(-cols // MX_BLOCK)
    v = fp8_decode_array(c.reshape(-1), fmt, lib=lib).reshape(rows, cols)
    e = np.repeat(s.astype(np.int64), MX_BLOCK, axis=1)[:, :cols]
    mult = np.where(e == 255, np.nan, np.ldexp(1.0, (e - 127).clip(-127, 127)))
    return v * mult


def grouped_glu_forward_mx(x_codes, x_scales, w_codes, w_scales, m_offsets, rw, fmt="e4m3", beta: float = 4.0,
                           linear_beta=25.0, threads: int = 1, want_terms: bool = True, lib=None) -> dict:
    """The fused FC1 + weighted SiTU-GLU on MX block-scaled operands: x and
    every expert's weight are decoded (mx_dequantize, scales along the hidden
    axis) and the products taken exactly (grouped_glu_forward)."""
    lib = lib or load()
    xc = np.asarray(x_codes, dtype=np.uint8)
    wc = np.asarray(w_codes, dtype=np.uint8)
    E, two_i, K = wc.shape
    x = mx_dequantize(xc, x_scales, fmt, lib=lib)
    w = mx_dequantize(wc.reshape(E * two_i, K), np.asarray(w_scales, dtype=np.uint8).reshape(E * two_i, -1), fmt,
                      lib=lib).reshape(E, two_i, K)
    return grouped_glu_forward(x, w, m_offsets, rw, beta, linear_beta, threads=threads, want_terms=want_terms,
                               lib=lib)
