"""Pins of the fp64 oracle to facts that do not come from the oracle itself.

Each ``pin_*`` function takes a loaded oracle library and raises
AssertionError when the oracle disagrees with:
  * hand-derived closed forms (tests/golden/*.txt),
  * algebraic closed forms of the whole curve for b1 = 2 and b1 = 4 in terms
    of exp(-G) / exp(-G/2), derived by hand below (not the oracle's
    tanh/sigmoid/cosh expressions),
  * Taylor series at 0 and exponential asymptotics in the tails,
  * the SiLU limit b1 -> infinity against torch's silu,
  * central finite differences of the oracle's own forward,
  * the exact linearity of Y in the routing weight,
  * bfloat16 / fp32 rounding by torch and numpy,
  * attention-residual mixing: hand-worked cases
    (tests/golden/attn_res_cases.txt), the same chain composed of torch's
    library routines (rms_norm, matmul, softmax), and its invariants,
  * MXFP8: hand-worked blocks (tests/golden/mx_blocks.txt), torch's own
    float8_e4m3fn / float8_e5m2 codecs, numpy's binary16 (whose top byte is
    E5M2), exact rational rounding with Python's fractions, and the bounds
    the scale rules imply.
The same functions run against mutated copies of the oracle
(test_oracle_mutants.py): every planted mistake must trip at least one pin.
"""
from __future__ import annotations

import math

import numpy as np

import oracle
from golden_io import attn_res_cases, closed_forms, mx_blocks, worked_cases

# tribonacci constant: real root of t^3 = t^2 + t + 1 (Cardano)
_TRIB = (1.0 + (19.0 + 3.0 * math.sqrt(33.0)) ** (1.0 / 3.0)
         + (19.0 - 3.0 * math.sqrt(33.0)) ** (1.0 / 3.0)) / 3.0


def _close(got, want, rtol, atol=0.0, what=""):
    got = float(got)
    want = float(want)
    assert math.isfinite(got), f"{what}: got {got}"
    assert abs(got - want) <= atol + rtol * abs(want), \
        f"{what}: got {got!r}, want {want!r} (diff {got - want:.3e})"


# --------------------------------------------------------------------------
# golden fixtures
# --------------------------------------------------------------------------

def pin_closed_forms(lib):
    for row in closed_forms():
        k, x, want = row["kind"], row["x"], float(row["expected"])
        lb = None if row["beta2"] == "none" else row["beta2"]
        if k == "gate":
            got = oracle.gate(x, row["beta1"], lib=lib)
        elif k == "gate_grad":
            got = oracle.gate_grad(x, row["beta1"], lib=lib)
        elif k == "up":
            got = oracle.up(x, lb, lib=lib)
        else:
            got = oracle.up_grad(x, lb, lib=lib)
        # x is the double nearest to an irrational point: allow |f'|*ulp(x)
        _close(got, want, 1e-13, 1e-14, f"{k}(b1={row['beta1']}, b2={row['beta2']}, x={row['x_text']})")


def pin_worked_rows(lib):
    for c in worked_cases():
        rows = len(c["G"])
        gate_up = np.array([c["G"][i] + c["U"][i] for i in range(rows)], dtype=np.float64)
        go = np.array(c["go"], dtype=np.float64)
        r = np.array([float(v) for v in c["r"]], dtype=np.float64)
        y = oracle.forward(gate_up, r, c["beta1"], c["beta2"], lib=lib)
        b = oracle.backward(gate_up, r, go, c["beta1"], c["beta2"], want_dr=True, want_scales=True, lib=lib)
        inter = gate_up.shape[1] // 2
        for i in range(rows):
            for j in range(inter):
                _close(y[i, j], c["Y"][i][j], 1e-12, 1e-13, f"{c['name']} Y[{i},{j}]")
                _close(b["d_gate_up"][i, j], c["dG"][i][j], 1e-12, 1e-13, f"{c['name']} dG[{i},{j}]")
                _close(b["d_gate_up"][i, inter + j], c["dU"][i][j], 1e-12, 1e-13, f"{c['name']} dU[{i},{j}]")
                # the tolerance scales the parity bars rest on (dG's term scale)
                _close(b["dg_scale"][i, j], c["dg_scale"][i][j], 1e-12, 1e-13, f"{c['name']} dg_scale[{i},{j}]")
        assert len(b["dr"]) == len(c["dr"]), c["name"]
        for i, v in enumerate(c["dr"]):
            _close(b["dr"][i], v, 1e-12, 1e-12, f"{c['name']} dr[{i}]")
        # dr's condition scale, one per row
        assert len(b["dr_abs"]) == len(c["dr_abs"]) == rows, c["name"]
        for i, v in enumerate(c["dr_abs"]):
            _close(b["dr_abs"][i], v, 1e-12, 1e-12, f"{c['name']} dr_abs[{i}]")


# --------------------------------------------------------------------------
# whole-curve algebraic closed forms (derived by hand)
# --------------------------------------------------------------------------
#
# b1 = 2, E = exp(-G):  tanh(G/2) = (1-E)/(1+E), sigmoid(G) = 1/(1+E), so
#   T_g = 2(1-E)/(1+E)^2 and, with dE/dG = -E,
#   T_g' = 2E(3-E)/(1+E)^3          (root at E = 3, i.e. G* = -ln 3).
# b1 = 4, u = exp(-G/2):  tanh(G/4) = (1-u)/(1+u), sigmoid(G) = 1/(1+u^2), so
#   T_g = 4(1-u)/((1+u)(1+u^2)) and, with du/dG = -u/2,
#   T_g' = 4u(1+u+u^2-u^3)/((1+u)^2 (1+u^2)^2)
#   (root where u^3 = u^2+u+1: u = tribonacci constant, G* = -2 ln(trib)).
# (1-E) and (1-u) are evaluated with expm1 so that the pin keeps its own
# relative accuracy near G = 0.
# b2 = 25 (any b2), v = exp(-2U/b2): T_u = b2(1-v)/(1+v), T_u' = 4v/(1+v)^2.

_GRID = np.concatenate([np.linspace(-60.0, 60.0, 241),
                        [-1.21875, -1.2187557, -1.0986123, 1e-6, -1e-6, 3e-9, 0.0]])


def _tg_b2(g):
    e = math.exp(-g)
    one_minus_e = -math.expm1(-g)      # 1 - E without cancellation near G = 0
    return (2 * one_minus_e / (1 + e) ** 2, 2 * e * (3 - e) / (1 + e) ** 3,
            2 * e * (3 + e) / (1 + e) ** 3)


def _tg_b4(g):
    u = math.exp(-g / 2)
    d = (1 + u) ** 2 * (1 + u * u) ** 2
    val = 4 * -math.expm1(-g / 2) / ((1 + u) * (1 + u * u))
    der = 4 * u * (1 + u + u * u - u ** 3) / d
    der_scale = 4 * u * (1 + u + u * u + u ** 3) / d  # same terms, all added
    return val, der, der_scale


def pin_gate_curve_b2(lib):
    for g in _GRID:
        val, der, scale = _tg_b2(float(g))
        _close(oracle.gate(g, 2.0, lib=lib), val, 1e-12, 1e-300, f"T_g(b1=2, G={g})")
        _close(oracle.gate_grad(g, 2.0, lib=lib), der, 1e-10, 1e-14 * scale, f"T_g'(b1=2, G={g})")


def pin_gate_curve_b4(lib):
    for g in _GRID:
        val, der, scale = _tg_b4(float(g))
        _close(oracle.gate(g, 4.0, lib=lib), val, 1e-12, 1e-300, f"T_g(b1=4, G={g})")
        _close(oracle.gate_grad(g, 4.0, lib=lib), der, 1e-10, 1e-14 * scale, f"T_g'(b1=4, G={g})")


def pin_gate_minimum(lib):
    gs = -2.0 * math.log(_TRIB)
    assert abs(gs - (-1.2187557268720125)) < 1e-15
    u0 = _TRIB  # exp(-G*/2)
    tmin = 4 * (1 - u0) / ((1 + u0) * (1 + u0 * u0))
    _close(oracle.gate(gs, 4.0, lib=lib), tmin, 1e-14, 0, "T_g(G*)")
    assert abs(oracle.gate_grad(gs, 4.0, lib=lib)) < 1e-15
    assert oracle.gate_grad(gs - 1e-4, 4.0, lib=lib) < 0 < oracle.gate_grad(gs + 1e-4, 4.0, lib=lib)
    # b1 = 2: root at -ln 3 with T_g = -1/4
    assert abs(oracle.gate_grad(-math.log(3.0), 2.0, lib=lib)) < 1e-15
    _close(oracle.gate(-math.log(3.0), 2.0, lib=lib), -0.25, 1e-14, 0, "T_g(b1=2, -ln3)")


def pin_up_curve(lib):
    for b2 in (25.0, 3.0):
        for uval in np.concatenate([np.linspace(-80, 80, 161), [1e-7, -2.5e-4, 0.3]]):
            v = math.exp(-2 * abs(uval) / b2)
            want = math.copysign(b2 * (1 - v) / (1 + v), uval) if uval != 0 else 0.0
            wantp = 4 * v / (1 + v) ** 2
            if abs(uval) < 1e-3:   # (1-v) cancels: use the odd Taylor series instead
                x = uval / b2
                want = b2 * (x - x ** 3 / 3 + 2 * x ** 5 / 15)
            _close(oracle.up(uval, b2, lib=lib), want, 1e-12, 1e-300, f"T_u(b2={b2}, U={uval})")
            _close(oracle.up_grad(uval, b2, lib=lib), wantp, 1e-12, 1e-300, f"T_u'(b2={b2}, U={uval})")


# --------------------------------------------------------------------------
# series, asymptotics, limits, symmetry
# --------------------------------------------------------------------------

def pin_series_at_zero(lib):
    # T_g = G/2 + G^2/4 - G^3/(6 b1^2) - G^4 (1/48 + 1/(12 b1^2)) + O(G^5)
    for b1 in (4.0, 2.0, 7.5):
        for g in (1e-2, -1e-2, 1e-3, -3e-4, 2.5e-5):
            s = g / 2 + g * g / 4 - g ** 3 / (6 * b1 * b1) - g ** 4 * (1 / 48 + 1 / (12 * b1 * b1))
            d = 0.5 + g / 2 - g * g / (2 * b1 * b1) - 4 * g ** 3 * (1 / 48 + 1 / (12 * b1 * b1))
            _close(oracle.gate(g, b1, lib=lib), s, 2e-9, 0, f"series T_g(b1={b1}, G={g})")
            _close(oracle.gate_grad(g, b1, lib=lib), d, 2e-8, 0, f"series T_g'(b1={b1}, G={g})")
    # T_u = U - U^3/(3 b2^2) + 2U^5/(15 b2^4) - 17U^7/(315 b2^6) + O(U^9),
    # T_u' = 1 - U^2/b2^2 + 2U^4/(3 b2^4) - 17U^6/(45 b2^6) + O(U^8)
    for u in (1e-2, -3e-3, 0.5):
        b2 = 25.0
        _close(oracle.up(u, b2, lib=lib), u - u ** 3 / (3 * b2 * b2) + 2 * u ** 5 / (15 * b2 ** 4)
               - 17 * u ** 7 / (315 * b2 ** 6), 1e-12, 0, f"series T_u({u})")
        _close(oracle.up_grad(u, b2, lib=lib), 1 - u * u / (b2 * b2) + 2 * u ** 4 / (3 * b2 ** 4)
               - 17 * u ** 6 / (45 * b2 ** 6),
               1e-11, 0, f"series T_u'({u})")


def pin_tails(lib):
    # b1 = 4, large |G|: T_g = 4 - 8e^{-G/2} + 4e^{-G} + O(e^{-3G/2}),
    # T_g' = 4e^{-G/2} - 4e^{-G} + O(e^{-3G/2});
    # G -> -inf: T_g = -4e^{G}(1 - 2e^{G/2} + O(e^{G})), T_g' = -4e^{G}(1 - 3e^{G/2} + O(e^{G}))
    for g in (30.0, 45.0, 60.0):
        _close(4.0 - oracle.gate(g, 4.0, lib=lib), 8 * math.exp(-g / 2) - 4 * math.exp(-g),
               3e-3, 0, f"4 - T_g({g})")
        _close(oracle.gate_grad(g, 4.0, lib=lib), 4 * math.exp(-g / 2) - 4 * math.exp(-g),
               1e-11, 0, f"T_g'({g})")
        _close(oracle.gate(-g, 4.0, lib=lib), -4 * math.exp(-g) * (1 - 2 * math.exp(-g / 2)),
               1e-11, 0, f"T_g(-{g})")
        _close(oracle.gate_grad(-g, 4.0, lib=lib), -4 * math.exp(-g) * (1 - 3 * math.exp(-g / 2)),
               1e-11, 0, f"T_g'(-{g})")
    # saturation limits
    assert oracle.gate(800.0, 4.0, lib=lib) == 4.0
    assert oracle.gate(-800.0, 4.0, lib=lib) == 0.0
    assert oracle.up(1e4, 25.0, lib=lib) == 25.0
    assert oracle.up(-1e4, 25.0, lib=lib) == -25.0


def pin_silu_limit(lib):
    import torch
    g = np.linspace(-30, 30, 121)
    silu = torch.nn.functional.silu(torch.tensor(g, dtype=torch.float64)).numpy()
    sig = torch.sigmoid(torch.tensor(g, dtype=torch.float64)).numpy()
    dsilu = sig * (1 + g * (1 - sig))   # textbook derivative of x*sigmoid(x)
    for i, x in enumerate(g):
        _close(oracle.gate(x, 1e8, lib=lib), silu[i], 1e-12, 1e-300, f"SiLU limit T_g({x})")
        _close(oracle.gate_grad(x, 1e8, lib=lib), dsilu[i], 1e-10, 1e-15, f"SiLU limit T_g'({x})")


def pin_up_symmetry_and_bounds(lib):
    rng = np.random.default_rng(1)
    for b2 in (25.0, 0.7, 300.0):
        for uval in np.concatenate([rng.normal(0, 40, 200), [0.0, 1e-30, 5e3, 1e300]]):
            a = oracle.up(uval, b2, lib=lib)
            assert oracle.up(-uval, b2, lib=lib) == -a, "T_u must be odd"
            assert abs(a) <= b2, "T_u must be bounded by b2"
            assert 0.0 <= oracle.up_grad(uval, b2, lib=lib) <= 1.0
    # linear_beta None: identity, derivative 1, bit for bit
    for uval in (0.1, -3.75, 1e-40, 7e30):
        assert oracle.up(uval, None, lib=lib) == uval
        assert oracle.up_grad(uval, None, lib=lib) == 1.0
    # b2 -> infinity approaches the identity
    _close(oracle.up(3.0, 1e9, lib=lib), 3.0, 1e-15, 0, "b2 -> inf")


# --------------------------------------------------------------------------
# gradients by finite differences of the forward
# --------------------------------------------------------------------------

def _tiny_case(seed, rows=3, inter=6):
    rng = np.random.default_rng(seed)
    g = rng.normal(0, 2, (rows, inter))
    u = rng.normal(0, 3, (rows, inter))
    special = [40.0, -40.0, -1.21875, 0.0, 1e-6, 2 * math.log(3)]
    g[0, :len(special)] = special[:inter]
    u[1, :3] = [35.0, -1e-6, 0.0]
    go = rng.normal(0, 1, (rows, inter))
    r = rng.uniform(0.1, 1.0, rows)
    return np.concatenate([g, u], axis=1), r, go


def _fd(f, x, h):
    d1 = (f(x + h) - f(x - h)) / (2 * h)
    d2 = (f(x + h / 2) - f(x - h / 2)) / h
    return (4 * d2 - d1) / 3      # Richardson: error O(h^4)


def pin_fd_gradients(lib):
    for b1, b2 in ((4.0, 25.0), (2.5, None), (4.0, None), (9.0, 3.0)):
        gu, r, go = _tiny_case(7)
        rows, two_i = gu.shape
        inter = two_i // 2
        b = oracle.backward(gu, r, go, b1, b2, want_dr=True, lib=lib)
        y0 = oracle.forward(gu, r, b1, b2, lib=lib)
        for i in range(rows):
            for j in range(two_i):
                def f(x, i=i, j=j):
                    p = gu.copy()
                    p[i, j] = x
                    return oracle.forward(p, r, b1, b2, lib=lib)[i, j % inter] * go[i, j % inter]
                x0 = gu[i, j]
                h = 1e-3 * max(1.0, abs(x0))
                fd = _fd(f, x0, h)
                an = b["d_gate_up"][i, j]
                if j < inter:
                    scale = b["dg_scale"][i, j]
                else:
                    scale = abs(an) + abs(y0[i, j - inter] * go[i, j - inter])
                assert abs(fd - an) <= 1e-7 * scale + 1e-12, \
                    f"FD b1={b1} b2={b2} [{i},{j}] x={x0}: fd={fd!r} analytic={an!r}"


def pin_dr(lib):
    gu, r, go = _tiny_case(11, rows=4, inter=5)
    for b1, b2 in ((4.0, 25.0), (3.0, None)):
        b = oracle.backward(gu, r, go, b1, b2, want_dr=True, lib=lib)
        y = oracle.forward(gu, r, b1, b2, lib=lib)
        for i in range(gu.shape[0]):
            # Y is linear in r_i, so the central difference is exact up to rounding
            def loss(ri, i=i):
                rr = r.copy()
                rr[i] = ri
                return float(np.sum(oracle.forward(gu, rr, b1, b2, lib=lib)[i] * go[i]))
            h = 0.25
            fd = (loss(r[i] + h) - loss(r[i] - h)) / (2 * h)
            scale = b["dr_abs"][i]
            _close(b["dr"][i], fd, 0, 1e-12 * scale + 1e-300, f"dr FD row {i}")
            # r_i * dr_i = sum_j go_ij * Y_ij
            _close(r[i] * b["dr"][i], float(np.sum(go[i] * y[i])), 0, 1e-12 * scale * r[i],
                   f"r*dr identity row {i}")
        # one broadcast weight: dr is the sum over rows, and the C code's own
        # broadcast mode agrees with the row-by-row path
        rs = np.array([0.37])
        bs = oracle.backward(gu, rs, go, b1, b2, want_dr=True, lib=lib)
        rowsum = oracle.backward(gu, np.full(gu.shape[0], 0.37), go, b1, b2, want_dr=True, lib=lib)["dr"]
        _close(bs["dr"][0], float(np.sum(rowsum)), 0, 1e-12 * float(np.sum(bs["dr_abs"])), "broadcast dr")
        import ctypes
        dp = ctypes.POINTER(ctypes.c_double)
        dr1 = np.zeros(1)
        dgu = np.empty_like(gu)
        guc = np.ascontiguousarray(gu)
        goc = np.ascontiguousarray(go)
        lib.situ_oracle_backward(gu.shape[0], gu.shape[1] // 2, guc.ctypes.data_as(dp),
                                 rs.ctypes.data_as(dp), 1, b1, 0 if b2 is None else 1,
                                 0.0 if b2 is None else b2, goc.ctypes.data_as(dp),
                                 dgu.ctypes.data_as(dp), dr1.ctypes.data_as(dp), dp(), dp())
        assert dr1[0] == bs["dr"][0]
        np.testing.assert_array_equal(dgu, bs["d_gate_up"])


def pin_row_independence(lib):
    gu, r, go = _tiny_case(3, rows=9, inter=4)
    y = oracle.forward(gu, r, 4.0, 25.0, lib=lib)
    y3 = oracle.forward(gu, r, 4.0, 25.0, threads=3, lib=lib)
    np.testing.assert_array_equal(y, y3)
    ys = oracle.forward(gu[2:5], r[2:5], 4.0, 25.0, lib=lib)
    np.testing.assert_array_equal(ys, y[2:5])
    b = oracle.backward(gu, r, go, 4.0, 25.0, lib=lib)
    b4 = oracle.backward(gu, r, go, 4.0, 25.0, threads=4, lib=lib)
    for k in ("d_gate_up", "dr", "dr_abs", "dg_scale"):
        np.testing.assert_array_equal(b[k], b4[k])


# --------------------------------------------------------------------------
# rounding
# --------------------------------------------------------------------------

_BF16_CASES = [
    (1.0, 0x3F80),
    (1.0 + 2.0 ** -8, 0x3F80),                 # tie, even neighbour is 1.0
    (1.0 + 3 * 2.0 ** -8, 0x3F82),             # tie, even neighbour is above
    (1.0 + 2.0 ** -8 + 2.0 ** -40, 0x3F81),    # just above the tie
    (-(1.0 + 2.0 ** -8 - 2.0 ** -40), 0xBF80), # just below the tie, negative
    (2.0 ** -133, 0x0001),                     # smallest subnormal
    (2.0 ** -134, 0x0000),                     # tie between 0 and 2^-133 -> 0
    (3 * 2.0 ** -134, 0x0002),                 # tie between 1 and 2 quanta -> 2
    (-(2.0 ** -134) * 1.0000001, 0x8001),      # above the tie, negative
    (2.0 ** -126, 0x0080),                     # smallest normal
    (2.0 ** -126 - 2.0 ** -134, 0x0080),       # tie between 0x7f and 0x80 quanta -> even (0x80)
    (3.3895313892515355e38, 0x7F7F),           # largest finite
    (255.5 * 2.0 ** 120, 0x7F80),              # halfway to 2^128: ties to even -> inf
    (255.49 * 2.0 ** 120, 0x7F7F),
    (-0.0, 0x8000),
    (0.0, 0x0000),
    (float("inf"), 0x7F80),
    (float("-inf"), 0xFF80),
    (1e-300, 0x0000),
    (-1e300, 0xFF80),
]


def pin_bf16_rounding(lib):
    for x, bits in _BF16_CASES:
        got = int(oracle.round_bf16_bits([x], lib=lib)[0])
        assert got == bits, f"bf16({x!r}) = {got:#06x}, want {bits:#06x}"
    nan = int(oracle.round_bf16_bits([float("nan")], lib=lib)[0])
    assert (nan & 0x7F80) == 0x7F80 and (nan & 0x007F) != 0
    # agreement with torch's own float32 -> bfloat16 rounding on fp32 values
    import torch
    rng = np.random.default_rng(5)
    f = np.concatenate([
        rng.normal(0, 1, 20000), rng.normal(0, 1e-38, 2000), rng.normal(0, 1e30, 2000),
        np.ldexp(rng.integers(1, 2 ** 24, 4000).astype(np.float64), -149),
    ]).astype(np.float32)
    want = torch.from_numpy(f).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    got = oracle.round_bf16_bits(f.astype(np.float64), lib=lib)
    bad = np.nonzero(got != want)[0]
    assert bad.size == 0, f"{bad.size} mismatches vs torch, first x={f[bad[0]]!r}"


def pin_f32_rounding(lib):
    rng = np.random.default_rng(9)
    x = np.concatenate([rng.normal(0, 1, 5000), rng.normal(0, 1e-40, 500), rng.normal(0, 1e38, 500)])
    np.testing.assert_array_equal(oracle.round_f32(x, lib=lib), x.astype(np.float32))


# --------------------------------------------------------------------------
# MXFP8 (OCP OFP8 element formats, OCP MX v1.0 block scales)
# --------------------------------------------------------------------------

_FP8 = {"e4m3": dict(mbits=3, bias=7, maxv=448.0, emax=8),
        "e5m2": dict(mbits=2, bias=15, maxv=57344.0, emax=15)}


def pin_mx_golden_blocks(lib):
    for b in mx_blocks():
        codes, scales = oracle.mx_quantize(np.array([b["values"]]), b["fmt"], b["mode"], lib=lib)
        assert scales[0].tolist() == b["scales"], f"{b['name']}: scales {scales[0].tolist()} != {b['scales']}"
        if b["codes"] is not None:
            got = [int(c) for c in codes[0]]
            assert got == b["codes"], f"{b['name']}: codes {[hex(c) for c in got]}"


def pin_fp8_decode_vs_torch(lib):
    import torch
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    for fmt, dt in (("e4m3", torch.float8_e4m3fn), ("e5m2", torch.float8_e5m2)):
        want = codes.view(dt).to(torch.float64).numpy()
        got = np.array([oracle.fp8_decode(c, fmt, lib=lib) for c in range(256)])
        both_nan = np.isnan(want) & np.isnan(got)
        assert np.array_equal(np.isnan(want), np.isnan(got)), f"{fmt}: NaN codes differ"
        assert np.array_equal(got[~both_nan], want[~both_nan]), f"{fmt}: decoded values differ from torch"
    # E5M2 is the upper byte of IEEE binary16
    half = (np.arange(256, dtype=np.uint16) << 8).view(np.float16).astype(np.float64)
    got = np.array([oracle.fp8_decode(c, "e5m2", lib=lib) for c in range(256)])
    fin = ~np.isnan(half)
    assert np.array_equal(np.isnan(half), np.isnan(got)) and np.array_equal(got[fin], half[fin])
    # hand facts
    assert oracle.fp8_decode(0x7E, "e4m3", lib=lib) == 448.0
    assert oracle.fp8_decode(0x01, "e4m3", lib=lib) == 2.0 ** -9
    assert oracle.fp8_decode(0x08, "e4m3", lib=lib) == 2.0 ** -6
    assert oracle.fp8_decode(0x38, "e4m3", lib=lib) == 1.0
    assert oracle.fp8_decode(0x7B, "e5m2", lib=lib) == 57344.0
    assert oracle.fp8_decode(0x01, "e5m2", lib=lib) == 2.0 ** -16


def _fp8_points(fmt):
    """fp32-exact test points: every finite value, every midpoint between
    neighbours, their fp32 neighbours, and random fp32 values."""
    p = _FP8[fmt]
    vals = sorted({oracle.fp8_decode(c, fmt) for c in range(256)} - {float("nan")})
    vals = [v for v in vals if math.isfinite(v) and v >= 0]
    mids = [(a + b) / 2 for a, b in zip(vals, vals[1:])]
    pts = np.array(vals + mids, dtype=np.float32)
    near = np.concatenate([np.nextafter(pts, np.float32(np.inf)), np.nextafter(pts, np.float32(0))])
    rng = np.random.default_rng(17)
    rnd = np.exp(rng.uniform(np.log(2.0 ** -(p["bias"] + p["mbits"] + 2)), np.log(p["maxv"]), 20000))
    allp = np.concatenate([pts, near, rnd.astype(np.float32)])
    return np.concatenate([allp, -allp]).astype(np.float32)


def pin_fp8_encode_vs_torch(lib):
    import torch
    for fmt, dt in (("e4m3", torch.float8_e4m3fn), ("e5m2", torch.float8_e5m2)):
        x = _fp8_points(fmt)
        # torch does not saturate: compare below the last rounding midpoint
        lim = _FP8[fmt]["maxv"] * (1 + 2.0 ** -(_FP8[fmt]["mbits"] + 1))
        x = x[np.abs(x) < lim]
        want = torch.from_numpy(x).to(dt).view(torch.uint8).numpy()
        got = np.array([oracle.fp8_encode(float(v), fmt, lib=lib) for v in x], dtype=np.uint8)
        bad = np.nonzero(got != want)[0]
        assert bad.size == 0, f"{fmt}: {bad.size} codes differ from torch, first x={x[bad[0]]!r}"


def pin_fp8_encode_exact_rational(lib):
    """Round to nearest, ties to even, by exact rational arithmetic: the
    quantum of |x| is 2^(max(floor(log2|x|), 1 - bias) - mbits); Python's
    round() of a Fraction rounds half to even."""
    from fractions import Fraction
    rng = np.random.default_rng(23)
    for fmt, p in _FP8.items():
        xs = list(_fp8_points(fmt)[::7]) + list(rng.normal(0, 3, 500))
        for x in xs:
            x = float(x)
            a = Fraction(abs(x))
            if a == 0:
                want = 0.0
            else:
                e = max(math.floor(math.log2(a)), 1 - p["bias"])
                # log2 of a Fraction near a power of two: settle the binade exactly
                while a < Fraction(2) ** e and e > 1 - p["bias"]:
                    e -= 1
                while a >= Fraction(2) ** (e + 1):
                    e += 1
                q = Fraction(2) ** (e - p["mbits"])
                want = float(min(round(a / q) * q, Fraction(p["maxv"])))
            got = oracle.fp8_decode(oracle.fp8_encode(x, fmt, lib=lib), fmt, lib=lib)
            assert abs(got) == want, f"{fmt}: encode({x!r}) decodes to {got!r}, want {want!r}"
            assert got == 0 or math.copysign(1, got) == math.copysign(1, x), f"{fmt}: sign of {x!r}"


def pin_fp8_encode_saturates(lib):
    for fmt, p in _FP8.items():
        mx = oracle.fp8_encode(p["maxv"], fmt, lib=lib)
        for x in (p["maxv"] * 1.01, p["maxv"] * 2, 1e30, float("inf")):
            assert oracle.fp8_encode(x, fmt, lib=lib) == mx, f"{fmt}: {x} must clamp to the largest value"
            assert oracle.fp8_encode(-x, fmt, lib=lib) == mx | 0x80
        assert oracle.fp8_decode(mx, fmt, lib=lib) == p["maxv"]


def pin_mx_scale_rules(lib):
    """floor: amax / X in [2^emax, 2^(emax+1)); ceil: amax / X in
    (maxv / 2, maxv]; both clamped to the E8M0 range; hand values."""
    hand = [("e4m3", "floor", 448.0, 127), ("e4m3", "floor", 1.0, 119), ("e4m3", "floor", 0.75, 118),
            ("e4m3", "floor", 500.0, 127), ("e4m3", "floor", 512.0, 128), ("e4m3", "ceil", 448.0, 127),
            ("e4m3", "ceil", 448.00001, 128), ("e4m3", "ceil", 1.0, 119), ("e4m3", "ceil", 1.75, 119),
            ("e4m3", "ceil", 1.7500001, 120), ("e5m2", "floor", 57344.0, 127), ("e5m2", "floor", 1.0, 112),
            ("e5m2", "ceil", 57344.0, 127), ("e5m2", "ceil", 57345.0, 128), ("e4m3", "floor", 0.0, 0),
            ("e4m3", "ceil", 0.0, 0), ("e4m3", "floor", 2.0 ** -140, 0), ("e4m3", "floor", float("inf"), 255),
            ("e4m3", "ceil", float("nan"), 255)]
    for fmt, mode, amax, want in hand:
        got = oracle.mx_scale_code(amax, fmt, mode, lib=lib)
        assert got == want, f"scale({fmt}, {mode}, {amax!r}) = {got}, want {want}"
    rng = np.random.default_rng(29)
    for amax in np.exp(rng.uniform(-80, 80, 3000)):
        for fmt, p in _FP8.items():
            s = oracle.mx_scale_code(amax, fmt, "floor", lib=lib) - 127
            if -127 < s < 127:
                t = amax / 2.0 ** s
                assert 2.0 ** p["emax"] <= t < 2.0 ** (p["emax"] + 1), (fmt, amax, s)
            s = oracle.mx_scale_code(amax, fmt, "ceil", lib=lib) - 127
            if -127 < s < 127:
                t = amax / 2.0 ** s
                assert p["maxv"] / 2 < t <= p["maxv"], (fmt, amax, s)


def pin_mx_block_properties(lib):
    """Random rows: each block's scale depends only on its own 32 values;
    ceil mode never saturates; every dequantised value lies within half a
    quantum of V / X (or at the clamp in floor mode)."""
    rng = np.random.default_rng(31)
    cols = 32 * 5 + 7
    x = rng.normal(0, 1, (6, cols)) * np.exp(rng.uniform(-20, 20, (6, 1)))
    x[2, 40] = 0.0
    for fmt, p in _FP8.items():
        for mode in ("floor", "ceil"):
            codes, scales = oracle.mx_quantize(x, fmt, mode, lib=lib)
            assert scales.shape == (6, 6) and codes.shape == x.shape
            y = x.copy()
            y[:, 33] *= 1e6           # touches block 1 only (and makes it the row's largest)
            c2, s2 = oracle.mx_quantize(y, fmt, mode, lib=lib)
            assert np.array_equal(np.delete(s2, 1, axis=1), np.delete(scales, 1, axis=1))
            assert np.array_equal(np.delete(c2, np.s_[32:64], axis=1), np.delete(codes, np.s_[32:64], axis=1))
            for i in range(x.shape[0]):
                for j in range(cols):
                    b = j // 32
                    X = 2.0 ** (int(scales[i, b]) - 127)
                    v = x[i, j] / X
                    d = oracle.fp8_decode(int(codes[i, j]), fmt, lib=lib)
                    if abs(v) >= p["maxv"]:
                        assert mode == "floor" or abs(v) == p["maxv"], (fmt, mode, i, j)
                        assert abs(d) == p["maxv"]
                        continue
                    e = max(math.floor(math.log2(abs(v))) if v else 0, 1 - p["bias"])
                    q = 2.0 ** (e - p["mbits"])
                    assert abs(d - v) <= q / 2, (fmt, mode, i, j, v, d)


# --------------------------------------------------------------------------
# attention-residual mixing
# --------------------------------------------------------------------------

def pin_ares_golden(lib):
    for c in attn_res_cases():
        H = c["H"]
        blocks = np.array(c["blocks"], dtype=np.float64).reshape(1, -1, H)
        prefix = None if c["prefix"] is None else np.array(c["prefix"]).reshape(1, H)
        r = oracle.attn_res_forward(blocks, prefix, c["w"], c["p"], c["eps"], lib=lib)
        for got, want in zip(r["probs"][0], c["probs"]):
            _close(got, float(want), 1e-14, 1e-15, f"{c['name']} probs")
        for got, want in zip(r["out"][0], c["out"]):
            _close(got, float(want), 1e-14, 1e-14, f"{c['name']} out")


def _ares_library(blocks, prefix, w, p, eps):
    """The chain composed of torch library routines (float64)."""
    import torch
    v = torch.from_numpy(blocks)
    if prefix is not None:
        v = torch.cat([v, torch.from_numpy(prefix).unsqueeze(1)], dim=1)
    n = torch.nn.functional.rms_norm(v, (v.shape[-1],), weight=torch.from_numpy(np.asarray(w, np.float64)),
                                     eps=eps)
    logits = torch.matmul(n, torch.from_numpy(np.asarray(p, np.float64)))
    prob = torch.softmax(logits, dim=1)
    out = torch.matmul(prob.unsqueeze(1), v).squeeze(1)
    return out.numpy(), prob.numpy()


def pin_ares_vs_library(lib):
    rng = np.random.default_rng(41)
    for T, m, H, pref, eps in ((5, 3, 64, True, 1e-6), (4, 8, 200, True, 1e-2), (3, 2, 33, False, 0.5),
                               (2, 1, 16, False, 1e-6)):
        blocks = rng.normal(0, 1, (T, m, H)) * np.exp(rng.uniform(-2, 2, (T, m, 1)))
        prefix = rng.normal(0, 3, (T, H)) if pref else None
        w = 1 + 0.3 * rng.normal(0, 1, H)
        p = rng.normal(0, 2 / np.sqrt(H), H)
        r = oracle.attn_res_forward(blocks, prefix, w, p, eps, lib=lib)
        out, prob = _ares_library(blocks, prefix, w, p, eps)
        np.testing.assert_allclose(r["probs"], prob, rtol=1e-12, atol=1e-15)
        np.testing.assert_allclose(r["out"], out, rtol=1e-11, atol=1e-12 * np.abs(out).max())


def pin_ares_invariants(lib):
    rng = np.random.default_rng(43)
    T, m, H = 3, 4, 24
    blocks = rng.normal(0, 1, (T, m, H))
    prefix = rng.normal(0, 1, (T, H))
    w = 1 + 0.2 * rng.normal(0, 1, H)
    p = rng.normal(0, 0.5, H)
    base = oracle.attn_res_forward(blocks, prefix, w, p, 1e-3, lib=lib)
    # the prefix is the last block: split and stacked forms agree
    stacked = np.concatenate([blocks, prefix[:, None, :]], axis=1)
    st = oracle.attn_res_forward(stacked, None, w, p, 1e-3, lib=lib)
    np.testing.assert_allclose(st["out"], base["out"], rtol=1e-14, atol=1e-15)
    np.testing.assert_allclose(st["probs"], base["probs"], rtol=1e-14)
    # permuting the blocks permutes the probabilities and leaves out unchanged
    perm = [2, 4, 0, 3, 1]
    pm = oracle.attn_res_forward(stacked[:, perm], None, w, p, 1e-3, lib=lib)
    np.testing.assert_allclose(pm["probs"], base["probs"][:, perm], rtol=1e-13)
    np.testing.assert_allclose(pm["out"], base["out"], rtol=1e-13, atol=1e-14)
    # a zero projection gives equal probabilities: the mean of the blocks
    z = oracle.attn_res_forward(stacked, None, w, np.zeros(H), 1e-3, lib=lib)
    np.testing.assert_allclose(z["out"], stacked.mean(axis=1), rtol=1e-13, atol=1e-15)
    # identical blocks: out is that block
    same = np.repeat(prefix[:, None, :], 3, axis=1)
    np.testing.assert_allclose(oracle.attn_res_forward(same, None, w, p, 1e-3, lib=lib)["out"], prefix,
                               rtol=1e-14, atol=1e-15)
    # eps = 0: RMSNorm ignores a block's scale, so scaling block 1 by k keeps
    # the probabilities and adds P_1 (k - 1) x_1 to the output
    e0 = oracle.attn_res_forward(stacked, None, w, p, 0.0, lib=lib)
    sc = stacked.copy()
    sc[:, 1] *= 7.5
    e1 = oracle.attn_res_forward(sc, None, w, p, 0.0, lib=lib)
    np.testing.assert_allclose(e1["probs"], e0["probs"], rtol=1e-13)
    np.testing.assert_allclose(e1["out"], e0["out"] + e0["probs"][:, 1:2] * 6.5 * stacked[:, 1], rtol=1e-12,
                               atol=1e-13)
    # a projection aligned with one block's normalised row and scaled up makes
    # that block win: out tends to its raw values (not the normalised ones)
    tgt = stacked[0, 2] / w * 50.0
    big = oracle.attn_res_forward(stacked[:1], None, w, tgt, 0.0, lib=lib)
    np.testing.assert_allclose(big["out"][0], stacked[0, 2], rtol=1e-9, atol=1e-9)
    assert big["probs"][0, 2] > 1 - 1e-12
    # the magnitudes the tests scale tolerances with
    np.testing.assert_allclose(base["scale"], np.einsum("tb,tbh->th", base["probs"], np.abs(stacked)),
                               rtol=1e-13)
    assert np.all(base["absdot"] >= np.abs(base["logits"]) - 1e-12)


# --------------------------------------------------------------------------
# grouped FC1 + SiTU-GLU
# --------------------------------------------------------------------------

def pin_grouped_glu_brute_force(lib):
    """Tiny problems against triple loops written out: the grouping (rows of
    expert e use weight e), the gate/up halves of each weight, the routing
    weight per row, and the derivative terms against finite differences."""
    rng = np.random.default_rng(47)
    E, K, I = 3, 5, 2
    off = [0, 2, 2, 5]                      # expert 1 owns no rows
    M = off[-1]
    x = rng.integers(-3, 4, (M, K)).astype(np.float64) / 4
    w = rng.integers(-3, 4, (E, 2 * I, K)).astype(np.float64) / 4
    r = rng.uniform(0.1, 1.0, M)
    res = oracle.grouped_glu_forward(x, w, off, r, 4.0, 25.0, lib=lib)
    for e in range(E):
        for m in range(off[e], off[e + 1]):
            for j in range(I):
                g = sum(x[m, k] * w[e, j, k] for k in range(K))
                u = sum(x[m, k] * w[e, I + j, k] for k in range(K))
                assert abs(res["gate_up"][m, j] - g) < 1e-14 and abs(res["gate_up"][m, I + j] - u) < 1e-14
                want = r[m] * oracle.gate(g, 4.0, lib=lib) * oracle.up(u, 25.0, lib=lib)
                _close(res["out"][m, j], want, 1e-14, 1e-15, f"grouped out[{m},{j}]")
                sg = sum(abs(x[m, k] * w[e, j, k]) for k in range(K))
                _close(res["sG"][m, j], sg, 1e-14, 1e-15, "sG")
    # derivative terms: central differences of the output in G and U
    h = 1e-6
    for m, j in ((0, 1), (3, 0), (4, 1)):
        g, u = res["gate_up"][m, j], res["gate_up"][m, I + j]
        f = lambda gg, uu: r[m] * oracle.gate(gg, 4.0, lib=lib) * oracle.up(uu, 25.0, lib=lib)
        _close(res["dY_dG"][m, j], (f(g + h, u) - f(g - h, u)) / (2 * h), 1e-6, 1e-9, "dY/dG")
        _close(res["dY_dU"][m, j], (f(g, u + h) - f(g, u - h)) / (2 * h), 1e-6, 1e-9, "dY/dU")


def pin_mx_dequantize_vs_torch(lib):
    """MX decoding against torch's float8 dtypes and ldexp written out here:
    every code of both formats at several scales, ragged last blocks, and the
    E8M0 NaN scale."""
    import torch
    rng = np.random.default_rng(51)
    for fmt, tdt in (("e4m3", torch.float8_e4m3fn), ("e5m2", torch.float8_e5m2)):
        codes = rng.integers(0, 256, (3, 70), dtype=np.uint8)
        if fmt == "e4m3":
            codes[codes & 0x7F == 0x7F] = 0x11        # keep the NaN codes out of this part
        else:
            codes[(codes & 0x7C) == 0x7C] = 0x21      # inf / NaN codes out
        scales = np.array([[127, 120, 140], [0, 127, 254], [130, 100, 160]], dtype=np.uint8)
        got = oracle.mx_dequantize(codes, scales, fmt, lib=lib)
        dec = torch.from_numpy(codes).view(tdt).to(torch.float64).numpy()
        for r in range(3):
            for c in range(70):
                want = dec[r, c] * 2.0 ** (int(scales[r, c // 32]) - 127)
                assert got[r, c] == want, (fmt, r, c, got[r, c], want)
    nan = oracle.mx_dequantize(np.full((1, 40), 0x38, np.uint8), np.array([[255, 127]], np.uint8), "e4m3", lib=lib)
    assert np.all(np.isnan(nan[0, :32])) and np.all(nan[0, 32:] == 1.0)


def pin_grouped_mx_brute_force(lib):
    """The block-scaled grouped forward on a tiny problem against loops that
    decode every code by the E4M3 definition (sign, 4-bit exponent with bias
    7, 3-bit mantissa, subnormals at exponent 0) and apply the scales."""
    rng = np.random.default_rng(53)
    E, K, I = 2, 64, 2
    off = [0, 1, 3]
    xc = rng.integers(0, 0x7F, (3, K), dtype=np.uint8) | (rng.integers(0, 2, (3, K), dtype=np.uint8) << 7)
    wc = rng.integers(0, 0x7F, (E, 2 * I, K), dtype=np.uint8)
    xs = rng.integers(120, 135, (3, K // 32), dtype=np.uint8)
    ws = rng.integers(120, 135, (E, 2 * I, K // 32), dtype=np.uint8)
    r = rng.uniform(0.2, 1.0, 3)

    def dec(code):
        s, e, m = code >> 7, (code >> 3) & 15, code & 7
        v = (1 + m / 8) * 2.0 ** (e - 7) if e else (m / 8) * 2.0 ** -6
        return -v if s else v

    res = oracle.grouped_glu_forward_mx(xc, xs, wc, ws, off, r, "e4m3", 4.0, 25.0, lib=lib)
    for ex in range(E):
        for m in range(off[ex], off[ex + 1]):
            for j in range(I):
                g = sum(dec(int(xc[m, k])) * 2.0 ** (int(xs[m, k // 32]) - 127) * dec(int(wc[ex, j, k]))
                        * 2.0 ** (int(ws[ex, j, k // 32]) - 127) for k in range(K))
                u = sum(dec(int(xc[m, k])) * 2.0 ** (int(xs[m, k // 32]) - 127) * dec(int(wc[ex, I + j, k]))
                        * 2.0 ** (int(ws[ex, I + j, k // 32]) - 127) for k in range(K))
                assert abs(res["gate_up"][m, j] - g) <= 1e-13 * max(1.0, abs(g))
                assert abs(res["gate_up"][m, I + j] - u) <= 1e-13 * max(1.0, abs(u))
                want = r[m] * oracle.gate(g, 4.0, lib=lib) * oracle.up(u, 25.0, lib=lib)
                _close(res["out"][m, j], want, 1e-13, 1e-15, "grouped mx out")


ALL_PINS = [v for k, v in sorted(globals().items()) if k.startswith("pin_")]
