"""Planted mistakes in the oracle must be caught by the pins.

Each mutant is a copy of oracle/situ_oracle.c, oracle/mx_oracle.c or
oracle/attn_res_oracle.c with one
plausible slip (a dropped term, a wrong sign, a swapped operand or index, the
wrong rounding, a wrong format constant),
compiled with gcc into a temporary directory, or (the grouped FC1 oracle,
which is Python) a copy of oracle.grouped_glu_forward with one slip, swapped
in for the duration of the pins.  The mistakes are planted in the
CPU oracle only; no GPU code is involved.  A mutant that passes every pin
would mean the pins cannot see that kind of error.
"""
import os
import tempfile

import pytest

import oracle
from oracle_pins import ALL_PINS

SRC = os.path.join(os.path.dirname(oracle.__file__), "situ_oracle.c")
MX_SRC = os.path.join(os.path.dirname(oracle.__file__), "mx_oracle.c")
ARES_SRC = os.path.join(os.path.dirname(oracle.__file__), "attn_res_oracle.c")

MUTANTS = {
    "sech2_as_one_minus_tanh2": (
        "    double c = cosh(x);\n    return 1.0 / (c * c);",
        "    double t = tanh(x);\n    return 1.0 - t * t;"),
    "gate_grad_drops_second_term": (
        "return s * sech2(g / beta1) + beta1 * tanh(g / beta1) * s * sm;",
        "return s * sech2(g / beta1);"),
    "gate_grad_wrong_sign": (
        "return s * sech2(g / beta1) + beta1 * tanh(g / beta1) * s * sm;",
        "return s * sech2(g / beta1) - beta1 * tanh(g / beta1) * s * sm;"),
    "gate_grad_sigmoid_not_mirrored": (
        "    double sm = logistic(-g);\n    return s",
        "    double sm = logistic(g);\n    return s"),
    "gate_grad_missing_beta": (
        "+ beta1 * tanh(g / beta1) * s * sm;",
        "+ tanh(g / beta1) * s * sm;"),
    "gate_scaled_wrong_way": (
        "return beta1 * tanh(g / beta1) * logistic(g);",
        "return beta1 * tanh(g * beta1) * logistic(g);"),
    "logistic_negative_branch": (
        "    return e / (1.0 + e);", "    return 1.0 / (1.0 + e);"),
    "up_missing_beta2": (
        "return has_lb ? beta2 * tanh(u / beta2) : u;", "return has_lb ? tanh(u / beta2) : u;"),
    "up_ignores_none": (
        "return has_lb ? beta2 * tanh(u / beta2) : u;", "return beta2 * tanh(u / (beta2 + 1e-300));"),
    "up_grad_squared_wrong": (
        "return has_lb ? sech2(u / beta2) : 1.0;", "return has_lb ? sech2(u / beta2) / beta2 : 1.0;"),
    "gate_up_halves_swapped": (
        "double tg = situ_oracle_gate(gu[j], beta1);\n            double tu = situ_oracle_up(gu[inter + j], has_lb, beta2);\n            y[",
        "double tg = situ_oracle_gate(gu[inter + j], beta1);\n            double tu = situ_oracle_up(gu[j], has_lb, beta2);\n            y["),
    "forward_ignores_row_weight_index": (
        "double r = rw[rw_rows == 1 ? 0 : i];\n        const double *gu = gate_up + i * 2 * inter;\n        for",
        "double r = rw[0];\n        const double *gu = gate_up + i * 2 * inter;\n        for"),
    "dG_without_r": ("dgu[j] = o * r * tu * tgp;", "dgu[j] = o * tu * tgp;"),
    "dU_uses_gate_grad": ("dgu[inter + j] = o * r * tg * tup;", "dgu[inter + j] = o * r * tgp * tup;"),
    "dG_dU_swapped": (
        "dgu[j] = o * r * tu * tgp;\n            dgu[inter + j] = o * r * tg * tup;",
        "dgu[inter + j] = o * r * tu * tgp;\n            dgu[j] = o * r * tg * tup;"),
    "dr_includes_r": ("double p = o * tg * tu;", "double p = o * r * tg * tu;"),
    "dr_uses_abs": ("acc += p;", "acc += fabs(p);"),
    "dr_abs_includes_r": ("acc_abs += fabs(p);", "acc_abs += fabs(r * p);"),
    "dr_abs_signed": ("acc_abs += fabs(p);", "acc_abs += p;"),
    "dg_scale_drops_second_term": ("* (fabs(t1) + fabs(t2));", "* fabs(t1);"),
    "dg_scale_signed_sum": ("* (fabs(t1) + fabs(t2));", "* fabs(t1 + t2);"),
    "dg_scale_extra_beta": ("double t2 = beta1 * tanh(g / beta1) * s * sm;",
                            "double t2 = beta1 * beta1 * tanh(g / beta1) * s * sm;"),
    "dg_scale_without_r_and_tu": ("dg_scale[i * inter + j] = fabs(o * r * tu)", "dg_scale[i * inter + j] = fabs(o)"),
    "dg_scale_sigmoid_not_mirrored": ("double s = logistic(g), sm = logistic(-g);",
                                      "double s = logistic(g), sm = logistic(g);"),
    "bf16_truncates": ("double q = nearbyint(ax / quantum);", "double q = floor(ax / quantum);"),
    "bf16_ties_away": ("double q = nearbyint(ax / quantum);", "double q = round(ax / quantum);"),
    "bf16_no_subnormal_floor": ("    if (e < -126)\n        e = -126;", ""),
    "bf16_one_bit_short": ("double quantum = ldexp(1.0, e - 7);", "double quantum = ldexp(1.0, e - 6);"),
}

MX_MUTANTS = {
    "e4m3_bias_8": ("f.mbits = 3; f.bias = 7;", "f.mbits = 3; f.bias = 8;"),
    "e5m2_bias_16": ("f.mbits = 2; f.bias = 15;", "f.mbits = 2; f.bias = 16;"),
    "e4m3_emax_7": ("f.max_finite = 448.0; f.emax = 8;", "f.max_finite = 448.0; f.emax = 7;"),
    "e4m3_max_480": ("f.max_finite = 448.0;", "f.max_finite = 480.0;"),
    "subnormal_exponent_off_by_one": ("ldexp((double)m, 1 - f.bias - f.mbits)", "ldexp((double)m, -f.bias - f.mbits)"),
    "ties_away_from_zero": ("(above == below && ((lo + 1) & 1) == 0)", "(above == below)"),
    "ties_toward_zero": ("if (above < below || (above == below && ((lo + 1) & 1) == 0))", "if (above < below)"),
    "truncates": ("        if (above < below || (above == below && ((lo + 1) & 1) == 0))\n            pick = lo + 1;\n", ""),
    "no_saturation_nan": ("        return (uint8_t)(sign | f.max_code);", "        return (uint8_t)(sign | 0x7f);"),
    "drops_sign": ("uint8_t sign = signbit(x) ? 0x80 : 0x00;", "uint8_t sign = 0x00;"),
    "floor_scale_rounds_up": ("s = (e2 - 1) - f.emax;            /* floor", "s = e2 - f.emax;            /* floor"),
    "ceil_mode_is_floor": ("        while (amax > ldexp(f.max_finite, s))\n            ++s;\n", ""),
    "scale_divides_wrong_way": ("mx_oracle_fp8_encode(ldexp(v[i], -(sc - 127)), fmt)", "mx_oracle_fp8_encode(ldexp(v[i], sc - 127), fmt)"),
    "scale_no_low_clamp": ("    if (s < -127)\n        s = -127;\n", ""),
    "nan_block_finite_scale": ("int sc = nonfinite ? 255 : mx_oracle_scale_code", "int sc = nonfinite ? 254 : mx_oracle_scale_code"),
    "block_spans_rest_of_row": ("int n = (int)(cols - j0 < MX_BLOCK ? cols - j0 : MX_BLOCK);", "int n = (int)(cols - j0);"),
    "amax_signed": ("else if (fabs(v[i]) > amax)\n            amax = fabs(v[i]);", "else if (v[i] > amax)\n            amax = v[i];"),
    "scale_index_transposed": ("scales + i * nblk + b);", "scales + b * rows + i);"),
}


ARES_MUTANTS = {
    "rmsnorm_without_eps": ("sqrt(ss / (double)H + eps)", "sqrt(ss / (double)H)"),
    "rmsnorm_sum_not_mean": ("sqrt(ss / (double)H + eps)", "sqrt(ss + eps)"),
    "rmsnorm_not_inverted": ("double r = 1.0 / sqrt(", "double r = sqrt("),
    "norm_weight_dropped": ("double n = x * r * norm_w[h];", "double n = x * r;"),
    "logit_from_raw_values": ("dot += n * proj_w[h];", "dot += x * proj_w[h];"),
    "softmax_not_normalised": ("        P[b] /= den;\n", ""),
    "softmax_sign_flipped": ("P[b] = exp(l[b] - lmax);", "P[b] = exp(lmax - l[b]);"),
    "combine_normalised_values": ("o += P[b] * x;", "o += P[b] * x * norm_w[h];"),
    "prefix_ignored": ("const int64_t nb = m + (has_prefix ? 1 : 0);", "const int64_t nb = m;"),
    "always_block_zero": ("return blocks[(t * m + b) * H + h];", "return blocks[(t * m) * H + h];"),
    "prefix_row_index": ("return prefix[t * H + h];", "return prefix[h];"),
}


GROUPED_MUTANTS = {
    "grouped_always_expert_zero": ("gu[a:b] = X[a:b] @ W[e].T", "gu[a:b] = X[a:b] @ W[0].T"),
    "grouped_next_expert": ("gu[a:b] = X[a:b] @ W[e].T", "gu[a:b] = X[a:b] @ W[min(e + 1, E - 1)].T"),
    "grouped_halves_swapped": ("gu[a:b] = X[a:b] @ W[e].T", "gu[a:b] = X[a:b] @ np.roll(W[e], inter, axis=0).T"),
    "grouped_last_row_dropped": ("a, b = off[e], off[e + 1]", "a, b = off[e], max(off[e + 1] - 1, off[e])"),
    "grouped_offsets_start_at_one": ("a, b = off[e], off[e + 1]", "a, b = off[e] + (e == 0), off[e + 1]"),
    "grouped_magnitude_signed_x": ("s[a:b] = np.abs(X[a:b]) @ np.abs(W[e]).T", "s[a:b] = X[a:b] @ np.abs(W[e]).T"),
    "grouped_dG_without_r": ("dY_dG=rr * vgp(g) * tu", "dY_dG=vgp(g) * tu"),
    "grouped_dU_uses_gate_grad": ("dY_dU=rr * tg * vup(u)", "dY_dU=rr * vgp(g) * vup(u)"),
    "grouped_dG_uses_gate": ("dY_dG=rr * vgp(g) * tu", "dY_dG=rr * tg * tu"),
}


MXDQ_MUTANTS = {
    "mx_scale_bias_126": ("np.ldexp(1.0, (e - 127).clip(-127, 127))", "np.ldexp(1.0, (e - 126).clip(-127, 127))"),
    "mx_block_of_16": ("e = np.repeat(s.astype(np.int64), MX_BLOCK, axis=1)[:, :cols]",
                       "e = np.repeat(s.astype(np.int64), 16, axis=1)[:, :cols]; e = np.pad(e, ((0, 0), (0, max(0, cols - e.shape[1]))), mode='edge')[:, :cols]"),
    "mx_scale_ignored": ("return v * mult", "return v"),
    "mx_nan_scale_ignored": ("mult = np.where(e == 255, np.nan, np.ldexp", "mult = np.where(e == 256, np.nan, np.ldexp"),
    "mx_scale_negated": ("np.ldexp(1.0, (e - 127).clip(-127, 127))", "np.ldexp(1.0, (127 - e).clip(-127, 127))"),
}


GROUPED_MX_MUTANTS = {
    "mxg_weight_scales_of_expert_0": (
        "np.asarray(w_scales, dtype=np.uint8).reshape(E * two_i, -1)",
        "np.ascontiguousarray(np.broadcast_to(np.asarray(w_scales, dtype=np.uint8)[:1], "
        "np.asarray(w_scales).shape)).reshape(E * two_i, -1)"),
    "mxg_x_scales_rows_reversed": ("x = mx_dequantize(xc, x_scales, fmt, lib=lib)",
                                   "x = mx_dequantize(xc, np.asarray(x_scales)[::-1], fmt, lib=lib)"),
    "mxg_weight_format_swapped": (".reshape(E * two_i, -1), fmt,",
                                  ".reshape(E * two_i, -1), 'e5m2' if fmt == 'e4m3' else 'e4m3',"),
    "mxg_weight_rows_transposed": ("wc.reshape(E * two_i, K)", "wc.transpose(1, 0, 2).reshape(E * two_i, K)"),
}


def _py_mutant(func, table, name):
    import inspect
    old, new = table[name]
    text = inspect.getsource(func)
    assert text.count(old) == 1, f"mutation site for {name} not unique/found"
    ns = dict(vars(oracle))
    exec(compile(text.replace(old, new), f"<mutant {name}>", "exec"), ns)
    return ns[func.__name__]


def _grouped_mutant(name):
    return _py_mutant(oracle.grouped_glu_forward, GROUPED_MUTANTS, name)


@pytest.mark.parametrize("name", sorted(MXDQ_MUTANTS))
def test_mx_dequantize_mutant_is_caught(name, monkeypatch):
    monkeypatch.setattr(oracle, "mx_dequantize", _py_mutant(oracle.mx_dequantize, MXDQ_MUTANTS, name))
    lib = oracle.load()
    caught = []
    for pin in ALL_PINS:
        try:
            pin(lib)
        except (AssertionError, ValueError, FloatingPointError, OverflowError, IndexError):
            caught.append(pin.__name__)
    assert caught, f"mutant {name} passed every pin"


@pytest.mark.parametrize("name", sorted(GROUPED_MUTANTS))
def test_grouped_mutant_is_caught(name, monkeypatch):
    monkeypatch.setattr(oracle, "grouped_glu_forward", _grouped_mutant(name))
    lib = oracle.load()
    caught = []
    for pin in ALL_PINS:
        try:
            pin(lib)
        except (AssertionError, ValueError, FloatingPointError, OverflowError, IndexError):
            caught.append(pin.__name__)
    assert caught, f"mutant {name} passed every pin"


def _build_mutant(name, tmp):
    mx = name in MX_MUTANTS
    ares = name in ARES_MUTANTS
    table = MX_MUTANTS if mx else ARES_MUTANTS if ares else MUTANTS
    old, new = table[name]
    with open(MX_SRC if mx else ARES_SRC if ares else SRC) as f:
        text = f.read()
    assert text.count(old) == 1, f"mutation site for {name} not unique/found"
    path = os.path.join(tmp, f"m_{name}.c")
    with open(path, "w") as f:
        f.write(text.replace(old, new))
    out = os.path.join(tmp, f"libm_{name}.so")
    if mx:
        return oracle.build(mx_src=path, out=out)
    if ares:
        return oracle.build(ares_src=path, out=out)
    return oracle.build(src=path, out=out)


@pytest.mark.parametrize("name", sorted(MUTANTS) + sorted(MX_MUTANTS) + sorted(ARES_MUTANTS))
def test_mutant_is_caught(name):
    with tempfile.TemporaryDirectory() as tmp:
        lib = oracle.load(_build_mutant(name, tmp))
        caught = []
        for pin in ALL_PINS:
            try:
                pin(lib)
            except (AssertionError, ValueError, FloatingPointError, OverflowError) as e:
                caught.append(pin.__name__)
        assert caught, f"mutant {name} passed every pin"


@pytest.mark.parametrize("name", sorted(GROUPED_MX_MUTANTS))
def test_grouped_mx_mutant_is_caught(name, monkeypatch):
    """Mistakes in how the block-scaled grouped oracle decodes its operands
    (the composition of mx_dequantize and grouped_glu_forward)."""
    monkeypatch.setattr(oracle, "grouped_glu_forward_mx",
                        _py_mutant(oracle.grouped_glu_forward_mx, GROUPED_MX_MUTANTS, name))
    lib = oracle.load()
    caught = []
    for pin in ALL_PINS:
        try:
            pin(lib)
        except (AssertionError, ValueError, FloatingPointError, OverflowError, IndexError):
            caught.append(pin.__name__)
    assert caught, f"mutant {name} passed every pin"
