"""Readers for the hand-derived fixtures under tests/golden/."""
from __future__ import annotations

import math
import os
import re
from fractions import Fraction

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")

_LN = re.compile(r"^(-?[0-9/]+)\*ln\((\d+)\)(?:/(\d+))?$")


def parse_rational(tok: str) -> Fraction:
    return Fraction(tok)


def parse_x(tok: str) -> float:
    """A number, or k*ln(n) / k*ln(n)/m with rational k, as the nearest double."""
    m = _LN.match(tok)
    if m:
        k = Fraction(m.group(1))
        n = int(m.group(2))
        d = int(m.group(3)) if m.group(3) else 1
        return float(k) * math.log(n) / d
    return float(Fraction(tok))


def closed_forms():
    rows = []
    with open(os.path.join(GOLDEN, "closed_forms.txt")) as f:
        for line in f:
            line = line.split("#", 1)[0].strip()
            if not line:
                continue
            kind, b1, b2, x, exp = line.split()
            if b2 == "-":
                beta2 = None          # not used by this kind
            elif b2 == "none":
                beta2 = "none"        # linear_beta None
            else:
                beta2 = float(b2)
            rows.append({
                "kind": kind,
                "beta1": None if b1 == "-" else float(b1),
                "beta2": beta2,
                "x": parse_x(x),
                "x_text": x,
                "expected": Fraction(exp),
            })
    return rows


def worked_cases():
    cases = []
    cur = None
    with open(os.path.join(GOLDEN, "worked_rows.txt")) as f:
        for line in f:
            line = line.split("#", 1)[0].strip()
            if not line:
                continue
            key, _, rest = line.partition(" ")
            rest = rest.strip()
            if key == "case":
                cur = {"name": rest}
                cases.append(cur)
            elif key == "beta1":
                cur["beta1"] = float(rest)
            elif key == "beta2":
                cur["beta2"] = None if rest == "none" else float(rest)
            elif key in ("G", "U", "go"):
                cur[key] = [[parse_x(t) for t in row.split()] for row in rest.split(";")]
            elif key in ("r", "dr", "dr_abs"):
                cur[key] = [Fraction(t.strip()) for t in rest.split(";")]
            else:  # Y, dG, dU, dg_scale: exact rationals per row
                cur[key] = [[Fraction(t) for t in row.split()] for row in rest.split(";")]
    return cases


def _num(tok: str) -> float:
    if tok.lower() == "nan":
        return float("nan")
    if "0x" in tok.lower():
        return float.fromhex(tok)
    return float(tok)


def mx_blocks():
    """Hand-worked MXFP8 blocks: dicts with name, fmt, mode, cols, values
    (padded with zeros to cols), scales and codes (None when not given)."""
    out = []
    cur = None
    with open(os.path.join(GOLDEN, "mx_blocks.txt")) as f:
        for line in f:
            line = line.split("#", 1)[0].strip()
            if not line:
                continue
            key, *toks = line.split()
            if key == "block":
                name, fmt, mode, cols = toks
                cur = {"name": name, "fmt": fmt, "mode": mode, "cols": int(cols)}
                out.append(cur)
            elif key == "values":
                v = [_num(t) for t in toks]
                cur["values"] = v + [0.0] * (cur["cols"] - len(v))
            elif key == "scales":
                cur["scales"] = [int(t) for t in toks]
            elif key == "codes":
                if toks == ["-"]:
                    cur["codes"] = None
                else:
                    c = [int(t, 16) for t in toks]
                    cur["codes"] = c + [0] * (cur["cols"] - len(c))
    return out


def attn_res_cases():
    """Hand-worked attention-residual cases (tests/golden/attn_res_cases.txt)."""
    out = []
    cur = None
    with open(os.path.join(GOLDEN, "attn_res_cases.txt")) as f:
        for line in f:
            line = line.split("#", 1)[0].strip()
            if not line:
                continue
            key, *toks = line.split()
            if key == "case":
                cur = {"name": toks[0], "blocks": [], "prefix": None}
                out.append(cur)
            elif key == "H":
                cur["H"] = int(toks[0])
            elif key == "eps":
                cur["eps"] = float(Fraction(toks[0]))
            elif key in ("w", "p"):
                cur[key] = [parse_x(t) for t in toks]
            elif key == "block":
                cur["blocks"].append([float(Fraction(t)) for t in toks])
            elif key == "prefix":
                cur["prefix"] = [float(Fraction(t)) for t in toks]
            elif key in ("probs", "out"):
                cur[key] = [Fraction(t) for t in toks]
    return out
