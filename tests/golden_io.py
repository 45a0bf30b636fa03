"""Readers for the hand-worked fixtures under tests/golden/ (test helper)."""
from __future__ import annotations

import math
import os
from fractions import Fraction

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _lines(name):
    with open(os.path.join(GOLDEN, name)) as f:
        for raw in f:
            line = raw.strip()
            if line and not line.startswith("#"):
                yield line


def _value(tok: str) -> float:
    if tok in ("inf", "-inf", "nan"):
        return float(tok)
    neg = tok.startswith("-")
    v = float(Fraction(tok.lstrip("-")))
    return -v if neg else v  # keeps the sign of -0


def handworked_block():
    """Returns (qs bytes, q_minus_8 list, {d_bits: value}, [(d_bits, index, value)])."""
    qs, qm8, ds, checks = None, None, {}, []
    for line in _lines("q4_0_block_handworked.txt"):
        key, rest = line.split(":", 1)
        toks = rest.split()
        if key == "qs":
            qs = bytes(int(t, 16) for t in toks)
        elif key == "q_minus_8":
            qm8 = [int(t) for t in toks]
        elif key == "d":
            ds[int(toks[0], 16)] = _value(toks[1])
        elif key == "check":
            checks.append((int(toks[0], 16), int(toks[1]), float(toks[2])))
    return qs, qm8, ds, checks


def fp16_patterns():
    out = []
    for line in _lines("fp16_bit_patterns.txt"):
        bits, val = line.split()
        out.append((int(bits, 16), _value(val)))
    return out


def gemv_cases():
    out = []
    for line in _lines("gemv_handworked.txt"):
        _, rest = line.split(":", 1)
        xs, ys = rest.split("|")
        out.append(([float(t) for t in xs.split()], [float(t) for t in ys.split()]))
    return out


def same_float(a: float, b: float) -> bool:
    """Bitwise-style equality: NaN == NaN, and the sign of zero must match."""
    if math.isnan(a) or math.isnan(b):
        return math.isnan(a) and math.isnan(b)
    return a == b and math.copysign(1.0, a) == math.copysign(1.0, b)
