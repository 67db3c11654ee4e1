"""Write constant_rows.txt: closed-form outputs of RMSNorm on constant rows.

For a row holding H copies of c and a weight of ones, the kernscope contract
("Numerical contract", RMSNorm) gives mean(x^2) = c^2, so every output element
is c / sqrt(c^2 + eps), rounded to the input dtype.  This script evaluates that
closed form to 60 digits and rounds it once (ties to even) with the
exact-rational rounding of ``oracle/brute64.py``; it calls nothing else.

Each case is chosen so that every partial sum k*c^2 (k <= H) is exact in fp32,
so any summation order reaches the same fp32 mean and a correct implementation
must hit these bits for 16-bit dtypes.  ``margin`` is the distance, in output
ulps, from the closed-form value to the nearest rounding boundary: a large
margin means the fp32 rounding of the intermediate steps cannot move the
result across a boundary.

Run from the repository root:  python tests/golden/make_constant_rows.py [OUTPUT]
(default output: tests/golden/constant_rows.txt)
"""
from __future__ import annotations

import os
import sys
from decimal import Decimal, localcontext
from fractions import Fraction

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)
from oracle.brute64 import FORMATS, round_to  # noqa: E402

OUT = os.path.join(os.path.dirname(os.path.abspath(__file__)), "constant_rows.txt")

# (dtype, c as an exact decimal string, eps, [H ...])
CASES = [
    ("bfloat16", "1", 1e-6, [1, 5, 1000, 4096, 16384]),
    ("bfloat16", "0.5", 1e-6, [1, 1000, 4096]),
    ("bfloat16", "3", 1e-6, [5, 4096, 16384]),
    ("bfloat16", "-1.5", 1e-6, [3, 4096]),
    ("bfloat16", "0.0009765625", 1e-6, [1, 4096, 16384]),   # 2^-10: c^2 close to eps
    ("bfloat16", "0.001953125", 1e-5, [4096]),              # 2^-9 with eps 1e-5
    ("bfloat16", "0.000244140625", 1e-6, [16384]),          # 2^-12: eps dominates
    ("bfloat16", "1000", 1e-6, [64, 512]),
    ("float16", "1", 1e-6, [1, 5, 1000, 4096, 16384]),
    ("float16", "-1", 1e-5, [4096]),
    ("float16", "0.0009765625", 1e-6, [1, 4096]),
    ("float16", "0.001953125", 1e-5, [4096]),
    ("float16", "0.000244140625", 1e-6, [16384]),
    ("float16", "3", 1e-5, [4096]),
    ("float32", "1", 1e-6, [1, 4096]),
    ("float32", "0.0009765625", 1e-6, [4096]),
    ("float32", "-2", 1e-5, [1000]),
]

_BITS = {"bfloat16": 16, "float16": 16, "float32": 32}


def _fp32(v: float) -> Fraction:
    return Fraction(float(np.float32(v)))


def _closed_form(c: Fraction, eps32: Fraction) -> Fraction:
    with localcontext() as ctx:
        ctx.prec = 60
        m = c * c + eps32
        root = (Decimal(m.numerator) / Decimal(m.denominator)).sqrt()
        return Fraction(Decimal(c.numerator) / Decimal(c.denominator) / root)


def _margin(y: Fraction, fmt: str) -> float:
    """Distance from y to the nearest rounding boundary of fmt, in ulps of fmt at y."""
    prec, emin, _ = FORMATS[fmt]
    a = abs(y)
    lead = a.numerator.bit_length() - a.denominator.bit_length()
    if Fraction(2) ** (lead + 1) <= a:
        lead += 1
    elif Fraction(2) ** lead > a:
        lead -= 1
    lead = max(lead, emin)
    q = Fraction(2) ** (lead - (prec - 1))
    frac = (a / q) - int(a / q)           # position inside one quantum, in [0, 1)
    return float(abs(frac - Fraction(1, 2)))


def _pattern(value: float, fmt: str) -> int:
    if fmt == "float32":
        return int(np.array([value], dtype=np.float32).view(np.uint32)[0])
    if fmt == "float16":
        return int(np.array([value], dtype=np.float16).view(np.uint16)[0])
    f32 = int(np.array([value], dtype=np.float32).view(np.uint32)[0])
    assert f32 & 0xFFFF == 0, "bf16 value must be exact in fp32 with a zero low half"
    return f32 >> 16


def table() -> str:
    """The table's text."""
    lines = [
        "# RMSNorm of constant rows with unit weight: y = c / sqrt(c^2 + eps), one rounding",
        "# Source: kernscope README, 'Numerical contract' > 'RMSNorm' (closed form for a constant row).",
        "# eps is first rounded to fp32, as the contract adds it in fp32.",
        "# Written by tests/golden/make_constant_rows.py; do not edit by hand.",
        "# dtype c eps H expected_bits margin_ulps",
    ]
    for fmt, cs, eps, hs in CASES:
        c = Fraction(Decimal(cs))
        assert round_to(c, fmt) == float(c), f"c={cs} is not a {fmt} value"
        eps32 = _fp32(eps)
        y = _closed_form(c, eps32)
        yv = round_to(y, fmt)
        for h in hs:
            c2 = c * c
            odd = c2.numerator
            while odd % 2 == 0:
                odd //= 2
            bits_needed = odd.bit_length() + h.bit_length()  # significant bits of k*c^2 for k <= H
            assert c2.denominator & (c2.denominator - 1) == 0 and bits_needed <= 24, (fmt, cs, h)
            width = _BITS[fmt] // 4
            lines.append(f"{fmt} {cs} {eps:g} {h} 0x{_pattern(yv, fmt):0{width}x} {_margin(y, fmt):.4f}")
    return "\n".join(lines) + "\n"


def main(argv: list[str]) -> None:
    """Write the table to the path given (default: constant_rows.txt next to this script)."""
    out = argv[0] if argv else OUT
    text = table()
    with open(out, "w") as f:
        f.write(text)
    print(f"wrote {out} ({text.count(chr(10)) - 5} cases)")


if __name__ == "__main__":
    main(sys.argv[1:])
