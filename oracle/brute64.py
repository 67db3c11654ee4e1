"""Exact-arithmetic brute force for tiny inputs.  TEST INFRASTRUCTURE ONLY.

A second statement of the kernscope "Numerical contract" (sections "RMSNorm",
"Fused residual-add RMSNorm", "SwiGLU activation" and "Softmax") that shares nothing with
``ks_oracle.c``:
the sum of squares, the mean and eps are exact rationals, the square root is
taken to 80 significant digits, and the result is rounded ONCE to the output
format (round to nearest, ties to even) by integer arithmetic on the rational.
Only the fused form's fp32 residual sum is rounded to fp32 first, because the
contract defines s as an fp32 value.

It is meant for a few hundred elements at most (pure Python).  The SwiGLU
and softmax statements at the end follow the same approach.
"""
from __future__ import annotations

import math
from decimal import Decimal, localcontext
from fractions import Fraction

# (significand bits incl. the implicit one, smallest normal exponent, largest finite value)
FORMATS = {
    "float32": (24, -126, (2 - Fraction(1, 2**23)) * Fraction(2) ** 127),
    "float16": (11, -14, Fraction(65504)),
    "bfloat16": (8, -126, (2 - Fraction(1, 2**7)) * Fraction(2) ** 127),
}


def round_to(q: Fraction, fmt: str) -> float:
    """Nearest value of ``fmt`` to the rational q, ties to even; +-inf past the largest finite."""
    prec, emin, max_finite = FORMATS[fmt]
    if q == 0:
        return 0.0
    neg = q < 0
    a = -q if neg else q
    lead = a.numerator.bit_length() - a.denominator.bit_length()  # 2^lead <= a < 2^(lead+2)
    if Fraction(2) ** (lead + 1) <= a:
        lead += 1
    elif Fraction(2) ** lead > a:
        lead -= 1
    lead = max(lead, emin)
    qexp = lead - (prec - 1)
    n = round(a / Fraction(2) ** qexp)  # Fraction rounding: half to even
    v = n * Fraction(2) ** qexp
    if v > max_finite:
        return -math.inf if neg else math.inf
    out = float(v)  # exact: v has at most 24 significant bits
    return -out if neg else out


def _inv_sqrt(m: Fraction) -> Fraction:
    with localcontext() as ctx:
        ctx.prec = 80
        d = Decimal(m.numerator) / Decimal(m.denominator)
        return Fraction(1 / d.sqrt())


def rms_norm(x: list[list[float]], w: list[float], eps32: float, fmt: str) -> list[list[float]]:
    """Rows x (exact values of the stored elements), weight w, eps already rounded to fp32."""
    out = []
    hidden = len(w)
    for row in x:
        assert len(row) == hidden
        m = sum(Fraction(v) ** 2 for v in row) / hidden + Fraction(eps32)
        inv = _inv_sqrt(m)
        out.append([round_to(Fraction(v) * Fraction(wj) * inv, fmt) for v, wj in zip(row, w)])
    return out


def fused_add_rms_norm(x: list[list[float]], r: list[list[float]], w: list[float], eps32: float,
                       fmt: str) -> tuple[list[list[float]], list[list[float]]]:
    """Returns (x_out, residual_out) as values."""
    s = [[round_to(Fraction(a) + Fraction(b), "float32") for a, b in zip(xr, rr)] for xr, rr in zip(x, r)]
    residual = [[round_to(Fraction(v), fmt) for v in row] for row in s]
    return rms_norm(s, w, eps32, fmt), residual


def rms_norm_residual(x: list[list[float]], r: list[list[float]], w: list[float], eps32: float,
                      fmt: str) -> list[list[float]]:
    """Out of place: the normalisation of the fp32 sum s = x + r (rounded to fp32,
    as the fused contract defines s), nothing else written."""
    s = [[round_to(Fraction(a) + Fraction(b), "float32") for a, b in zip(xr, rr)] for xr, rr in zip(x, r)]
    return rms_norm(s, w, eps32, fmt)


def rms_norm_backward(dy: list[list[float]], x: list[list[float]], w: list[float], eps32: float,
                      fmt: str) -> tuple[list[list[float]], list[float]]:
    """Gradients of y_j = x_j rho w_j, rho = (sum x^2 / H + eps)^(-1/2), for the
    incoming dy: exact rationals with an 80-digit rho, each rounded once."""
    hidden = len(w)
    dx, dw = [], [Fraction(0)] * hidden
    for grow, row in zip(dy, x):
        m = sum(Fraction(v) ** 2 for v in row) / hidden + Fraction(eps32)
        rho = _inv_sqrt(m)
        dot = sum(Fraction(g) * Fraction(wj) * Fraction(v) for g, wj, v in zip(grow, w, row))
        coef = rho ** 3 * dot / hidden
        dx.append([round_to(rho * Fraction(g) * Fraction(wj) - coef * Fraction(v), fmt)
                   for g, wj, v in zip(grow, w, row)])
        dw = [acc + Fraction(g) * Fraction(v) * rho for acc, g, v in zip(dw, grow, row)]
    return dx, [round_to(v, fmt) for v in dw]


def _sigmoid(g: Fraction) -> Fraction:
    with localcontext() as ctx:
        ctx.prec = 80
        e = (-Decimal(g.numerator) / Decimal(g.denominator)).exp()
        return Fraction(1 / (1 + e))


def silu_and_mul(x: list[list[float]], fmt: str) -> list[list[float]]:
    """SwiGLU of rows of 2D values (kernscope "Numerical contract" > "SwiGLU
    activation"): gate * sigmoid(gate) * up with an 80-digit exponential and one
    rounding to the output format."""
    out = []
    for row in x:
        d = len(row) // 2
        out.append([round_to(Fraction(g) * _sigmoid(Fraction(g)) * Fraction(u), fmt)
                    for g, u in zip(row[:d], row[d:])])
    return out


def _exp(q: Fraction) -> Fraction:
    with localcontext() as ctx:
        ctx.prec = 80
        return Fraction((Decimal(q.numerator) / Decimal(q.denominator)).exp())


def softmax(x: list[list[float]], fmt: str) -> list[list[float]]:
    """Softmax of rows of finite values (kernscope "Numerical contract" >
    "Softmax"): the row maximum, z = the fp32 rounding of each element minus it
    (the contract forms z in fp32), 80-digit exponentials, an exact sum and
    quotient, rounded to fp32 and then to the output format."""
    out = []
    for row in x:
        m = max(Fraction(v) for v in row)
        es = [_exp(Fraction(round_to(Fraction(v) - m, "float32"))) for v in row]
        s = sum(es)
        out.append([round_to(Fraction(round_to(e / s, "float32")), fmt) for e in es])
    return out
