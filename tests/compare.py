"""Comparison helpers for parity tests: bit patterns, ulp distances, gates.

The gates follow the parity bar for this operator: the fused residual output
is bit-exact; normalised outputs are within 1 ulp of the output dtype (or
|difference| <= 1e-6 near zero) for fp16/bf16, and within rtol = atol = 1e-6
for fp32 (kernscope README, "Numerical tolerances" table, FP32 row).  Large
16-bit cases must also match bit for bit on at least 99.9% of elements,
because a 1-ulp bound alone cannot tell normalising the unrounded residual
sum from normalising its rounded copy.
"""
from __future__ import annotations

from dataclasses import dataclass

import torch

_INT_VIEW = {torch.float16: torch.int16, torch.bfloat16: torch.int16, torch.float32: torch.int32}


def bits(t: torch.Tensor) -> torch.Tensor:
    """Raw bit patterns as int64 (unsigned value of the storage word)."""
    t = t.detach().cpu().contiguous()
    iv = t.view(_INT_VIEW[t.dtype]).to(torch.int64)
    width = 16 if t.dtype in (torch.float16, torch.bfloat16) else 32
    return iv & ((1 << width) - 1)


def _ordered(t: torch.Tensor) -> torch.Tensor:
    """Map bit patterns onto integers ordered like the values (+0 and -0 both map to 0)."""
    width = 16 if t.dtype in (torch.float16, torch.bfloat16) else 32
    b = bits(t)
    sign = (b >> (width - 1)) & 1
    mag = b & ((1 << (width - 1)) - 1)
    return torch.where(sign == 1, -mag, mag)


def ulp_distance(a: torch.Tensor, b: torch.Tensor) -> torch.Tensor:
    """Elementwise distance in units in the last place of the storage dtype.

    Two NaNs are at distance 0; a NaN against a number is at distance 2**40.
    """
    assert a.dtype == b.dtype and a.shape == b.shape, (a.dtype, b.dtype, a.shape, b.shape)
    a, b = a.detach().cpu(), b.detach().cpu()
    d = (_ordered(a) - _ordered(b)).abs()
    na, nb = torch.isnan(a.float()), torch.isnan(b.float())
    d = torch.where(na & nb, torch.zeros_like(d), d)
    d = torch.where(na ^ nb, torch.full_like(d, 2**40), d)
    return d


@dataclass
class ParityStats:
    n: int
    max_ulp: int
    exact_rate: float
    max_abs: float
    worst_index: int

    def __str__(self) -> str:
        return (f"n={self.n} max_ulp={self.max_ulp} exact={self.exact_rate:.6f} "
                f"max_abs={self.max_abs:.3g} worst@{self.worst_index}")


def stats(out: torch.Tensor, ref: torch.Tensor) -> ParityStats:
    d = ulp_distance(out, ref).reshape(-1)
    n = d.numel()
    if n == 0:
        return ParityStats(0, 0, 1.0, 0.0, -1)
    diff = (out.detach().cpu().float() - ref.detach().cpu().float()).abs().reshape(-1)
    diff = torch.nan_to_num(diff, nan=0.0, posinf=float("inf"))
    worst = int(torch.argmax(d))
    return ParityStats(n, int(d.max()), float((d == 0).sum()) / n, float(diff.max()), worst)


# The RMSNorm oracle's own fp32 results stay within 4 fp32 ulps of the fp64
# brute force (its pin); the normalisation bar for fp32 outputs adds this
# ceiling to rtol = atol = 1e-6.
FP32_MAX_ULP = 4


def check_normalised(out: torch.Tensor, ref: torch.Tensor, min_exact_rate: float | None = None,
                     fp32_max_ulp: int | None = None) -> ParityStats:
    """Gate for a normalised output; raises AssertionError with the stats on failure.
    fp32_max_ulp: for fp32 outputs, also a ceiling on the ulp distance."""
    st = stats(out, ref)
    if st.n == 0:
        return st
    o, r = out.detach().cpu(), ref.detach().cpu()
    if o.dtype == torch.float32:
        ok = torch.isclose(o, r, rtol=1e-6, atol=1e-6, equal_nan=True)
        assert bool(ok.all()), f"fp32 outside rtol=atol=1e-6: {st}"
        if fp32_max_ulp is not None:
            assert st.max_ulp <= fp32_max_ulp, f"fp32 more than {fp32_max_ulp} ulps apart: {st}"
    else:
        d = ulp_distance(o, r)
        near_zero = (o.float() - r.float()).abs() <= 1e-6
        bad = (d > 1) & ~near_zero
        assert not bool(bad.any()), f"more than 1 ulp apart: {st}"
    # The exact-match gate is for 16-bit outputs, where an fp32 pipeline lands on
    # the same rounded value almost always.  fp32 outputs carry the fp32 pipeline's
    # own few-ulp differences (summation order) and are judged by rtol/atol alone.
    if min_exact_rate is not None and o.dtype != torch.float32:
        assert st.exact_rate >= min_exact_rate, f"exact-match rate below {min_exact_rate}: {st}"
    return st


def check_bitexact(out: torch.Tensor, ref: torch.Tensor) -> None:
    """Gate for the fused residual output: every bit equal (NaNs compared by NaN-ness)."""
    o, r = out.detach().cpu(), ref.detach().cpu()
    assert o.shape == r.shape and o.dtype == r.dtype
    same = bits(o) == bits(r)
    nan_both = torch.isnan(o.float()) & torch.isnan(r.float())
    bad = ~(same | nan_both)
    if bool(bad.any()):
        idx = int(torch.nonzero(bad.reshape(-1))[0])
        raise AssertionError(f"{int(bad.sum())} of {o.numel()} elements differ; first at flat index {idx}: "
                             f"{hex(int(bits(o).reshape(-1)[idx]))} vs {hex(int(bits(r).reshape(-1)[idx]))}")


def check_gradient(out: torch.Tensor, ref: torch.Tensor, magnitude: torch.Tensor,
                   min_exact_rate: float | None = None, rel: float = 2.0 ** -16) -> ParityStats:
    """Gate for a gradient, whose value may be a difference of much larger terms:
    each element meets the normalisation bar (1 ulp of bf16/fp16 or |difference|
    <= 1e-6; fp32 rtol = atol = 1e-6) against the exact value, or lies within
    rel * magnitude of it, where magnitude bounds the terms an fp32 evaluation
    rounds (2^-16 is 256 fp32 ulps: room for a sum over up to 2^16 elements)."""
    st = stats(out, ref)
    if st.n == 0:
        return st
    o, r = out.detach().cpu(), ref.detach().cpu()
    if o.dtype == torch.float32:
        ok = torch.isclose(o, r, rtol=1e-6, atol=1e-6, equal_nan=True)
    else:
        ok = (ulp_distance(o, r) <= 1) | ((o.float() - r.float()).abs() <= 1e-6)
    ok = ok | ((o.double() - r.double()).abs() <= rel * magnitude.double().cpu())
    assert bool(ok.all()), f"gradient outside the bar at {int((~ok).sum())} elements: {st}"
    if min_exact_rate is not None and o.dtype != torch.float32:
        assert st.exact_rate >= min_exact_rate, f"exact-match rate below {min_exact_rate}: {st}"
    return st


def backward_magnitudes(dy: torch.Tensor, x: torch.Tensor, w: torch.Tensor, eps: float):
    """For the RMSNorm backward, the sizes of the terms behind each gradient
    element, in float64 from the widened inputs (used for the tolerance only):
    dx_j = rho (g_j - c x_j) with g = dy w and c = rho^2 sum(g x) / H, whose sum
    rounds terms of size |g x|; dw_j sums dy_j x_j rho over the rows."""
    import numpy as np

    h = x.shape[-1]
    xd, dyd, wd = x.double().reshape(-1, h), dy.double().reshape(-1, h), w.double()
    rho = 1.0 / torch.sqrt(xd.pow(2).mean(-1, keepdim=True) + float(np.float32(eps)))
    g = dyd * wd
    gx = g * xd
    c = rho ** 2 * gx.sum(-1, keepdim=True) / h
    mdx = rho * (g.abs() + (c * xd).abs() + xd.abs() * rho ** 2 / h * gx.abs().sum(-1, keepdim=True))
    mdw = (dyd * xd * rho).abs().sum(0)
    return mdx.reshape(x.shape), mdw
