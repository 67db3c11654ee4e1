"""Checks that pin the CPU oracle to facts fixed outside the oracle itself.

Each check takes an oracle library handle (``oracle.load()`` or a build of a
deliberately broken copy) and raises AssertionError when the oracle
disagrees.  Sources of truth:

- closed forms and invariants that follow from the kernscope contract
  ("Numerical contract": RMSNorm, Fused residual-add RMSNorm);
- an exact-rational brute force (``oracle/brute64.py``, tiny inputs);
- library routines that compute the same thing by a different route: torch
  and numpy casts, torch's fp32 evaluation of the formula.
"""
from __future__ import annotations

import os

import numpy as np
import torch

import oracle
from oracle import brute64
from compare import bits, check_bitexact, check_normalised, stats, ulp_distance
import workloads

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", "constant_rows.txt")
DT = {"float32": torch.float32, "float16": torch.float16, "bfloat16": torch.bfloat16}


def read_constant_rows():
    rows = []
    with open(GOLDEN) as f:
        for line in f:
            if line.startswith("#") or not line.strip():
                continue
            fmt, c, eps, h, expected, margin = line.split()
            rows.append((fmt, float(c), float(eps), int(h), int(expected, 16), float(margin)))
    return rows


def _pattern_tensor(pattern: int, dtype: torch.dtype, n: int) -> torch.Tensor:
    if dtype == torch.float32:
        return torch.full((n,), pattern, dtype=torch.int64).to(torch.int32).view(torch.float32)
    signed = pattern - (1 << 16) if pattern >= (1 << 15) else pattern
    return torch.full((n,), signed, dtype=torch.int16).view(dtype)


# --------------------------------------------------------------------------
# P-a: constant rows against the closed form c / sqrt(c^2 + eps)
# --------------------------------------------------------------------------
def pin_constant_rows(lib) -> None:
    for fmt, c, eps, h, expected, margin in read_constant_rows():
        dt = DT[fmt]
        x = torch.full((2, h), c, dtype=dt)
        w = torch.ones(h, dtype=dt)
        want = _pattern_tensor(expected, dt, h).expand(2, h)
        y = oracle.rms_norm(x, w, eps, lib=lib)
        if fmt == "float32":
            assert int(ulp_distance(y, want).max()) <= 4, (fmt, c, eps, h)
        else:
            check_bitexact(y, want)
        # fused: x + residual = c exactly (two halves), residual_out must be c
        half = torch.full((2, h), c / 2, dtype=dt)
        xo, ro = oracle.fused_add_rms_norm(half, half.clone(), w, eps, lib=lib)
        check_bitexact(ro, x)
        if fmt == "float32":
            assert int(ulp_distance(xo, want).max()) <= 4, (fmt, c, eps, h)
        else:
            check_bitexact(xo, want)


# --------------------------------------------------------------------------
# P-b: unit weight gives output RMS sqrt(ms / (ms + eps))
# --------------------------------------------------------------------------
def pin_unit_weight_rms(lib) -> None:
    for dtype, seed in (("bfloat16", 11), ("float16", 12), ("float32", 13)):
        inp = workloads.random_case((16, 512), dtype, seed)
        x = inp["x"]
        w = torch.ones(512, dtype=x.dtype)
        for eps in (1e-6, 0.5):
            y = oracle.rms_norm(x, w, eps, lib=lib).double()
            ms = x.double().pow(2).mean(-1)
            want = torch.sqrt(ms / (ms + float(np.float32(eps))))
            got = y.pow(2).mean(-1).sqrt()
            rel = ((got - want).abs() / want).max().item()
            assert rel < 2.0 ** -8, (dtype, eps, rel)


# --------------------------------------------------------------------------
# P-c: exact-rational brute force on tiny inputs
# --------------------------------------------------------------------------
BRUTE_SHAPES = [(5,), (2, 3, 5), (3, 1000), (4, 1), (3, 2), (2, 3), (2, 8), (2, 64)]


def _values(t: torch.Tensor) -> list:
    t = t.float().reshape(-1, t.shape[-1])
    return [[float(v) for v in row] for row in t]


def _from_values(vals: list, dtype: torch.dtype, shape) -> torch.Tensor:
    return torch.tensor(vals, dtype=torch.float64).to(torch.float32).to(dtype).reshape(shape)


def pin_brute_force(lib) -> None:
    for dtype in ("bfloat16", "float16", "float32"):
        for i, shape in enumerate(BRUTE_SHAPES):
            inp = workloads.random_case(shape, dtype, 100 + i, residual=workloads.normal(0, 0.7))
            x, r, w = inp["x"], inp["residual"], inp["weight"]
            eps = 1e-6 if i % 2 == 0 else 1e-5
            eps32 = float(np.float32(eps))
            want = _from_values(brute64.rms_norm(_values(x), [float(v) for v in w.float()], eps32, dtype),
                                x.dtype, shape)
            got = oracle.rms_norm(x, w, eps, lib=lib)
            _check_brute(got, want, dtype, shape)
            bx, br = brute64.fused_add_rms_norm(_values(x), _values(r), [float(v) for v in w.float()], eps32, dtype)
            gx, gr = oracle.fused_add_rms_norm(x, r, w, eps, lib=lib)
            check_bitexact(gr, _from_values(br, x.dtype, shape))
            _check_brute(gx, _from_values(bx, x.dtype, shape), dtype, shape)


def _check_brute(got: torch.Tensor, want: torch.Tensor, dtype: str, shape) -> None:
    d = int(ulp_distance(got, want).max())
    # 16-bit outputs: at most 1 ulp.  fp32 outputs: the oracle rounds about six
    # times in fp32 against one rounding for the brute force, so a few ulps.
    limit = 4 if dtype == "float32" else 1
    assert d <= limit, (dtype, shape, d)


# --------------------------------------------------------------------------
# P-d: power-of-two scaling;  P-e: sign symmetry
# --------------------------------------------------------------------------
def pin_scaling_and_sign(lib) -> None:
    for dtype in ("bfloat16", "float16", "float32"):
        inp = workloads.random_case((8, 300), dtype, 21)
        x, r, w = inp["x"], inp["residual"], inp["weight"]
        # keep |x| >= 2^-6 so that neither scaled inputs nor scaled outputs reach
        # the fp16 subnormal range, where power-of-two scaling stops being exact
        x = (torch.sign(x.float()) * x.float().abs().clamp_min(2.0 ** -6)).to(x.dtype)
        eps = 1e-6
        eps32 = float(np.float32(eps))
        y = oracle.rms_norm(x, w, eps, lib=lib)
        for k in (-3, 2):
            xs = (x.float() * 2.0 ** k).to(x.dtype)   # exact: power-of-two scaling in range
            ys = oracle.rms_norm(xs, w, eps32 * 4.0 ** k, lib=lib)
            check_bitexact(ys, y)
            ws = (w.float() * 2.0 ** k).to(w.dtype)
            yw = oracle.rms_norm(x, ws, eps, lib=lib)
            check_bitexact(yw, (y.float() * 2.0 ** k).to(y.dtype))
        check_bitexact(oracle.rms_norm(-x, w, eps, lib=lib), -y)
        # fused: (x, r) -> (-x, -r) flips both outputs.  Compared by value: where
        # x = -r the IEEE sum is +0 for both signs, so only the zero's sign differs.
        gx, gr = oracle.fused_add_rms_norm(x, r, w, eps, lib=lib)
        nx, nr = oracle.fused_add_rms_norm(-x, -r, w, eps, lib=lib)
        assert int(ulp_distance(nx, -gx).max()) == 0
        assert int(ulp_distance(nr, -gr).max()) == 0


# --------------------------------------------------------------------------
# P-f: fused residual closed form;  P-g: zero residual reduces to rms_norm
# --------------------------------------------------------------------------
def pin_fused_residual(lib) -> None:
    for dtype in ("bfloat16", "float16", "float32"):
        inp = workloads.random_case((32, 1000), dtype, 31, residual=workloads.normal(0, 3))
        x, r, w = inp["x"], inp["residual"], inp["weight"]
        _, ro = oracle.fused_add_rms_norm(x, r, w, 1e-6, lib=lib)
        check_bitexact(ro, (x.float() + r.float()).to(x.dtype))   # torch fp32 add + RNE cast
        zx, zr = oracle.fused_add_rms_norm(x, torch.zeros_like(x), w, 1e-6, lib=lib)
        check_bitexact(zr, x)
        check_bitexact(zx, oracle.rms_norm(x, w, 1e-6, lib=lib))


# --------------------------------------------------------------------------
# P-h: each row is independent of the batch around it
# --------------------------------------------------------------------------
def pin_batch_invariance(lib) -> None:
    inp = workloads.random_case((9, 777), "bfloat16", 41)
    x, r, w = inp["x"], inp["residual"], inp["weight"]
    y = oracle.rms_norm(x, w, 1e-6, lib=lib)
    gx, gr = oracle.fused_add_rms_norm(x, r, w, 1e-6, lib=lib)
    for i in (0, 4, 8):
        check_bitexact(oracle.rms_norm(x[i:i + 1].contiguous(), w, 1e-6, lib=lib), y[i:i + 1])
        ox, orr = oracle.fused_add_rms_norm(x[i:i + 1].contiguous(), r[i:i + 1].contiguous(), w, 1e-6, lib=lib)
        check_bitexact(ox, gx[i:i + 1])
        check_bitexact(orr, gr[i:i + 1])


# --------------------------------------------------------------------------
# P-i: casts against torch (bf16) and numpy (fp16)
# --------------------------------------------------------------------------
def _fp32_from_bits(b: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(b.astype(np.uint32).view(np.int32)).view(torch.float32)


def cast_test_patterns(dtype: torch.dtype) -> torch.Tensor:
    """fp32 inputs for the rounding test: every 16-bit prefix with tie and near-tie tails,
    plus every midpoint between neighbouring 16-bit values and its fp32 neighbours."""
    rng = np.random.default_rng(7)
    if dtype == torch.bfloat16:
        hi = np.arange(1 << 16, dtype=np.uint64) << 16
        lows = np.array([0, 1, 0x7FFF, 0x8000, 0x8001, 0xFFFF], dtype=np.uint64)
        pats = (hi[:, None] | lows[None, :]).reshape(-1)
        extra = rng.integers(0, 1 << 32, size=1 << 20, dtype=np.uint64)
    else:
        hi = np.arange(1 << 19, dtype=np.uint64) << 13
        lows = np.array([0, 1, 0xFFF, 0x1000, 0x1001, 0x1FFF], dtype=np.uint64)
        pats = (hi[:, None] | lows[None, :]).reshape(-1)
        # around the fp16 subnormal and overflow ranges, where the rounding bit moves
        sub = rng.integers(0, 1 << 23, size=1 << 20, dtype=np.uint64)
        ex = rng.integers(100, 114, size=1 << 20, dtype=np.uint64)
        extra = (ex << 23) | sub | (rng.integers(0, 2, size=1 << 20, dtype=np.uint64) << 31)
    vals = _fp32_from_bits(np.concatenate([pats, extra]))
    # midpoints between consecutive positive finite 16-bit values, and their neighbours
    b = torch.arange(0, 0x7C00 if dtype == torch.float16 else 0x7F80, dtype=torch.int32)
    v0 = b.to(torch.int16).view(dtype).double()
    v1 = (b + 1).to(torch.int16).view(dtype).double()
    mid = ((v0 + v1) / 2).float()    # exact in fp32 for both formats
    up = torch.nextafter(mid, torch.tensor(float("inf")))
    dn = torch.nextafter(mid, torch.tensor(float("-inf")))
    allv = torch.cat([vals, mid, up, dn])
    return torch.cat([allv, -allv])


def pin_casts(lib) -> None:
    # widening: every 16-bit pattern
    allbits = torch.arange(-(1 << 15), 1 << 15, dtype=torch.int32).to(torch.int16)
    for dtype in (torch.bfloat16, torch.float16):
        got = oracle.widen(allbits, dtype, lib=lib)
        ref = allbits.view(dtype).float()
        same = (got.view(torch.int32) == ref.view(torch.int32)) | (torch.isnan(got) & torch.isnan(ref))
        assert bool(same.all()), f"widen {dtype}: {int((~same).sum())} patterns differ"
    # rounding
    for dtype in (torch.bfloat16, torch.float16):
        v = cast_test_patterns(dtype)
        got = oracle.round_f32(v, dtype, lib=lib)
        if dtype == torch.bfloat16:
            ref = v.to(torch.bfloat16).view(torch.int16)
        else:
            with np.errstate(over="ignore"):   # overflow to inf is the expected result
                ref = torch.from_numpy(v.numpy().astype(np.float16).view(np.int16))
        gv, rv = got.view(dtype).float(), ref.view(dtype).float()
        same = (got == ref) | (torch.isnan(gv) & torch.isnan(rv))
        if not bool(same.all()):
            i = int(torch.nonzero(~same)[0])
            raise AssertionError(f"round {dtype}: {int((~same).sum())} of {v.numel()} differ; "
                                 f"first {v[i].item()!r}: {int(got[i]) & 0xFFFF:#06x} vs {int(ref[i]) & 0xFFFF:#06x}")


# --------------------------------------------------------------------------
# P-j: torch's fp32 evaluation of the formula (a different summation order)
# --------------------------------------------------------------------------
def torch_fp32_rms_norm(x: torch.Tensor, w: torch.Tensor, eps: float) -> torch.Tensor:
    x32 = x.float()
    scale = torch.rsqrt(x32.pow(2).mean(-1, keepdim=True) + np.float32(eps))
    return (x32 * scale * w.float()).to(x.dtype)


def pin_library_formula(lib) -> None:
    for name in ("C2", "C3", "C3b"):
        wl = workloads.WORKLOADS[name]
        inp = workloads.make_inputs(wl, rows=256)
        x, r, w = inp["x"], inp["residual"], inp["weight"]
        y = oracle.rms_norm(x, w, wl.eps, lib=lib)
        check_normalised(y, torch_fp32_rms_norm(x, w, wl.eps), min_exact_rate=0.999)
        f = torch.nn.functional.rms_norm(x.float(), (wl.hidden,), w.float(), wl.eps).to(x.dtype)
        check_normalised(y, f, min_exact_rate=0.999)
        # fused: normalise the fp32 sum
        gx, _ = oracle.fused_add_rms_norm(x, r, w, wl.eps, lib=lib)
        s = x.float() + r.float()
        ref = (s * torch.rsqrt(s.pow(2).mean(-1, keepdim=True) + np.float32(wl.eps)) * w.float()).to(x.dtype)
        check_normalised(gx, ref, min_exact_rate=0.999)
    # fp32 dtype against torch with the page's fp32 tolerance
    inp = workloads.random_case((64, 4096), "float32", 51)
    y = oracle.rms_norm(inp["x"], inp["weight"], 1e-6, lib=lib)
    check_normalised(y, torch_fp32_rms_norm(inp["x"], inp["weight"], 1e-6))


# --------------------------------------------------------------------------
# P-k: the contract normalises the UNROUNDED fp32 sum; the exact-match gate
# separates that from normalising the stored (rounded) residual
# --------------------------------------------------------------------------
def pin_unrounded_sum(lib) -> None:
    wl = workloads.WORKLOADS["C2"]
    inp = workloads.make_inputs(wl, rows=128)
    x, r, w = inp["x"], inp["residual"], inp["weight"]
    gx, gr = oracle.fused_add_rms_norm(x, r, w, wl.eps, lib=lib)
    wrong = oracle.rms_norm(gr, w, wl.eps, lib=lib)      # normalising the rounded sum
    st = stats(gx, wrong)
    assert st.max_ulp <= 2, st                              # a ulp bound alone barely tells them apart
    assert st.exact_rate < 0.95, st                         # the exact-match gate does
    s = x.float() + r.float()
    ref = (s * torch.rsqrt(s.pow(2).mean(-1, keepdim=True) + np.float32(wl.eps)) * w.float()).to(x.dtype)
    assert stats(gx, ref).exact_rate > stats(wrong, ref).exact_rate


# --------------------------------------------------------------------------
# zeros, and empty batches
# --------------------------------------------------------------------------
def pin_zeros_and_empty(lib) -> None:
    for dtype in (torch.bfloat16, torch.float16, torch.float32):
        x = torch.zeros(3, 64, dtype=dtype)
        w = torch.ones(64, dtype=dtype)
        y = oracle.rms_norm(x, w, 1e-6, lib=lib)
        assert bool((bits(y) == 0).all())
        e = torch.zeros(0, 64, dtype=dtype)
        assert oracle.rms_norm(e, w, 1e-6, lib=lib).shape == (0, 64)
        ex, er = oracle.fused_add_rms_norm(e, e.clone(), w, 1e-6, lib=lib)
        assert ex.shape == er.shape == (0, 64)


# --------------------------------------------------------------------------
# Out-of-place residual RMSNorm (Triton Kernels README, "Kernels")
# --------------------------------------------------------------------------
def pin_residual_out_of_place(lib) -> None:
    """Brute force on tiny shapes; x + x is RMSNorm of x with eps / 4 bit for bit
    (every step scales by a power of two); a zero residual is rms_norm; the
    inputs are left unchanged; the sum is not rounded before normalising."""
    for dtype in ("bfloat16", "float16", "float32"):
        for i, shape in enumerate(BRUTE_SHAPES):
            inp = workloads.random_case(shape, dtype, 500 + i, residual=workloads.normal(0, 0.7))
            x, r, w = inp["x"], inp["residual"], inp["weight"]
            eps32 = float(np.float32(1e-6))
            want = brute64.rms_norm_residual(_values(x), _values(r), [float(v) for v in w.float()], eps32, dtype)
            got = oracle.rms_norm_residual(x, r, w, 1e-6, lib=lib)
            _check_brute(got, _from_values(want, x.dtype, shape), dtype, shape)
        inp = workloads.random_case((16, 1000), dtype, 510)
        x, r, w = inp["x"], inp["residual"], inp["weight"]
        # keep x away from the fp16 subnormal range, where doubling is still exact
        # but the eps / 4 identity needs every scaled value normal
        x = (torch.sign(x.float()) * x.float().abs().clamp_min(2.0 ** -6)).to(x.dtype)
        x0, r0 = x.clone(), r.clone()
        eps32 = float(np.float32(1e-5))
        check_bitexact(oracle.rms_norm_residual(x, x, w, eps32, lib=lib), oracle.rms_norm(x, w, eps32 / 4, lib=lib))
        check_bitexact(oracle.rms_norm_residual(x, torch.zeros_like(x), w, 1e-6, lib=lib),
                       oracle.rms_norm(x, w, 1e-6, lib=lib))
        y = oracle.rms_norm_residual(x, r, w, 1e-6, lib=lib)
        check_bitexact(x, x0)
        check_bitexact(r, r0)
        if dtype != "float32":
            # normalising the rounded sum is a different (<= 1 ulp away) result
            rounded = oracle.rms_norm((x.float() + r.float()).to(x.dtype), w, 1e-6, lib=lib)
            assert float((ulp_distance(y, rounded) == 0).double().mean()) < 0.999


# --------------------------------------------------------------------------
# RMSNorm backward: the gradients of the forward contract (no page states a
# backward contract; the kernscope reference supports autograd)
# --------------------------------------------------------------------------
def _autograd64(dy, x, w, eps32):
    """torch autograd, in float64, of the forward formula on the widened inputs."""
    xd = x.double().requires_grad_()
    wd = w.double().requires_grad_()
    y = xd * torch.rsqrt(xd.pow(2).mean(-1, keepdim=True) + eps32) * wd
    y.backward(dy.double())
    return xd.grad, wd.grad


def _round_like(v: torch.Tensor, dtype: torch.dtype) -> torch.Tensor:
    return v.to(torch.float32).to(dtype)


def pin_backward_autograd(lib) -> None:
    """fp64 autograd (a different route to the same derivative) within 1 ulp."""
    for dtype in ("bfloat16", "float16", "float32"):
        for i, shape in enumerate([(3, 7), (4, 64), (2, 3, 100), (16, 1000)]):
            inp = workloads.random_case(shape, dtype, 600 + i)
            x, w = inp["x"], inp["weight"]
            dy = workloads.random_case(shape, dtype, 650 + i)["residual"]
            eps32 = float(np.float32(1e-5))
            gx, gw = oracle.rms_norm_backward(dy, x, w, 1e-5, lib=lib)
            ax, aw = _autograd64(dy.reshape(-1, shape[-1]), x.reshape(-1, shape[-1]), w, eps32)
            ax = _round_like(ax.reshape(shape), x.dtype)
            aw = _round_like(aw, x.dtype)
            assert int(ulp_distance(gx, ax).max()) <= 1, (dtype, shape)
            assert int(ulp_distance(gw, aw).max()) <= 1, (dtype, shape)
            assert float((ulp_distance(gx, ax) == 0).double().mean()) >= 0.99


def pin_backward_brute_force(lib) -> None:
    for dtype in ("bfloat16", "float16", "float32"):
        for i, shape in enumerate([(5,), (2, 3, 5), (3, 17), (2, 64)]):
            inp = workloads.random_case(shape, dtype, 700 + i)
            x, w = inp["x"], inp["weight"]
            dy = workloads.random_case(shape, dtype, 750 + i)["residual"]
            eps32 = float(np.float32(1e-6))
            bx, bw = brute64.rms_norm_backward(_values(dy), _values(x), [float(v) for v in w.float()], eps32, dtype)
            gx, gw = oracle.rms_norm_backward(dy, x, w, 1e-6, lib=lib)
            assert int(ulp_distance(gx, _from_values(bx, x.dtype, shape)).max()) <= 1
            assert int(ulp_distance(gw, _from_values([bw], x.dtype, (1, shape[-1])).reshape(-1)).max()) <= 1


def pin_backward_identities(lib) -> None:
    """Scale invariance up to eps: sum_j dx_j x_j = eps rho^3 sum_j dy_j w_j x_j;
    a single row with dy = 1 has dw = x rho, the forward output with unit
    weight; finite differences of the (pinned) forward oracle; zero dy gives
    zero gradients; dy scales the gradients exactly; no rows: dw = 0."""
    inp = workloads.random_case((6, 300), "float32", 801)
    x, w = inp["x"], inp["weight"]
    dy = workloads.random_case((6, 300), "float32", 802)["residual"]
    eps = 1e-2                       # large enough that the identity's right side is not tiny
    eps32 = float(np.float32(eps))
    gx, gw = oracle.rms_norm_backward(dy, x, w, eps, lib=lib)
    xd, wd, dyd = x.double(), w.double(), dy.double()
    rho = 1.0 / torch.sqrt(xd.pow(2).mean(-1) + eps32)
    lhs = (gx.double() * xd).sum(-1)
    rhs = eps32 * rho ** 3 * (dyd * wd * xd).sum(-1)
    bound = (gx.double() * xd).abs().sum(-1) * 2.0 ** -23 + rhs.abs() * 1e-12
    assert bool(((lhs - rhs).abs() <= bound).all()), (lhs - rhs, bound)
    one = torch.ones(1, 300, dtype=torch.float32)
    _, g1 = oracle.rms_norm_backward(one, x[:1].contiguous(), w, eps, lib=lib)
    fwd = oracle.rms_norm(x[:1].contiguous(), torch.ones(300, dtype=torch.float32), eps, lib=lib).reshape(-1)
    assert int(ulp_distance(g1, fwd).max()) <= 1
    # central differences of L(x) = sum(dy * y(x)) with the forward oracle in fp32
    h = 2.0 ** -7
    for j in (0, 17, 299):
        xp, xm = x[2:3].clone(), x[2:3].clone()
        xp[0, j] += h
        xm[0, j] -= h
        lp = (dyd[2:3] * oracle.rms_norm(xp, w, eps, lib=lib).double()).sum()
        lm = (dyd[2:3] * oracle.rms_norm(xm, w, eps, lib=lib).double()).sum()
        fd = float((lp - lm) / (2 * h))
        assert abs(fd - float(gx[2, j])) <= 2e-3 * (abs(float(gx[2, j])) + 0.05), (j, fd, float(gx[2, j]))
    zx, zw = oracle.rms_norm_backward(torch.zeros_like(dy), x, w, eps, lib=lib)
    assert bool((zx == 0).all()) and bool((zw == 0).all())
    for dtype in (torch.bfloat16, torch.float16):
        xb, wb, db = x.to(dtype), w.to(dtype), (dy * 0.25).to(dtype)
        ax, aw = oracle.rms_norm_backward(db, xb, wb, eps, lib=lib)
        bx, bw = oracle.rms_norm_backward((db.float() * 4).to(dtype), xb, wb, eps, lib=lib)
        # exact where the smaller gradient is a normal number (subnormals have a
        # fixed quantum, so scaling them is not exact)
        normal = ax.float().abs() >= torch.finfo(dtype).tiny
        check_bitexact(bx[normal], (ax.float() * 4).to(dtype)[normal])
        check_bitexact(bw, (aw.float() * 4).to(dtype))
    ex, ew = oracle.rms_norm_backward(torch.zeros(0, 300), torch.zeros(0, 300), w, eps, lib=lib)
    assert ex.shape == (0, 300) and bool((ew == 0).all())


# --------------------------------------------------------------------------
# SwiGLU (kernscope "Numerical contract" > "SwiGLU activation")
# --------------------------------------------------------------------------
SWIGLU_SHAPES = [(2,), (3, 10), (2, 3, 14), (2, 64), (3, 402)]


def _swiglu_case(shape, dtype, seed):
    x = workloads.random_case(shape, dtype, seed, x=workloads.normal(0, 2))["x"]
    flat = x.reshape(-1)
    # extreme gate values: the sigmoid saturates at both ends
    extremes = torch.tensor([0.0, -0.0, 20.0, -20.0, 100.0, -100.0, 1e-3, -1e-3]).to(x.dtype)
    k = min(len(extremes), flat.numel() // 2)
    flat[:k] = extremes[:k]
    return x


def pin_swiglu_brute_force(lib) -> None:
    for dtype in ("bfloat16", "float16", "float32"):
        for i, shape in enumerate(SWIGLU_SHAPES):
            x = _swiglu_case(shape, dtype, 300 + i)
            want = brute64.silu_and_mul(_values(x), dtype)
            got = oracle.silu_and_mul(x, lib=lib)
            want_t = _from_values(want, x.dtype, got.shape)
            # 16-bit outputs: at most 1 ulp.  fp32 outputs: the page's fp32 tolerance
            # (the contract's fp32 sigmoid is subnormal for very negative gates, so a
            # count of ulps there says nothing)
            check_normalised(got, want_t)


def torch_swiglu(x: torch.Tensor) -> torch.Tensor:
    d = x.shape[-1] // 2
    g, u = x[..., :d].float(), x[..., d:].float()
    return (torch.nn.functional.silu(g) * u).to(x.dtype)


def pin_swiglu_library(lib) -> None:
    for dtype in ("bfloat16", "float16"):
        x = workloads.random_case((256, 2 * 1024), dtype, 310, x=workloads.normal(0, 2))["x"]
        check_normalised(oracle.silu_and_mul(x, lib=lib), torch_swiglu(x), min_exact_rate=0.999)
    x = workloads.random_case((64, 2 * 512), "float32", 311)["x"]
    check_normalised(oracle.silu_and_mul(x, lib=lib), torch_swiglu(x))


def pin_swiglu_closed_forms(lib) -> None:
    for dtype in (torch.bfloat16, torch.float16, torch.float32):
        d = 300
        g = torch.full((4, d), 0.0)
        g[0] = torch.linspace(18.0, 60.0, d)      # fp32 sigmoid rounds to exactly 1 from g >= 18
        g[1] = 0.0                                 # silu(0) = 0
        g[2] = -torch.linspace(18.0, 60.0, d)
        g[3] = torch.linspace(-3, 3, d)
        u = torch.linspace(-2.0, 2.0, d).expand(4, d)
        x = torch.cat([g, u], dim=1).to(dtype).contiguous()
        y = oracle.silu_and_mul(x, lib=lib)
        gq, uq = x[:, :d].float(), x[:, d:].float()
        check_bitexact(y[0], (gq[0] * uq[0]).to(dtype))
        assert bool((y[1].float() == 0).all())
        # very negative gates: |out| <= |g| e^g |u| (sigmoid(g) < e^g), up to the output's rounding
        # (1%, or half a quantum where the output is subnormal)
        quantum = torch.finfo(dtype).tiny * torch.finfo(dtype).eps
        bound = (gq[2].abs() * torch.exp(gq[2]) * uq[2].abs()) * 1.01 + quantum / 2
        assert bool((y[2].float().abs() <= bound).all())
        # odd in up: negating the up half negates the output exactly
        xn = torch.cat([x[:, :d], -x[:, d:]], dim=1).contiguous()
        assert int(ulp_distance(oracle.silu_and_mul(xn, lib=lib), -y).max()) == 0
    e = torch.zeros(0, 8, dtype=torch.bfloat16)
    assert oracle.silu_and_mul(e, lib=lib).shape == (0, 4)


# --------------------------------------------------------------------------
# Softmax (kernscope "Numerical contract" > "Softmax"; nonfinite rules there)
# --------------------------------------------------------------------------
SOFTMAX_SHAPES = [(1,), (2, 5), (3, 17), (2, 64), (2, 3, 40)]
INF, NAN = float("inf"), float("nan")


def _softmax_case(shape, dtype, seed):
    x = workloads.random_case(shape, dtype, seed, x=workloads.normal(0, 3))["x"]
    flat = x.reshape(-1)
    if flat.numel() >= 8:
        # mixed magnitudes: z = x - max is inexact in fp32 here, so forming z in
        # a wider format would show; and logits far beyond exp's fp32 range
        flat[:4] = torch.tensor([100.0, 1e-3, -37.25, 99.5]).to(x.dtype)
        flat[4:8] = torch.tensor([-120.0, 3.0e-2, -0.0, 0.0]).to(x.dtype)
    return x


def pin_softmax_brute_force(lib) -> None:
    """Bit-exact agreement with exact rationals and an 80-digit exponential (the
    oracle's double evaluation is off by about 1e-15 relative, so the two can
    round differently only within about 2^-50 of a rounding boundary)."""
    for dtype in ("bfloat16", "float16", "float32"):
        for i, shape in enumerate(SOFTMAX_SHAPES):
            x = _softmax_case(shape, dtype, 400 + i)
            got = oracle.softmax(x, lib=lib)
            want = _from_values(brute64.softmax(_values(x), dtype), x.dtype, got.shape)
            check_bitexact(got, want)


def _sigmoid64(t: torch.Tensor) -> torch.Tensor:
    return 1.0 / (1.0 + torch.exp(-t))


def pin_softmax_closed_forms(lib) -> None:
    for dt in (torch.bfloat16, torch.float16, torch.float32):
        # a constant row gives 1/H everywhere (z = 0, exp = 1, sum = H)
        for h in (1, 3, 7, 100, 1000, 4096):
            for c in (0.0, -2.5, 7.0, 1024.0, -60000.0):
                x = torch.full((2, h), c).to(dt)
                want = torch.full((2, h), 1.0 / h, dtype=torch.float64).to(torch.float32).to(dt)
                check_bitexact(oracle.softmax(x, lib=lib), want)
        # two entries: the logistic function of their difference
        a = torch.linspace(-6, 6, 49).to(dt).float()
        b = torch.linspace(3, -3, 49).to(dt).float()
        x = torch.stack([a, b], dim=1).to(dt).contiguous()
        y = oracle.softmax(x, lib=lib)
        d = (a - b).double()       # exact here: both are multiples of 1/8 within +-9
        want = torch.stack([_sigmoid64(d), _sigmoid64(-d)], dim=1).to(torch.float32).to(dt)
        assert int(ulp_distance(y, want).max()) <= 1
        # logits far beyond exp's range: only differences matter, so the result
        # equals that of the shifted row exactly (the shifts are exact here)
        big = torch.tensor([[1024.0, 1016.0, 1008.0, 0.0], [0.0, -1024.0, -2048.0, -4096.0]]).to(dt)
        small = torch.tensor([[0.0, -8.0, -16.0, -1024.0], [0.0, -1024.0, -2048.0, -4096.0]]).to(dt)
        yb = oracle.softmax(big, lib=lib)
        check_bitexact(yb, oracle.softmax(small, lib=lib))
        assert bool(torch.isfinite(yb.float()).all()) and float(yb[1, 0]) == 1.0 and bool((yb[1, 1:] == 0).all())
        # shift invariance, bit for bit: values on a 1/2 grid below 64 in magnitude
        # (7 significant bits, so exact in every dtype, and so is every z)
        g = (torch.randint(-16, 16, (8, 33), generator=torch.Generator().manual_seed(5)).double() / 2)
        check_bitexact(oracle.softmax((g + 32).to(dt), lib=lib), oracle.softmax(g.to(dt), lib=lib))


def pin_softmax_invariants(lib) -> None:
    for dt, tol in ((torch.float32, 2.0**-23), (torch.float16, 2.0**-10), (torch.bfloat16, 2.0**-7)):
        x = workloads.random_case((64, 300), {torch.float32: "float32", torch.float16: "float16",
                                              torch.bfloat16: "bfloat16"}[dt], 410,
                                  x=workloads.normal(0, 4))["x"]
        y = oracle.softmax(x, lib=lib)
        yd = y.double()
        # each output is within half an ulp of an exact quotient: the row sums to 1
        # within about half an ulp of 1 in total
        assert float((yd.sum(-1) - 1).abs().max()) <= tol, float((yd.sum(-1) - 1).abs().max())
        # order preserving: larger logits never get smaller probabilities
        xs, order = x.float().sort(dim=-1)
        ys = torch.gather(yd, 1, order)
        assert bool((ys[:, 1:] >= ys[:, :-1]).all())
        # reversing a row reverses its output
        yr = oracle.softmax(x.flip(-1).contiguous(), lib=lib)
        assert int(ulp_distance(yr.flip(-1), y).max()) <= 1
        assert float((ulp_distance(yr.flip(-1), y) == 0).double().mean()) >= 0.99


def pin_softmax_nonfinite(lib) -> None:
    """The page's rules: NaN or +inf anywhere, or only -inf: NaN everywhere in
    the row; -inf entries of a row with finite values: 0, the rest as if they
    were absent.  A single element: 1 when finite."""
    for dt in (torch.bfloat16, torch.float16, torch.float32):
        rows = torch.tensor([[1.0, NAN, 2.0, -INF], [INF, 1.0, 2.0, 3.0], [-INF] * 4, [INF, INF, 0.0, -INF],
                             [NAN] * 4, [-INF, 0.5, -INF, 2.0]]).to(dt)
        y = oracle.softmax(rows, lib=lib).float()
        assert bool(torch.isnan(y[:5]).all())
        assert float(y[5, 0]) == 0.0 and float(y[5, 2]) == 0.0
        masked = oracle.softmax(torch.tensor([[0.5, 2.0]]).to(dt), lib=lib)
        check_bitexact(oracle.softmax(rows[5:6].contiguous(), lib=lib)[:, [1, 3]].contiguous(), masked)
        one = oracle.softmax(torch.tensor([[3.0], [-1e4], [INF], [-INF], [NAN]]).to(dt), lib=lib).float()
        assert one[0, 0] == 1.0 and one[1, 0] == 1.0 and bool(torch.isnan(one[2:]).all())
        assert oracle.softmax(torch.zeros(0, 7, dtype=dt), lib=lib).shape == (0, 7)


def pin_softmax_library(lib) -> None:
    """torch.softmax on the widened input (the page's own reference) lands within
    the output tolerance."""
    for dtype in ("bfloat16", "float16"):
        x = workloads.random_case((256, 1024), dtype, 420, x=workloads.normal(0, 2))["x"]
        ref = torch.softmax(x.float(), dim=-1).to(x.dtype)
        check_normalised(oracle.softmax(x, lib=lib), ref, min_exact_rate=0.999)
    x = workloads.random_case((64, 1000), "float32", 421, x=workloads.normal(0, 2))["x"]
    check_normalised(oracle.softmax(x, lib=lib), torch.softmax(x, dim=-1))


ALL_PINS = [
    pin_constant_rows, pin_unit_weight_rms, pin_brute_force, pin_scaling_and_sign, pin_fused_residual,
    pin_batch_invariance, pin_casts, pin_library_formula, pin_unrounded_sum, pin_zeros_and_empty,
    pin_swiglu_brute_force, pin_swiglu_library, pin_swiglu_closed_forms,
    pin_softmax_brute_force, pin_softmax_closed_forms, pin_softmax_invariants, pin_softmax_nonfinite,
    pin_softmax_library, pin_residual_out_of_place, pin_backward_autograd, pin_backward_brute_force,
    pin_backward_identities,
]


def first_failure(lib) -> str | None:
    """Run every pin; return the name and message of the first that fails, else None."""
    for pin in ALL_PINS:
        try:
            pin(lib)
        except (AssertionError, ValueError, ZeroDivisionError, OverflowError) as exc:
            return f"{pin.__name__}: {exc}"[:300]
    return None
