"""Seeded random cases across every operation: op, dtype, batch shape, row
width (odd, 16-byte multiples, past the vector path) and buffer alignment are
drawn from a fixed generator, each case is run through the C ABI and checked
against the CPU oracle with that operation's bar.  The draws are fixed, so a
failure names a reproducible case (printed before it runs)."""
import numpy as np
import pytest
import torch

import oracle
import rmsnorm_row_normalisation_amd as ks
import workloads
from compare import backward_magnitudes, check_bitexact, check_gradient, check_normalised
from gpu_cases import require_gpu, say

pytestmark = pytest.mark.gpu

OPS = ["rms_norm", "fused_add_rms_norm", "rms_norm_residual", "rms_norm_backward", "silu_and_mul", "softmax"]
DTYPES = ["bfloat16", "float16", "float32"]
HIDDEN = [1, 2, 3, 8, 17, 64, 96, 127, 512, 1000, 1536, 2047, 2880, 4096, 5120, 8192, 12288, 16384, 24576,
          32768, 40000, 65536, 128256]
ROWS = [1, 2, 3, 7, 33, 100, 256, 513, 2048, 4100]


def draw(i: int):
    g = np.random.default_rng(2024 + i)
    op = OPS[i % len(OPS)]
    dtype = DTYPES[int(g.integers(len(DTYPES)))]
    hidden = HIDDEN[int(g.integers(len(HIDDEN)))]
    if op == "silu_and_mul":
        hidden *= 2
    rows = ROWS[int(g.integers(len(ROWS)))]
    rows = max(1, min(rows, (1 << 21) // hidden))
    lead = (rows,) if g.random() < 0.7 else (1, rows)
    offset = int(g.integers(2)) if g.random() < 0.3 else 0
    eps = [1e-6, 1e-5, 1e-2][int(g.integers(3))]
    return op, dtype, (*lead, hidden), offset, eps, 3000 + i


def _dev(t: torch.Tensor, offset: int) -> torch.Tensor:
    if offset == 0:
        return t.cuda()
    buf = torch.empty(t.numel() + offset, dtype=t.dtype, device="cuda")
    v = buf[offset:].view(t.shape)
    v.copy_(t.cuda())
    return v


@pytest.fixture(autouse=True)
def _gpu():
    require_gpu()


@pytest.mark.parametrize("i", range(120))
def test_random_case(i):
    op, dtype, shape, offset, eps, seed = draw(i)
    say("random", i, op, dtype, shape, f"offset={offset}", f"eps={eps}")
    inp = workloads.random_case(shape, dtype, seed, x=workloads.normal(0, 2), residual=workloads.normal(0, 1))
    x, r, w = inp["x"], inp["residual"], inp["weight"]
    exact = 0.999 if x.numel() >= 20000 else None
    if op == "rms_norm":
        y = ks.rms_norm(_dev(x, offset), _dev(w, offset), eps)
        check_normalised(y.cpu(), oracle.rms_norm(x, w, eps), exact)
    elif op == "fused_add_rms_norm":
        xd, rd = _dev(x, offset), _dev(r, offset)
        ks.fused_add_rms_norm(xd, rd, _dev(w, offset), eps)
        torch.cuda.synchronize()
        ox, orr = oracle.fused_add_rms_norm(x, r, w, eps)
        check_bitexact(rd.cpu(), orr)
        check_normalised(xd.cpu(), ox, exact)
    elif op == "rms_norm_residual":
        y = ks.rms_norm_residual(_dev(x, offset), _dev(r, offset), _dev(w, offset), eps)
        check_normalised(y.cpu(), oracle.rms_norm_residual(x, r, w, eps), exact)
    elif op == "rms_norm_backward":
        gx, gw = ks.rms_norm_backward(_dev(r, offset), _dev(x, offset), _dev(w, offset), eps)
        torch.cuda.synchronize()
        rx, rw = oracle.rms_norm_backward(r, x, w, eps)
        mdx, mdw = backward_magnitudes(r, x, w, eps)
        check_gradient(gx.cpu(), rx, mdx, 0.99 if x.numel() >= 20000 else None)
        check_gradient(gw.cpu(), rw, mdw)
    elif op == "silu_and_mul":
        y = ks.silu_and_mul(_dev(x, offset))
        check_normalised(y.cpu(), oracle.silu_and_mul(x), 0.999 if y.numel() >= 20000 else None)
    else:
        y = ks.softmax(_dev(x, offset))
        check_normalised(y.cpu(), oracle.softmax(x), exact)
    torch.cuda.synchronize()
