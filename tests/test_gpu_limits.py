"""The widest row the C ABI accepts (hidden = 2^24: 32 MiB rows in 16-bit
dtypes, 64 MiB in fp32) through every operation, against the CPU oracle
element by element at the bars of the other parity tests (tests/compare.py).

Rows this wide take the generic path (one 1024-lane team per row, a lane
summing 2^14 elements in batches with a compensated running sum), or the
split path for softmax with a workspace.  Two rows per case keep the oracle
within seconds.
"""
import pytest
import torch

import oracle
import rmsnorm_row_normalisation_amd as ks
import workloads
from compare import backward_magnitudes as magnitudes
from compare import check_bitexact, check_gradient, check_normalised
from gpu_cases import require_gpu, say

pytestmark = pytest.mark.gpu
H = 1 << 24
ROWS = 2


@pytest.fixture(autouse=True)
def _gpu():
    require_gpu()


def inputs(dtype: str, seed: int) -> dict:
    return workloads.random_case((ROWS, H), dtype, seed=seed, x=workloads.normal(0, 2))


@pytest.mark.parametrize("dtype", ["bfloat16", "float32"])
def test_rms_norm_forms(dtype):
    inp = inputs(dtype, 24)
    x, r, w = inp["x"], inp["residual"], inp["weight"]
    xd, rd, wd = x.cuda(), r.cuda(), w.cuda()
    say("limits rms_norm", dtype, ks.get_plan("rms_norm", x.dtype, H, ROWS).as_dict())
    y = ks.rms_norm(xd, wd, 1e-6)
    torch.cuda.synchronize()
    say(check_normalised(y.cpu(), oracle.rms_norm(x, w, 1e-6)))
    del y
    say("limits rms_norm_residual", dtype)
    z = ks.rms_norm_residual(xd, rd, wd, 1e-6)
    torch.cuda.synchronize()
    say(check_normalised(z.cpu(), oracle.rms_norm_residual(x, r, w, 1e-6)))
    del z
    say("limits fused_add_rms_norm", dtype)
    ks.fused_add_rms_norm(xd, rd, wd, 1e-6)
    torch.cuda.synchronize()
    ox, orr = oracle.fused_add_rms_norm(x, r, w, 1e-6)
    check_bitexact(rd.cpu(), orr)
    say(check_normalised(xd.cpu(), ox))


@pytest.mark.parametrize("split", [True, False])
@pytest.mark.parametrize("dtype", ["bfloat16", "float32"])
def test_softmax(dtype, split):
    x = inputs(dtype, 25)["x"]
    say("limits softmax", dtype, ks.get_plan("softmax", x.dtype, H, ROWS, workspace=split).as_dict())
    y = ks.softmax(x.cuda(), split=split)
    torch.cuda.synchronize()
    say(check_normalised(y.cpu(), oracle.softmax(x)))


def test_silu_and_mul():
    x = workloads.random_case((ROWS, 2 * H), "bfloat16", seed=26, x=workloads.normal(0, 2))["x"]
    say("limits silu_and_mul", ks.get_plan("silu_and_mul", x.dtype, H, ROWS).as_dict())
    y = ks.silu_and_mul(x.cuda())
    torch.cuda.synchronize()
    say(check_normalised(y.cpu(), oracle.silu_and_mul(x)))


@pytest.mark.parametrize("dtype", ["bfloat16", "float32"])
def test_backward(dtype):
    inp = inputs(dtype, 27)
    dy, x, w = inp["residual"], inp["x"], inp["weight"]
    say("limits rms_norm_backward", dtype, ks.get_plan("rms_norm_backward", x.dtype, H, ROWS).as_dict())
    gx, gw = ks.rms_norm_backward(dy.cuda(), x.cuda(), w.cuda(), 1e-6)
    torch.cuda.synchronize()
    rx, rw = oracle.rms_norm_backward(dy, x, w, 1e-6)
    mdx, mdw = magnitudes(dy, x, w, 1e-6)
    say(check_gradient(gx.cpu(), rx, mdx))
    say(check_gradient(gw.cpu(), rw, mdw))


@pytest.mark.parametrize("op", ["rms_norm", "fused_add_rms_norm", "softmax"])
def test_batches_beyond_one_launch(op):
    """Batches whose grid would pass 2^31 work-items go out in slices of rows:
    2^29 + 4099 rows of 8 bf16 elements (8 GiB per tensor; 16-byte rows, 32
    rows per 256-thread workgroup, so slices of 2^28 rows, and more than 2^32
    work-items in all), checked against the oracle on the rows around the
    slice boundaries, the first and last rows and 2000 sampled rows."""
    rows, hidden = (1 << 29) + 4099, 8
    g = torch.Generator(device="cuda").manual_seed(28)
    x = torch.randn(rows, hidden, dtype=torch.bfloat16, device="cuda", generator=g)
    w = workloads.random_case((1, hidden), "bfloat16", seed=29)["weight"]
    edges = [0, 1, (1 << 28) - 1, 1 << 28, (1 << 28) + 1, (1 << 29) - 1, 1 << 29, (1 << 29) + 1, rows - 1]
    pick = torch.cat([torch.tensor(edges),
                      torch.randint(0, rows, (2000,), generator=torch.Generator().manual_seed(30))]).cuda()
    xs = x[pick].cpu()
    say("limits slices", op, rows, hidden, ks.get_plan(op, torch.bfloat16, hidden, rows).as_dict())
    if op == "rms_norm":
        y = ks.rms_norm(x, w.cuda(), 1e-6)
        torch.cuda.synchronize()
        say(check_normalised(y[pick].cpu(), oracle.rms_norm(xs, w, 1e-6)))
    elif op == "softmax":
        y = ks.softmax(x)
        torch.cuda.synchronize()
        say(check_normalised(y[pick].cpu(), oracle.softmax(xs)))
    else:
        r = torch.randn(rows, hidden, dtype=torch.bfloat16, device="cuda", generator=g)
        rs = r[pick].cpu()
        ks.fused_add_rms_norm(x, r, w.cuda(), 1e-6)
        torch.cuda.synchronize()
        ox, orr = oracle.fused_add_rms_norm(xs, rs, w, 1e-6)
        check_bitexact(r[pick].cpu(), orr)
        say(check_normalised(x[pick].cpu(), ox))
