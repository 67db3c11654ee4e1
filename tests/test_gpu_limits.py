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
