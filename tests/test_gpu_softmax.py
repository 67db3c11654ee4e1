"""Softmax on the GPU against the CPU oracle, element by element.

Bar: within 1 ulp of bf16/fp16 (|difference| <= 1e-6 near zero) and at least
99.9% bit-identical on large cases; fp32 within rtol = atol = 1e-6.  Cases:
the kernscope softmax measurement shapes (512 rows of 1024, 128 and 8192
bf16), its 65536-column fp16 accumulation case, the 2048x4096 bf16 batch,
widths 1..32776 in every dtype (vector and generic paths, ragged tails),
unaligned offset views, empty batches, large logits, the page's non-finite
row rules, every compiled plan (vector plans bit-identical), batch
invariance, in-place calls and graph replays.
"""
import pytest
import torch

import oracle
import rmsnorm_row_normalisation_amd as ks
import workloads
from compare import check_bitexact, check_normalised
from gpu_cases import HINTS, require_gpu, say

pytestmark = pytest.mark.gpu
DTYPES = ["bfloat16", "float16", "float32"]
INF, NAN = float("inf"), float("nan")


@pytest.fixture(autouse=True)
def _gpu():
    require_gpu()


def gpu_softmax(x: torch.Tensor, plan=None, offset: int = 0, inplace: bool = False) -> torch.Tensor:
    if offset:
        buf = torch.empty(x.numel() + offset, dtype=x.dtype, device="cuda")
        xd = buf[offset:].view(x.shape)
        xd.copy_(x.cuda())
        obuf = torch.empty(x.numel() + offset, dtype=x.dtype, device="cuda")
        out = ks.softmax(xd, out=obuf[offset:].view(x.shape), plan=plan)
    elif inplace:
        xd = x.cuda()
        out = ks.softmax(xd, out=xd, plan=plan)
    else:
        out = ks.softmax(x.cuda(), plan=plan)
    torch.cuda.synchronize()
    return out.cpu()


def check(name, x, plan=None, offset=0, exact=None, inplace=False):
    say("softmax", name, tuple(x.shape), x.dtype, plan.as_dict() if plan is not None else "policy", offset)
    got = gpu_softmax(x, plan, offset, inplace)
    ref = oracle.softmax(x)
    if exact is None:
        exact = got.numel() >= 20000
    return check_normalised(got, ref, 0.999 if exact else None)


@pytest.mark.parametrize("name", ["X1", "X2", "X3", "X4", "X5"])
def test_workloads(name):
    wl = workloads.WORKLOADS[name]
    x = workloads.make_inputs(wl)["x"]
    say(name, check(name, x))


SHAPES = [(1, 1), (3, 1), (5, 7), (4, 8), (2, 3, 40), (7, 1000), (3, 1023), (9, 1024), (5, 4095), (64, 4096),
          (2, 16384), (4, 32768), (2, 32776), (2, 70000)]


@pytest.mark.parametrize("dtype", DTYPES)
@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: "x".join(map(str, s)))
def test_shapes(shape, dtype):
    x = workloads.random_case(shape, dtype, seed=sum(shape) + 7, x=workloads.normal(0, 2))["x"]
    check("shape", x)


@pytest.mark.parametrize("dtype", DTYPES)
def test_offset_views_inplace_and_empty(dtype):
    x = workloads.random_case((37, 1024), dtype, seed=5)["x"]
    check("offset", x, offset=1)
    check("inplace", x, inplace=True)
    e = torch.empty(0, 16, dtype=workloads.DTYPES[dtype], device="cuda")
    assert ks.softmax(e).shape == (0, 16)
    e3 = torch.empty(3, 0, 16, dtype=workloads.DTYPES[dtype], device="cuda")
    assert ks.softmax(e3).shape == (3, 0, 16)


@pytest.mark.parametrize("dtype", DTYPES)
def test_large_logits(dtype):
    """Logits far beyond exp's range: only differences matter."""
    rows = []
    g = torch.Generator().manual_seed(11)
    for scale, shift in ((10, 0), (100, 1000), (1000, -3000), (1e4, 0), (3e4, 3e4)):
        rows.append(torch.randn(2048, generator=g) * scale + shift)
    x = torch.stack(rows).to(workloads.DTYPES[dtype])
    x = torch.clamp(x.float(), -65000, 65000).to(x.dtype) if dtype == "float16" else x
    check("large", x.contiguous())


@pytest.mark.parametrize("dtype", DTYPES)
@pytest.mark.parametrize("hidden", [4, 1024, 40000])
def test_nonfinite_rows(dtype, hidden):
    """NaN or +inf anywhere, or only -inf: NaN everywhere in the row; -inf
    entries elsewhere: 0.  hidden 40000 in fp32/16-bit takes the generic path."""
    dt = workloads.DTYPES[dtype]
    x = workloads.random_case((8, hidden), dtype, seed=hidden)["x"].float()
    x[0, hidden // 2] = NAN
    x[1, hidden - 1] = INF
    x[2, :] = -INF
    x[3, 0] = INF
    x[3, 1 % hidden] = -INF
    x[4, ::3] = -INF
    x[5, :] = NAN
    x[6, 1:] = -INF
    x = x.to(dt).contiguous()
    got = gpu_softmax(x)
    ref = oracle.softmax(x)
    assert bool((torch.isnan(got) == torch.isnan(ref)).all())
    assert bool(torch.isnan(got[:4]).all()) and bool(torch.isnan(got[5]).all())
    assert bool((got[4].float()[::3] == 0).all())
    assert float(got[6, 0]) == 1.0
    check_normalised(got, ref)


def _vector_plans(hidden: int, es: int) -> list:
    plans = []
    tpr = 8
    while tpr <= 1024:
        maxv = 8
        for vpt in range(1, maxv + 1):
            if tpr * vpt * 16 >= hidden * es and (hidden * es) % 16 == 0:
                block = max(256, tpr)
                for lnt, snt, wl in HINTS:
                    if not wl:
                        plans.append(ks.Plan(path=0, threads_per_row=tpr, vectors_per_thread=vpt,
                                             elems_per_access=16 // es, rows_per_block=block // tpr,
                                             block_threads=block, load_nt=lnt, store_nt=snt))
        tpr *= 2
    return plans


@pytest.mark.parametrize("dtype,hidden", [("bfloat16", 4096), ("float16", 1536), ("float32", 1000), ("bfloat16", 72)])
def test_every_plan(dtype, hidden):
    """Every compiled vector plan gives the same bits; generic plans meet the bar."""
    x = workloads.random_case((70, hidden), dtype, seed=hidden)["x"]
    ref = oracle.softmax(x)
    es = x.element_size()
    vplans = _vector_plans(hidden, es)
    assert len(vplans) > 3
    first = None
    for plan in vplans:
        got = gpu_softmax(x, plan)
        check_normalised(got, ref, 0.999 if got.numel() >= 20000 else None)
        if first is None:
            first = got
        else:
            check_bitexact(got, first)
    for t in (8, 64, 256, 1024):
        for epa in (1, 16 // es):
            block = 1024 if t == 1024 else 256
            plan = ks.Plan(path=1, threads_per_row=t, vectors_per_thread=0, elems_per_access=epa,
                           rows_per_block=block // t, block_threads=block)
            check_normalised(gpu_softmax(x, plan), ref, 0.999 if x.numel() >= 20000 else None)


def test_batch_invariance():
    """A row's result does not depend on the batch it is in (vector path)."""
    x = workloads.make_inputs(workloads.WORKLOADS["X5"])["x"]
    full = gpu_softmax(x)
    for rows in (1, 3, 64, 700):
        check_bitexact(gpu_softmax(x[:rows].contiguous()), full[:rows])


def test_graph_replays_match_eager():
    x = workloads.make_inputs(workloads.WORKLOADS["X1"])["x"].cuda()
    out = ks.softmax(x)
    torch.cuda.synchronize()
    eager = out.clone()
    s = torch.cuda.Stream()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        ks.softmax(x, out=out)
    for rep in range(4):
        out.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        check_bitexact(out.cpu(), eager.cpu())
