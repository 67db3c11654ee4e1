"""RMSNorm backward on the GPU against the CPU oracle (the exact gradients).

Bar (tests/compare.py, check_gradient): each gradient element within 1 ulp of
bf16/fp16 (|difference| <= 1e-6 near zero; fp32 rtol = atol = 1e-6) of the
exact value, or within 2^-16 of the magnitude of the terms its fp32
evaluation rounds (cancellation in dx = rho (g - c x), the sums behind c and
dw); dx at least 99% bit-identical on large 16-bit cases.  Cases: the
headline shape, edge and ragged shapes in all dtypes (vector and generic
paths), unaligned buffers, dw off, a single row, every compiled plan (dx
bit-identical across vector plans), batch invariance of dx, graph replays.
"""
import pytest
import torch

import oracle
import rmsnorm_row_normalisation_amd as ks
import workloads
from compare import backward_magnitudes as magnitudes
from compare import check_bitexact, check_gradient
from gpu_cases import require_gpu, say

pytestmark = pytest.mark.gpu
DTYPES = ["bfloat16", "float16", "float32"]


@pytest.fixture(autouse=True)
def _gpu():
    require_gpu()


def _dev(t, offset):
    if offset == 0:
        return t.cuda()
    buf = torch.empty(t.numel() + offset, dtype=t.dtype, device="cuda")
    v = buf[offset:].view(t.shape)
    v.copy_(t.cuda())
    return v


def run(dy, x, w, eps, plan=None, offset=0, weight_grad=True):
    dxo = _dev(torch.empty_like(x), offset) if offset else None
    gx, gw = ks.rms_norm_backward(_dev(dy, offset), _dev(x, offset), _dev(w, offset), eps, plan=plan,
                                  weight_grad=weight_grad, dx=dxo)
    torch.cuda.synchronize()
    return gx.cpu(), (gw.cpu() if gw is not None else None)


def check(name, dy, x, w, eps, plan=None, offset=0, weight_grad=True):
    say("backward", name, tuple(x.shape), x.dtype, plan.as_dict() if plan is not None else "policy", offset)
    gx, gw = run(dy, x, w, eps, plan, offset, weight_grad)
    rx, rw = oracle.rms_norm_backward(dy, x, w, eps)
    mdx, mdw = magnitudes(dy, x, w, eps)
    st = check_gradient(gx, rx, mdx, 0.99 if gx.numel() >= 20000 else None)
    if weight_grad:
        check_gradient(gw, rw, mdw)
    return st, gx, gw


def test_workload():
    wl = workloads.WORKLOADS["B1"]
    inp = workloads.make_inputs(wl)
    st, _, _ = check("B1", inp["residual"], inp["x"], inp["weight"], wl.eps)
    say("B1", st)


SHAPES = [(5,), (2, 3, 5), (3, 1000), (512, 1024), (7, 1023), (300, 4096), (2, 8200), (3, 16384), (2, 32768),
          (2, 40000), (1000, 64)]


@pytest.mark.parametrize("dtype", DTYPES)
@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: "x".join(map(str, s)))
def test_shapes(shape, dtype):
    inp = workloads.random_case(shape, dtype, seed=sum(shape) + 11, residual=workloads.normal(0, 1))
    check("shape", inp["residual"], inp["x"], inp["weight"], 1e-6)


@pytest.mark.parametrize("dtype", DTYPES)
def test_unaligned_no_dw_and_empty(dtype):
    inp = workloads.random_case((37, 4096), dtype, seed=91)
    check("offset", inp["residual"], inp["x"], inp["weight"], 1e-5, offset=1)
    gx, gw = run(inp["residual"], inp["x"], inp["weight"], 1e-5, weight_grad=False)
    assert gw is None
    rx, _ = oracle.rms_norm_backward(inp["residual"], inp["x"], inp["weight"], 1e-5)
    check_gradient(gx, rx, magnitudes(inp["residual"], inp["x"], inp["weight"], 1e-5)[0])
    e = torch.empty(0, 64, dtype=workloads.DTYPES[dtype], device="cuda")
    w = torch.ones(64, dtype=e.dtype, device="cuda")
    ex, ew = ks.rms_norm_backward(e, e, w)
    torch.cuda.synchronize()
    assert ex.shape == (0, 64) and bool((ew.cpu() == 0).all())


def _vector_plans(hidden, es):
    """Every compiled vector plan that covers the row: 1024-thread workgroups with
    up to 3 (fp32) or 2 pieces per lane, 512-thread ones with up to 4."""
    nvec = hidden * es // 16
    out = []
    for block, maxv in ((1024, 3 if es == 4 else 2), (512, 4)):
        tpr = 8
        while tpr <= block:
            for vpt in range(1, maxv + 1):
                if tpr * vpt >= nvec:
                    out.append(ks.Plan(path=0, threads_per_row=tpr, vectors_per_thread=vpt, elems_per_access=16 // es,
                                       rows_per_block=block // tpr, block_threads=block, load_nt=1, store_nt=1))
            tpr *= 2
    return out


@pytest.mark.parametrize("dtype,hidden", [("bfloat16", 4096), ("float16", 1536), ("float32", 1000)])
def test_every_plan(dtype, hidden):
    """dx is the same bits for every vector plan; dw meets the bar for every plan."""
    inp = workloads.random_case((600, hidden), dtype, seed=hidden + 5)
    dy, x, w = inp["residual"], inp["x"], inp["weight"]
    rx, rw = oracle.rms_norm_backward(dy, x, w, 1e-6)
    mdx, mdw = magnitudes(dy, x, w, 1e-6)
    first = None
    plans = _vector_plans(hidden, x.element_size())
    assert len(plans) >= 4
    for plan in plans:
        gx, gw = run(dy, x, w, 1e-6, plan)
        check_gradient(gx, rx, mdx, 0.99)
        check_gradient(gw, rw, mdw)
        if first is None:
            first = gx
        else:
            check_bitexact(gx, first)
    es = x.element_size()
    for t in (8, 64, 256, 1024):
        for epa in (1, 16 // es):
            block = 1024 if t == 1024 else 256
            plan = ks.Plan(path=1, threads_per_row=t, vectors_per_thread=0, elems_per_access=epa,
                           rows_per_block=block // t, block_threads=block)
            gx, gw = run(dy, x, w, 1e-6, plan)
            check_gradient(gx, rx, mdx, 0.99)
            check_gradient(gw, rw, mdw)


POLICY_CASES = [("bfloat16", 4096, 2048), ("bfloat16", 2048, 4096), ("bfloat16", 1024, 64), ("float16", 8192, 512),
                ("float32", 2048, 2048), ("float32", 8192, 256)]


@pytest.mark.parametrize("dtype,hidden,rows", POLICY_CASES, ids=[f"{d}-{r}x{h}" for d, h, r in POLICY_CASES])
def test_policy_plans_at_full_size(dtype, hidden, rows):
    """The policy's plans of each kind (one piece per lane on 512 threads, teams
    of up to 128 lanes with up to 4 pieces, 512 lanes x 2 or 4) at full size:
    both gradients against the oracle, and dx the same bits as with the
    fewest lanes on 1024 threads."""
    inp = workloads.random_case((rows, hidden), dtype, seed=rows + 7 * hidden)
    dy, x, w = inp["residual"], inp["x"], inp["weight"]
    es = x.element_size()
    nvec = hidden * es // 16
    p = ks.get_plan("rms_norm_backward", x.dtype, hidden, rows, compute_units=256)
    assert p.block_threads == 512, p.as_dict()
    st, gx, _ = check(f"policy {dtype}", dy, x, w, 1e-6, plan=p)
    say("backward policy plan", dtype, rows, hidden, p.as_dict(), st)
    maxv = 3 if es == 4 else 2
    tpr = 8
    while tpr * maxv < nvec:
        tpr *= 2
    q = ks.Plan(path=0, threads_per_row=tpr, vectors_per_thread=-(-nvec // tpr), elems_per_access=16 // es,
                rows_per_block=1024 // tpr, block_threads=1024, load_nt=1, store_nt=1)
    gx2, _ = run(dy, x, w, 1e-6, q)
    check_bitexact(gx, gx2)


def test_dx_batch_invariance_and_dw_determinism():
    wl = workloads.WORKLOADS["B1"]
    inp = workloads.make_inputs(wl, rows=700)
    dy, x, w = inp["residual"], inp["x"], inp["weight"]
    gx, gw = run(dy, x, w, wl.eps)
    for rows in (1, 3, 64):
        sx, _ = run(dy[:rows].contiguous(), x[:rows].contiguous(), w, wl.eps)
        check_bitexact(sx, gx[:rows])
    gx2, gw2 = run(dy, x, w, wl.eps)
    check_bitexact(gx2, gx)
    check_bitexact(gw2, gw)


def test_graph_replays_match_eager():
    wl = workloads.WORKLOADS["B1"]
    inp = workloads.make_inputs(wl)
    dy, x, w = inp["residual"].cuda(), inp["x"].cuda(), inp["weight"].cuda()
    ws = torch.empty(ks.ks_rms_norm_backward_workspace_size(wl.rows, wl.hidden), dtype=torch.uint8, device="cuda")
    dx, dw = torch.empty_like(x), torch.empty_like(w)
    ks.rms_norm_backward(dy, x, w, wl.eps, workspace=ws, dx=dx, dweight=dw)
    torch.cuda.synchronize()
    ex, ew = dx.clone(), dw.clone()
    s = torch.cuda.Stream()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        ks.rms_norm_backward(dy, x, w, wl.eps, workspace=ws, dx=dx, dweight=dw)
    for _ in range(4):
        dx.zero_()
        dw.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        check_bitexact(dx.cpu(), ex.cpu())
        check_bitexact(dw.cpu(), ew.cpu())


@pytest.mark.parametrize("dtype", ["bfloat16", "float32"])
def test_autograd_wrapper(dtype):
    """rms_norm_autograd: the forward matches rms_norm and the gradients that
    reach x and weight are the backward's, checked against the oracle."""
    inp = workloads.random_case((64, 1024), dtype, seed=123)
    x = inp["x"].cuda().requires_grad_()
    w = inp["weight"].cuda().requires_grad_()
    dy = inp["residual"]
    y = ks.rms_norm_autograd(x, w, 1e-6)
    check_bitexact(y.detach().cpu(), ks.rms_norm(inp["x"].cuda(), inp["weight"].cuda(), 1e-6).cpu())
    y.backward(dy.cuda())
    torch.cuda.synchronize()
    rx, rw = oracle.rms_norm_backward(dy, inp["x"], inp["weight"], 1e-6)
    mdx, mdw = magnitudes(dy, inp["x"], inp["weight"], 1e-6)
    check_gradient(x.grad.cpu(), rx, mdx)
    check_gradient(w.grad.cpu(), rw, mdw)


@pytest.mark.parametrize("dtype", DTYPES)
@pytest.mark.parametrize("shape", [(2048, 4096), (300, 4096), (5, 1024), (700, 8)], ids=lambda s: "x".join(map(str, s)))
def test_workspace_alignment(shape, dtype):
    """A workspace only 4-byte aligned (4 bytes into an allocation) gives the
    gradients a 256-byte-aligned one gives, bit for bit, both within the bar,
    and every call the same."""
    inp = workloads.random_case(shape, dtype, seed=shape[0] + shape[1] + 23, residual=workloads.normal(0, 1))
    dy, x, w = (inp[k].cuda() for k in ("residual", "x", "weight"))
    need = ks.ks_rms_norm_backward_workspace_size(*shape)
    buf = torch.empty(need + 16, dtype=torch.uint8, device="cuda")
    rx, rw = oracle.rms_norm_backward(inp["residual"], inp["x"], inp["weight"], 1e-5)
    mdx, mdw = magnitudes(inp["residual"], inp["x"], inp["weight"], 1e-5)
    outs = []
    for off in (0, 4, 0, 4):
        say("backward workspace", shape, dtype, "offset", off)
        gx, gw = ks.rms_norm_backward(dy, x, w, 1e-5, workspace=buf[off:off + need])
        torch.cuda.synchronize()
        outs.append((gx.cpu(), gw.cpu()))
    check_gradient(outs[0][0], rx, mdx, 0.99 if outs[0][0].numel() >= 20000 else None)
    check_gradient(outs[0][1], rw, mdw)
    for gx, gw in outs[1:]:
        check_bitexact(gx, outs[0][0])
        check_bitexact(gw, outs[0][1])
