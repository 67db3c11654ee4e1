"""Parity of the HIP path with the CPU oracle, element by element, on cuda:0.

Bar: the fused residual output is bit-exact; normalised outputs are within
1 ulp of the dtype (|difference| <= 1e-6 near zero; fp32 within rtol = atol
= 1e-6) and, on large cases, identical on at least 99.9% of elements.

Cases: every benchmark workload of the operator pages (128x1024, 512x4096,
2048x4096 in fp16 with outliers and in bf16, decode 4x1536 and 1x8192, and the
large prefills 32768x8192 and 8192x16384, every row checked in chunks),
the kernscope edge shapes, ragged row counts, unaligned buffers, every
compiled launch plan, and the invariants that hold at any size.
"""
import numpy as np
import pytest
import torch

import oracle
import rmsnorm_row_normalisation_amd as ks
import workloads
from compare import check_bitexact, check_normalised, ulp_distance
from gpu_cases import all_plans, check_case, check_outputs, gpu_run, oracle_run, require_gpu, say

pytestmark = pytest.mark.gpu

DTYPES = ["bfloat16", "float16", "float32"]


@pytest.fixture(autouse=True)
def _gpu():
    require_gpu()


# ---------------------------------------------------------------------------
# the benchmark workloads at full size
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("name", ["C1", "C2", "C3", "C3b", "C4a", "C4b"])
def test_workload_full(name):
    wl = workloads.WORKLOADS[name]
    inp = workloads.make_inputs(wl)
    for op in wl.ops:
        st = check_case(name, op, inp, wl.eps)
        say(name, op, st)


@pytest.mark.parametrize("name", ["C5f", "C5r"])
def test_workload_large_full(name):
    """Full-size launch; every row checked against the oracle, in chunks of rows
    (the bar per element, the exact-match rate over the whole batch)."""
    wl = workloads.WORKLOADS[name]
    inp = workloads.make_inputs(wl)
    for op in wl.ops:
        say(name, op, "full launch", (wl.rows, wl.hidden))
        y, r = gpu_run(op, inp, wl.eps)
        exact = total = worst = 0
        for r0 in range(0, wl.rows, LARGE_CHUNK_ROWS):
            sl = slice(r0, min(wl.rows, r0 + LARGE_CHUNK_ROWS))
            sub = {k: (v[sl] if v.dim() == 2 else v) for k, v in inp.items()}
            ref = oracle_run(op, sub, wl.eps)
            st = check_outputs(op, (y[sl], r[sl] if r is not None else None), ref, exact_rate=False)
            exact += round(st.exact_rate * st.n)
            total += st.n
            worst = max(worst, st.max_ulp)
        say(name, op, f"rows {wl.rows}: max ulp {worst}, exact {exact / total:.6f}")
        assert total == wl.rows * wl.hidden
        assert exact / total >= 0.999


LARGE_CHUNK_ROWS = 2048


# ---------------------------------------------------------------------------
# edge shapes from the kernscope test list, odd and wide hidden sizes, ragged
# row counts (not multiples of any rows-per-workgroup)
# ---------------------------------------------------------------------------
EDGE_SHAPES = [(5,), (2, 3, 5), (3, 1000), (512, 1024), (1, 1), (3, 2), (7, 3), (9, 8), (5, 63), (5, 64),
               (13, 65), (3, 127), (17, 1001), (130, 1536), (33, 2880), (7, 4095), (7, 4096), (7, 4097),
               (3, 5120), (5, 8191), (3, 12288), (2, 20000), (3, 32768), (2, 40000), (2, 65536), (1, 70000)]


@pytest.mark.parametrize("dtype", DTYPES)
@pytest.mark.parametrize("shape", EDGE_SHAPES, ids=lambda s: "x".join(map(str, s)))
def test_edge_shapes(shape, dtype):
    inp = workloads.random_case(shape, dtype, seed=sum(shape) + len(dtype))
    for op in ("rms_norm", "fused_add_rms_norm"):
        check_case("edge", op, inp, 1e-6)


@pytest.mark.parametrize("rows", [1, 2, 3, 5, 17, 63, 129, 1000, 4097])
def test_ragged_row_counts(rows):
    inp = workloads.random_case((rows, 4096), "bfloat16", seed=rows)
    for op in ("rms_norm", "fused_add_rms_norm"):
        check_case("ragged", op, inp, 1e-5)


@pytest.mark.parametrize("dtype", DTYPES)
@pytest.mark.parametrize("hidden", [1000, 1024, 4096, 4097])
def test_unaligned_buffers(hidden, dtype):
    """Tensors starting one element into an allocation (offset views): the generic path."""
    inp = workloads.random_case((37, hidden), dtype, seed=hidden + 5)
    for op in ("rms_norm", "fused_add_rms_norm"):
        check_case("unaligned", op, inp, 1e-6, offset=1)


def test_empty_and_zero():
    w = torch.ones(64, dtype=torch.bfloat16, device="cuda")
    e = torch.empty(0, 64, dtype=torch.bfloat16, device="cuda")
    assert ks.rms_norm(e, w).shape == (0, 64)
    ks.fused_add_rms_norm(e, e.clone(), w)
    e3 = torch.empty(4, 0, 64, dtype=torch.bfloat16, device="cuda")
    assert ks.rms_norm(e3, w).shape == (4, 0, 64)
    for dtype in (torch.bfloat16, torch.float16, torch.float32):
        x = torch.zeros(33, 4096, dtype=dtype, device="cuda")
        y = ks.rms_norm(x, torch.ones(4096, dtype=dtype, device="cuda"))
        torch.cuda.synchronize()
        assert bool((y == 0).all())


# ---------------------------------------------------------------------------
# every compiled plan gives the oracle's result
# ---------------------------------------------------------------------------
PLAN_CASES = [("bfloat16", 4096), ("float16", 1536), ("float32", 2048), ("bfloat16", 8192), ("bfloat16", 16384),
              ("bfloat16", 264)]


@pytest.mark.parametrize("dtype,hidden", PLAN_CASES, ids=[f"{d}-{h}" for d, h in PLAN_CASES])
def test_every_plan(dtype, hidden):
    """Every compiled plan meets the oracle bar, and every vector plan gives the
    bitwise same result (the summation order does not depend on the launch shape)."""
    inp = workloads.random_case((70, hidden), dtype, seed=hidden)
    refs = {op: oracle_run(op, inp, 1e-6) for op in ("rms_norm", "fused_add_rms_norm")}
    plans = all_plans(inp["x"].dtype, hidden)
    assert len(plans) >= 8
    first_vector = {}
    for plan in plans:
        for op in ("rms_norm", "fused_add_rms_norm"):
            say("plan", op, dtype, hidden, plan.as_dict())
            got = gpu_run(op, inp, 1e-6, plan=plan)
            check_outputs(op, got, refs[op], exact_rate=True)
            if plan.path == 0:
                if op not in first_vector:
                    first_vector[op] = got
                else:
                    check_bitexact(got[0], first_vector[op][0])


SIXTEEN_CASES = [("float32", 4096, 2048), ("bfloat16", 8192, 1856), ("float16", 16384, 960)]


@pytest.mark.parametrize("dtype,hidden,rows", SIXTEEN_CASES, ids=[f"{d}-{r}x{h}" for d, h, r in SIXTEEN_CASES])
def test_sixteen_piece_plans_at_full_size(dtype, hidden, rows):
    """The batches where the policy (on a whole MI355X) gives rms_norm and the
    fused form 16 pieces per lane: every row against the oracle, and the same
    bits as the 8-piece plans the policy gave these batches before."""
    inp = workloads.random_case((rows, hidden), dtype, seed=rows + hidden)
    dt = inp["x"].dtype
    es = inp["x"].element_size()
    nvec = hidden * es // 16
    tpr8 = 128 if nvec <= 1024 else 256
    for op in ("rms_norm", "fused_add_rms_norm"):
        p16 = ks.get_plan(op, dt, hidden, rows, compute_units=256)
        assert p16.vectors_per_thread == 16, p16.as_dict()
        p8 = ks.Plan(path=0, threads_per_row=tpr8, vectors_per_thread=8, elems_per_access=16 // es,
                     rows_per_block=256 // tpr8, block_threads=256, load_nt=1, store_nt=1, weight_lds=p16.weight_lds)
        say("sixteen pieces", op, dtype, rows, hidden, p16.as_dict())
        got16 = gpu_run(op, inp, 1e-6, plan=p16)
        got8 = gpu_run(op, inp, 1e-6, plan=p8)
        check_outputs(op, got16, oracle_run(op, inp, 1e-6), exact_rate=True)
        check_bitexact(got16[0], got8[0])
        if got16[1] is not None:
            check_bitexact(got16[1], got8[1])


HUGE_CASES = [("bfloat16", 8192, 8192), ("float32", 4096, 8192), ("float16", 16384, 8192)]


@pytest.mark.parametrize("dtype,hidden,rows", HUGE_CASES, ids=[f"{d}-{r}x{h}" for d, h, r in HUGE_CASES])
def test_large_batch_rms_plans_at_full_size(dtype, hidden, rows):
    """rms_norm from 8192 rows of 16 KiB (512 lanes x 2 pieces, weight in LDS)
    or 16-bit rows of 32 KiB (128 lanes x 16 pieces): every row against the
    oracle, in chunks, and the same bits as the large-batch plan of 4 pieces
    per lane that the policy gives one row fewer."""
    inp = workloads.random_case((rows, hidden), dtype, seed=rows ^ hidden)
    dt = inp["x"].dtype
    es = inp["x"].element_size()
    nvec = hidden * es // 16
    p = ks.get_plan("rms_norm", dt, hidden, rows, compute_units=256)
    assert (p.threads_per_row, p.vectors_per_thread) == ((512, 2) if nvec == 1024 else (128, 16)), p.as_dict()
    q = ks.get_plan("rms_norm", dt, hidden, rows - 1, compute_units=256)
    assert q.vectors_per_thread == 4, q.as_dict()
    say("large-batch rms plans", dtype, rows, hidden, p.as_dict(), q.as_dict())
    y, _ = gpu_run("rms_norm", inp, 1e-6, plan=p)
    y4, _ = gpu_run("rms_norm", inp, 1e-6, plan=q)
    check_bitexact(y, y4)
    exact = total = 0
    for r0 in range(0, rows, LARGE_CHUNK_ROWS):
        sl = slice(r0, min(rows, r0 + LARGE_CHUNK_ROWS))
        sub = {k: (v[sl] if v.dim() == 2 else v) for k, v in inp.items()}
        st = check_outputs("rms_norm", (y[sl], None), oracle_run("rms_norm", sub, 1e-6), exact_rate=False)
        exact += round(st.exact_rate * st.n)
        total += st.n
    assert total == rows * hidden
    if dtype != "float32":
        assert exact / total >= 0.999


# ---------------------------------------------------------------------------
# invariants that hold at any size
# ---------------------------------------------------------------------------
def test_constant_rows_closed_form():
    import pins

    for fmt, c, eps, h, expected, _margin in pins.read_constant_rows():
        dt = pins.DT[fmt]
        x = torch.full((3, h), c, dtype=dt)
        w = torch.ones(h, dtype=dt)
        want = pins._pattern_tensor(expected, dt, h).expand(3, h).contiguous()
        say("constant", fmt, c, eps, h)
        y, _ = gpu_run("rms_norm", {"x": x, "weight": w}, eps)
        half = torch.full((3, h), c / 2, dtype=dt)
        fx, fr = gpu_run("fused_add_rms_norm", {"x": half, "residual": half.clone(), "weight": w}, eps)
        check_bitexact(fr, x)
        if fmt == "float32":
            assert int(ulp_distance(y, want).max()) <= 4
            assert int(ulp_distance(fx, want).max()) <= 4
        else:
            check_bitexact(y, want)
            check_bitexact(fx, want)


def test_batch_invariance():
    """A row's result does not depend on the batch around it, although the plan's
    launch shape and memory hints may change with the batch size."""
    for dtype, hidden in (("bfloat16", 4096), ("float16", 1536), ("bfloat16", 16384), ("bfloat16", 1001)):
        inp = workloads.random_case((300, hidden), dtype, seed=9)
        full = {op: gpu_run(op, inp, 1e-6) for op in ("rms_norm", "fused_add_rms_norm")}
        for lo, hi in ((0, 1), (17, 18), (299, 300), (5, 12), (100, 227)):
            sub = {k: (v[lo:hi].contiguous() if v.dim() == 2 else v) for k, v in inp.items()}
            for op in ("rms_norm", "fused_add_rms_norm"):
                y, r = gpu_run(op, sub, 1e-6)
                check_bitexact(y, full[op][0][lo:hi])
                if r is not None:
                    check_bitexact(r, full[op][1][lo:hi])


def test_scaling_sign_and_zero_residual():
    for dtype in DTYPES:
        inp = workloads.random_case((64, 4096), dtype, seed=3)
        x = inp["x"]
        x = (torch.sign(x.float()) * x.float().abs().clamp_min(2.0 ** -6)).to(x.dtype)
        w, r = inp["weight"], inp["residual"]
        eps32 = float(np.float32(1e-6))
        y, _ = gpu_run("rms_norm", {"x": x, "weight": w}, 1e-6)
        ys, _ = gpu_run("rms_norm", {"x": (x.float() * 4).to(x.dtype), "weight": w}, eps32 * 16)
        check_bitexact(ys, y)
        yw, _ = gpu_run("rms_norm", {"x": x, "weight": (w.float() * 0.5).to(w.dtype)}, 1e-6)
        check_bitexact(yw, (y.float() * 0.5).to(y.dtype))
        yn, _ = gpu_run("rms_norm", {"x": -x, "weight": w}, 1e-6)
        check_bitexact(yn, -y)
        zx, zr = gpu_run("fused_add_rms_norm", {"x": x, "residual": torch.zeros_like(x), "weight": w}, 1e-6)
        check_bitexact(zr, x)
        check_bitexact(zx, y)
        fx, fr = gpu_run("fused_add_rms_norm", {"x": x, "residual": r, "weight": w}, 1e-6)
        check_bitexact(fr, (x.float() + r.float()).to(x.dtype))


def test_in_place_rms_norm_and_streams():
    inp = workloads.random_case((257, 4096), "bfloat16", seed=12)
    ref = oracle.rms_norm(inp["x"], inp["weight"], 1e-6)
    x = inp["x"].cuda()
    w = inp["weight"].cuda()
    out = ks.rms_norm(x, w, 1e-6, out=x)          # out == x: in place
    assert out.data_ptr() == x.data_ptr()
    torch.cuda.synchronize()
    check_normalised(x.cpu(), ref, 0.999)
    s = torch.cuda.Stream()
    got = gpu_run("rms_norm", inp, 1e-6, stream=s)
    check_normalised(got[0], ref, 0.999)


def test_special_values():
    """IEEE propagation (no fast-math, no flush to zero): an infinite element makes the
    row's scale zero, subnormal outputs survive, overflow goes to infinity."""
    h = 256
    for dtype in (torch.bfloat16, torch.float16, torch.float32):
        x = torch.randn(6, h, generator=torch.Generator().manual_seed(1)).to(dtype)
        w = torch.ones(h, dtype=dtype)
        x[0, 3] = float("inf")
        x[1, 7] = float("nan")
        x[2] = 0.0
        tiny = {torch.bfloat16: 1e-39, torch.float16: 1e-7, torch.float32: 1e-44}[dtype]
        w_tiny = torch.full((h,), tiny, dtype=dtype)
        for weight in (w, w_tiny):
            y, _ = gpu_run("rms_norm", {"x": x, "weight": weight}, 1e-6)
            ref = oracle.rms_norm(x, weight, 1e-6)
            assert bool((torch.isnan(y) == torch.isnan(ref)).all())
            check_normalised(y, ref)
        big = torch.full((2, h), {torch.bfloat16: 3e38, torch.float16: 60000.0, torch.float32: 3e38}[dtype],
                         dtype=dtype)
        bw = torch.full((h,), 4.0, dtype=dtype)
        fx, fr = gpu_run("fused_add_rms_norm", {"x": big, "residual": big.clone(), "weight": bw}, 1e-6)
        rx, rr = oracle.fused_add_rms_norm(big, big.clone(), bw, 1e-6)
        check_bitexact(fr, rr)
        check_normalised(fx, rx)


def test_graph_replays_match_eager():
    """The launches captured into a HIP graph give the eager result on every replay
    (inputs restored by eager copies between replays)."""
    wl = workloads.WORKLOADS["C2"]
    inp = workloads.make_inputs(wl)
    x0, r0, w = inp["x"].cuda(), inp["residual"].cuda(), inp["weight"].cuda()
    xr, out, xf, rf = x0.clone(), torch.empty_like(x0), x0.clone(), r0.clone()
    ks.rms_norm(xr, w, wl.eps, out=out)
    ks.fused_add_rms_norm(xf, rf, w, wl.eps)
    torch.cuda.synchronize()
    eager = (out.clone(), xf.clone(), rf.clone())
    s = torch.cuda.Stream()
    g = torch.cuda.CUDAGraph()
    xf.copy_(x0)
    rf.copy_(r0)
    out.zero_()
    torch.cuda.synchronize()
    with torch.cuda.graph(g, stream=s):
        ks.rms_norm(xr, w, wl.eps, out=out)
        ks.fused_add_rms_norm(xf, rf, w, wl.eps)
    for rep in range(4):
        out.zero_()
        xf.copy_(x0)
        rf.copy_(r0)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        say("graph replay", rep)
        for got, want in zip((out, xf, rf), eager):
            check_bitexact(got.cpu(), want.cpu())


def test_fp16_outputs_round_through_fp32():
    """The contract rounds (v * scale) * w to fp32 and then to the dtype.  Constant
    rows with exact sums make scale identical on both sides, so every output is
    RN16(RN32(t * w)) and must match the oracle bit for bit; with every fp16
    weight in [1, 2) and several eps values, dozens of positions differ from a
    single rounding RN16(t * w), which a fused multiply-convert would produce."""
    import numpy as np

    h = 1024
    w = torch.arange(0x3C00, 0x4000, dtype=torch.int32).to(torch.int16).view(torch.float16)   # all of [1, 2)
    cs = [m * 2.0 ** k for m in range(64, 128) for k in range(-8, 4)]   # <= 7 significant bits: exact sums
    cs = cs + [-c for c in cs[::7]]
    x = torch.tensor(cs, dtype=torch.float32)[:, None].expand(len(cs), h).to(torch.float16).contiguous()
    half = (x.float() / 2).to(torch.float16)
    c32 = np.array(cs, dtype=np.float32)
    wn = w.float().numpy()
    discriminating = 0
    for eps in (1e-3, 3e-3, 1e-2, 0.1, 0.37, 1.0):
        # host model of the pipeline: mean of h equal squares is exact, then fp32 steps
        d = (c32 * c32 + np.float32(eps)).astype(np.float32)
        scale = (1.0 / np.sqrt(d.astype(np.float64))).astype(np.float32)
        t = (c32 * scale).astype(np.float32)
        double = (t[:, None] * wn[None, :]).astype(np.float32).astype(np.float16)
        single = (t[:, None].astype(np.float64) * wn[None, :].astype(np.float64)).astype(np.float16)
        discriminating += int((double.view(np.uint16) != single.view(np.uint16)).sum())
        y, _ = gpu_run("rms_norm", {"x": x, "weight": w}, eps)
        check_bitexact(y, torch.from_numpy(double))
        check_bitexact(y, oracle.rms_norm(x, w, eps))
        fx, fr = gpu_run("fused_add_rms_norm", {"x": half, "residual": half.clone(), "weight": w}, eps)
        check_bitexact(fr, x)
        check_bitexact(fx, torch.from_numpy(double))
    say("fp16 double rounding: positions where a single rounding differs:", discriminating)
    assert discriminating > 20
