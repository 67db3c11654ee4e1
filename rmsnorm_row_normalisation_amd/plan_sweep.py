"""Time every compiled launch plan of an operation on the GPU, for the shapes
given, next to the plan the launch policy picks: the measurement the policy in
``csrc/ks_api.cpp`` is fitted to, and the way to refit it on another part.

    python -m rmsnorm_row_normalisation_amd.plan_sweep --op rms_norm_backward \\
        --dtype bfloat16 --hidden 1024,4096 --rows 64,2048 [--passes 2] [--csv FILE]

Each plan runs a captured HIP graph of back-to-back calls over rotating input
copies (up to ``--rotate-mib``, so that large batches come from HBM), timed by
events around whole replays: per pass the minimum over three replays.  Every
vector plan is also checked to give the policy plan's bits (the canonical fold
makes them bit-identical; the backward's dw, summed per workgroup, excepted).

Only vector plans are enumerated (teams of 8..1024 lanes, the fewest pieces per
lane that cover the row and the compiled sizes above it, every workgroup size
and hint combination the library compiles); a candidate the library does not
compile for the shape is dropped by asking the C ABI to validate it on an empty
batch, which needs no GPU (``candidates`` runs on the CPU).
"""
from __future__ import annotations

import argparse
import sys

import torch

from . import binding as b

OPS = ("rms_norm", "fused_add_rms_norm", "rms_norm_residual", "rms_norm_backward", "silu_and_mul", "softmax")
DTYPES = {"bfloat16": torch.bfloat16, "float16": torch.float16, "float32": torch.float32}
# (load_nt, store_nt, weight_lds) combinations the library may compile
HINTS = ((1, 1, 0), (1, 1, 1), (0, 0, 0), (0, 1, 0))
_FAKE = 1 << 32            # a 256-byte-aligned address; an empty batch never touches it
_SPAN = 1 << 28            # distance between the fake buffers (no overlap)


def plan_name(p: b.Plan) -> str:
    return (f"{p.threads_per_row}x{p.vectors_per_thread}/{p.block_threads} "
            f"nt{p.load_nt}{p.store_nt} lds{p.weight_lds}")


def accepted(op: str, dtype: torch.dtype, hidden: int, plan: b.Plan) -> bool:
    """Whether the library accepts `plan` for this op, dtype and row size (an
    empty batch through the C ABI: validation only, no launch)."""
    code = b.KS_DTYPE[dtype]
    a = [_FAKE + k * _SPAN for k in range(5)]
    if op == "rms_norm":
        st = b.ks_rms_norm_ex(a[0], a[1], a[2], 0, hidden, 1e-6, code, plan, 0)
    elif op == "fused_add_rms_norm":
        st = b.ks_fused_add_rms_norm_ex(a[0], a[1], a[2], 0, hidden, 1e-6, code, plan, 0)
    elif op == "rms_norm_residual":
        st = b.ks_rms_norm_residual_ex(a[0], a[1], a[2], a[3], 0, hidden, 1e-6, code, plan, 0)
    elif op == "rms_norm_backward":
        st = b.ks_rms_norm_backward_ex(a[0], 0, a[1], a[2], a[3], 0, hidden, 1e-6, code, 0, 0, plan, 0)
    elif op == "silu_and_mul":
        st = b.ks_silu_and_mul_ex(a[0], a[1], 0, hidden, code, plan, 0)
    elif op == "softmax":
        st = b.ks_softmax_ex(a[0], a[1], 0, hidden, code, plan, 0)
    else:
        raise ValueError(f"unknown op {op!r}")
    return st == 0


def candidates(op: str, dtype: torch.dtype, hidden: int) -> list[b.Plan]:
    """Every compiled vector plan that covers a row of `hidden` elements (for
    silu_and_mul, `hidden` is the output width)."""
    es = torch.empty(0, dtype=dtype).element_size()
    row_bytes = hidden * es
    if row_bytes % 16:
        return []
    nvec = row_bytes // 16
    out = []
    tpr = 8
    while tpr <= 1024:
        least = -(-nvec // tpr)
        for vpt in range(least, min(16, 2 * least) + 1):
            blocks = (1024, 512) if op == "rms_norm_backward" else (max(256, tpr),)
            for block in blocks:
                if tpr > block:
                    continue
                for ln, sn, lds in HINTS:
                    p = b.Plan(path=0, threads_per_row=tpr, vectors_per_thread=vpt, elems_per_access=16 // es,
                               rows_per_block=block // tpr, block_threads=block, load_nt=ln, store_nt=sn,
                               weight_lds=lds)
                    if accepted(op, dtype, hidden, p):
                        out.append(p)
        tpr *= 2
    return out


class _Case:
    """Rotating inputs and outputs of one shape, and one call of the op."""

    def __init__(self, op: str, dtype: torch.dtype, hidden: int, rows: int, rotate_bytes: int):
        self.op = op
        width = 2 * hidden if op == "silu_and_mul" else hidden
        es = torch.empty(0, dtype=dtype).element_size()
        per_set = rows * width * es * (2 if op in ("fused_add_rms_norm", "rms_norm_residual",
                                                   "rms_norm_backward") else 1)
        self.nsets = max(2, min(64, rotate_bytes // max(1, per_set)))
        g = torch.Generator(device="cpu").manual_seed(rows * 131 + hidden)
        self.sets = [(torch.randn(rows, width, generator=g).to(dtype).cuda(),
                      torch.randn(rows, width, generator=g).to(dtype).cuda()) for _ in range(self.nsets)]
        self.w = (torch.rand(hidden, generator=g) + 0.5).to(dtype).cuda()
        # the bit check's inputs, apart from the copies the in-place form overwrites while it is timed
        self.check_inputs = tuple(t.clone() for t in self.sets[0])
        self.outs = [torch.empty(rows, hidden, dtype=dtype, device="cuda") for _ in range(self.nsets)]
        self.dw = torch.empty(hidden, dtype=dtype, device="cuda")
        self.ws = None
        if op == "rms_norm_backward":
            self.ws = torch.empty(b.ks_rms_norm_backward_workspace_size(rows, hidden), dtype=torch.uint8,
                                  device="cuda")

    def call(self, i: int, plan: b.Plan | None, x=None, r=None, out=None) -> None:
        x0, r0 = self.sets[i % self.nsets]
        x = x0 if x is None else x
        r = r0 if r is None else r
        out = self.outs[i % self.nsets] if out is None else out
        if self.op == "rms_norm":
            b.rms_norm(x, self.w, 1e-6, out=out, plan=plan)
        elif self.op == "fused_add_rms_norm":
            b.fused_add_rms_norm(x, r, self.w, 1e-6, plan=plan)
        elif self.op == "rms_norm_residual":
            b.rms_norm_residual(x, r, self.w, 1e-6, out=out, plan=plan)
        elif self.op == "rms_norm_backward":
            b.rms_norm_backward(r, x, self.w, 1e-6, plan=plan, workspace=self.ws, dx=out, dweight=self.dw)
        elif self.op == "silu_and_mul":
            b.silu_and_mul(x, out=out, plan=plan)
        else:
            b.softmax(x, out=out, plan=plan, split=False)

    def result(self, plan: b.Plan | None) -> tuple[torch.Tensor, ...]:
        """The op's outputs for plan on fresh copies of the check inputs."""
        x, r = (t.clone() for t in self.check_inputs)
        out = torch.empty_like(self.outs[0])
        self.call(0, plan, x, r, out)
        torch.cuda.synchronize()
        return (x, r) if self.op == "fused_add_rms_norm" else (out,)


def time_plan(case: _Case, plan: b.Plan | None, passes: int, stream: torch.cuda.Stream) -> list[float]:
    """Microseconds per call (per pass: the best of three replays of a graph of
    back-to-back calls over the rotating copies)."""
    n = max(case.nsets, 32)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(stream):
        case.call(0, plan)
        torch.cuda.synchronize()
        with torch.cuda.graph(g, stream=stream):
            for i in range(n):
                case.call(i, plan)
        out = []
        for _ in range(passes):
            g.replay()
            torch.cuda.synchronize()
            best = float("inf")
            for _ in range(3):
                e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                e0.record(stream)
                g.replay()
                e1.record(stream)
                torch.cuda.synchronize()
                best = min(best, e0.elapsed_time(e1) * 1e3 / n)
            out.append(best)
    del g
    return out


def sweep(ops, dtypes, hiddens, rows_list, passes=2, rotate_mib=1024, csv=None, log=sys.stdout) -> list[dict]:
    stream = torch.cuda.Stream()
    rows_out = []
    print("op,dtype,hidden,rows,plan,policy,us," + ",".join(f"pass{i + 1}" for i in range(passes)), file=csv or log,
          flush=True)
    for op in ops:
        for dname in dtypes:
            dtype = DTYPES[dname]
            for hidden in hiddens:
                plans = candidates(op, dtype, hidden)
                for rows in rows_list:
                    case = _Case(op, dtype, hidden, rows, rotate_mib << 20)
                    pol = b.get_plan(op, dtype, hidden, rows)
                    ref = case.result(pol)
                    results = []
                    for p in [pol] + plans:
                        is_pol = p is pol
                        if not is_pol and p.as_dict() == pol.as_dict():
                            continue
                        if not is_pol and pol.path == 0:
                            got = case.result(p)
                            if not all(torch.equal(a, c) for a, c in zip(got, ref)):
                                raise RuntimeError(f"{op} {dname} {rows}x{hidden}: plan {plan_name(p)} gives "
                                                   f"other bits than the policy plan {plan_name(pol)}")
                        t = time_plan(case, p, passes, stream)
                        rec = {"op": op, "dtype": dname, "hidden": hidden, "rows": rows, "plan": plan_name(p),
                               "policy": int(is_pol), "us": min(t), "passes": t}
                        results.append(rec)
                        print(f"{op},{dname},{hidden},{rows},{rec['plan']},{rec['policy']},{rec['us']:.3f}," +
                              ",".join(f"{v:.3f}" for v in t), file=csv or log, flush=True)
                    best = min(results, key=lambda r: r["us"])
                    polr = results[0]
                    print(f"# {op} {dname} {rows}x{hidden}: policy {polr['plan']} {polr['us']:.2f} us, best "
                          f"{best['plan']} {best['us']:.2f} us ({100 * (polr['us'] / best['us'] - 1):+.1f}%)",
                          file=log, flush=True)
                    rows_out += results
                    del case
                    torch.cuda.empty_cache()
    return rows_out


def main(argv=None) -> None:
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--op", default="rms_norm", help="comma-separated: " + ", ".join(OPS))
    ap.add_argument("--dtype", default="bfloat16", help="comma-separated: " + ", ".join(DTYPES))
    ap.add_argument("--hidden", default="4096", help="comma-separated row widths (silu_and_mul: output width)")
    ap.add_argument("--rows", default="2048", help="comma-separated batch sizes")
    ap.add_argument("--passes", type=int, default=2)
    ap.add_argument("--rotate-mib", type=int, default=1024)
    ap.add_argument("--csv", default=None, help="write the per-plan lines here instead of stdout")
    a = ap.parse_args(argv)
    ops = a.op.split(",")
    for op in ops:
        if op not in OPS:
            ap.error(f"unknown op {op!r}")
    if not torch.cuda.is_available():
        ap.error("the sweep needs a HIP device")
    csv = open(a.csv, "w") if a.csv else None
    try:
        sweep(ops, a.dtype.split(","), [int(h) for h in a.hidden.split(",")], [int(r) for r in a.rows.split(",")],
              a.passes, a.rotate_mib, csv)
    finally:
        if csv:
            csv.close()


if __name__ == "__main__":
    main()
