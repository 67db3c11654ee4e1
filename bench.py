"""Benchmark: RMSNorm and fused residual-add RMSNorm on one MI355X (the
default workload), and the SwiGLU (S*) and softmax (X*) workloads.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload C3b] [--dtype bf16|fp16|fp32]
    python bench.py --sweep-workloads [--out FILE]      # every workload, one table
    python bench.py --stream-reference                  # reference streams at 16 MiB and 1 GiB
    python bench.py --wave-timeline                     # per-wave clock stamps of the row layouts at 16 MiB

One step is one pass of the whole path over one batch: ks_rms_norm on the
batch, then ks_fused_add_rms_norm on it (both at 2048 x 4096 bf16 by
default; x ~ N(0,1) with 1% of elements x100, residual ~ N(0,0.5), weight ~
U(0.5,1.5), eps = 1e-5).  The inputs are resident in HBM before timing.

Cache state: the 256 MiB Infinity Cache and the L2s would hold a 64 MiB
working set, so the steps rotate over enough copies of the batch (1 GiB by
default) that every step reads data last touched more than a cache's worth
of traffic ago.  Numbers are therefore HBM numbers, not cache numbers.

Timing (exactly K steps in every timed region):
  * whole job (``value``): one rotation of steps over the copies is captured
    into a HIP graph (no host launch overhead inside the timed region) and
    replayed, plus a graph of the remaining K mod (copies) steps, between a
    synchronize and two events on the launch stream;
  * per op, launch period (``per_op[op].us_per_call``): the same, with graphs
    holding only that op's launches back to back (median of three timed
    regions): what a caller sees per call in a captured sequence;
  * per op, kernel duration (``per_op[op].kernel_us``, ``roofline``): K calls
    of that op on the launch stream (at most 2048), each timed by the
    runtime's kernel-dispatch events (``ks_time_next_call``), enqueued in runs
    of 32 behind a 1 ms spin kernel and one untimed lead call, so that each
    run executes back to back and every timed call follows another one:
    min / p50 / p95 / p99 / max / mean of the kernels' own durations.
    ``roofline.achieved`` is the dominant kernel's algorithmic bytes over its
    mean duration;
  * ``stream_reference``: the library-independent reference streams of
    ``libks_streamref.so`` timed the same way: an empty kernel (the
    per-launch floor) and a plain copy (one 16-byte load and store per lane)
    of one batch-sized tensor and of 1 GiB (context for the fractions, never
    their denominator, which is the 8 TB/s spec).
Bytes are the algorithmic bytes the contract must move: rms_norm reads x and
writes out, (2 R H + H) elements; the fused form reads x and residual and
writes both, (4 R H + H) elements; rms_norm_residual reads x and residual
and writes out, (3 R H + H); silu_and_mul reads [R, 2D] and writes [R, D];
softmax reads and writes [R, H].

Before any timing the outputs are checked against the CPU oracle (all rows, or
sampled rows for batches over 2^24 elements); on a mismatch nothing is timed
(exit status 1).
"""
from __future__ import annotations

import argparse
import ctypes
import hashlib
import json
import os
import platform
import re
import sys
import time

import numpy as np
import torch

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import workloads  # noqa: E402

METRIC = "HBM GB/s (% of MI355X peak) + µs/call, rms_norm & fused_add @2048x4096 bf16"
HBM_PEAK_GBPS = 8000.0          # MI355X HBM3E, published peak
DTYPE_TAG = {"bfloat16": "bf16", "float16": "fp16", "float32": "fp32"}
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "hbm_traffic.json")
KERNEL_SOURCES = [os.path.join(ROOT, "rmsnorm_row_normalisation_amd", "csrc", f)
                  for f in ("ks_device.hpp", "ks_launch.hpp", "ks_internal.h", "ks_api.cpp")]
FULL_PARITY_ELEMS = 1 << 24     # above this, the parity gate checks sampled rows
SAMPLED_ROWS = 64
COPY_REPS = 5
MAX_SETS = 1024
STREAMREF_LIB = os.path.join(ROOT, "rmsnorm_row_normalisation_amd", "libks_streamref.so")
REF_FLOOR_GROUPS = 512          # the empty reference kernel's grid (the headline kernels' workgroup count)
GIB = 1 << 30


def algorithmic_bytes(op: str, rows: int, hidden: int, esize: int) -> int:
    """Bytes the contract must move.  rms_norm: read x, write out, read the weight
    once; fused: read x and residual, write both, read the weight; silu_and_mul
    (hidden = input width 2D): read x, write the D-wide output; softmax: read x,
    write out; rms_norm_residual: read x and residual, write out, read the
    weight; rms_norm_backward: read x and dy, write dx, read the weight and
    write its gradient (the fp32 workspace of partial sums is extra)."""
    if op == "silu_and_mul":
        return (rows * hidden + rows * (hidden // 2)) * esize
    if op == "softmax":
        return 2 * rows * hidden * esize
    if op == "rms_norm_backward":
        return (3 * rows * hidden + 2 * hidden) * esize
    per_row = {"rms_norm": 2, "rms_norm_residual": 3}.get(op, 4)
    return (per_row * rows * hidden + hidden) * esize


def kernel_source_hash() -> str:
    """Hash of the kernel sources with comments and whitespace removed."""
    h = hashlib.sha256()
    for p in KERNEL_SOURCES:
        with open(p) as f:
            text = f.read()
        text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
        text = re.sub(r"//[^\n]*", "", text)
        h.update("".join(text.split()).encode())
    return h.hexdigest()[:16]


def parse() -> argparse.Namespace:
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=2048)
    ap.add_argument("--warmup", type=int, default=64)
    ap.add_argument("--workload", default="C3b", choices=sorted(workloads.WORKLOADS))
    ap.add_argument("--dtype", default=None, choices=sorted(workloads.DTYPE_TAGS),
                    help="run the workload's shape, distributions and seeds in this dtype instead")
    ap.add_argument("--op", default=None,
                    help="measure only this op of the workload (e.g. rms_norm of C3b); it is then the whole step")
    ap.add_argument("--sweep-dtypes", default="bf16,fp16,fp32",
                    help="with --sweep-workloads: the dtypes the RMSNorm workloads C1, C2 and C3b also run in")
    ap.add_argument("--stream-reference", action="store_true",
                    help="time the reference streams (reads, writes, copies) at 16 MiB and 1 GiB and exit")
    ap.add_argument("--wave-timeline", action="store_true",
                    help="record per-wave clock stamps of the row layouts at 16 MiB (rms_norm's and the fused "
                         "form's streams) and print a markdown summary (--out, --json-out) and exit")
    ap.add_argument("--rotate-mib", type=int, default=1024, help="total size of the rotating input copies")
    ap.add_argument("--cpu-seconds", type=float, default=10.0, help="budget for the CPU oracle baseline")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--sweep-workloads", action="store_true",
                    help="measure every workload (per op) and print a markdown table instead of the bench line")
    ap.add_argument("--out", default=None,
                    help="with --sweep-workloads: also write the table to this file; with --trace-summary or "
                         "--wave-timeline: write the summary there")
    ap.add_argument("--json-out", default=None, help="also write the per-case results (JSON) to this file")
    ap.add_argument("--baseline", default=None,
                    help="a previous --json-out file: exit with status 2 if any matching case got slower "
                         "by more than --max-regression-percent")
    ap.add_argument("--max-regression-percent", type=float, default=10.0)
    ap.add_argument("--copy-calibration", type=int, metavar="MIB", default=0,
                    help="only run device-to-device copies of MIB MiB (the counter calibration run) and exit")
    ap.add_argument("--trace-summary", metavar="TRACE_DIR", default=None,
                    help="render a rocprofv3 --kernel-trace output directory of a bench run of --workload "
                         "(--dtype) as a markdown summary and exit (no GPU needed)")
    ap.add_argument("--trace-bench", metavar="JSON", default=None,
                    help="with --trace-summary: the bench line of an uninstrumented run of the same command")
    ap.add_argument("--trace-command", default=None,
                    help="with --trace-summary: the command line the trace was taken with, quoted in the summary")
    ap.add_argument("--traffic-summary", nargs=4, metavar=("FETCH", "WRITE", "COPY_FETCH", "COPY_WRITE"),
                    help="turn four rocprofv3 --pmc output directories into profiles/hbm_traffic.json and exit")
    return ap.parse_args()


def fail(msg: str, code: int = 1):
    print(json.dumps({"metric": METRIC, "error": msg}), flush=True)
    sys.exit(code)


def log(*a):
    print("[bench]", *a, file=sys.stderr, flush=True)


# ---------------------------------------------------------------------------
# parity gate
# ---------------------------------------------------------------------------
def parity_gate(wl, inp, ks, oracle_mod) -> dict:
    """GPU vs oracle on the full batch (or on sampled rows of a large one) before any timing."""
    sys.path.insert(0, os.path.join(ROOT, "tests"))
    from compare import backward_magnitudes, check_bitexact, check_gradient, check_normalised

    if wl.rows * wl.hidden <= FULL_PARITY_ELEMS:
        idx = None
    else:
        idx = torch.from_numpy(np.unique(np.concatenate([
            np.random.default_rng(77).choice(wl.rows, size=SAMPLED_ROWS, replace=False), [0, wl.rows - 1]])))

    def pick(t):
        return t if idx is None else t[idx].contiguous()

    def ref_inputs():
        return {k: (pick(v) if v.dim() == 2 else v) for k, v in inp.items()}

    out = {"rows_checked": wl.rows if idx is None else int(idx.numel())}
    if "silu_and_mul" in wl.ops:
        y = ks.silu_and_mul(inp["x"].cuda())
        torch.cuda.synchronize()
        ref = oracle_mod.silu_and_mul(pick(inp["x"]))
        st = check_normalised(pick(y.cpu()), ref, 0.999)
        out["silu_and_mul"] = {"max_ulp": st.max_ulp, "exact_match": round(st.exact_rate, 6)}
        return out
    if "rms_norm_backward" in wl.ops:
        gx, gw = ks.rms_norm_backward(inp["residual"].cuda(), inp["x"].cuda(), inp["weight"].cuda(), wl.eps)
        torch.cuda.synchronize()
        rx, rw = oracle_mod.rms_norm_backward(inp["residual"], inp["x"], inp["weight"], wl.eps)
        mdx, mdw = backward_magnitudes(inp["residual"], inp["x"], inp["weight"], wl.eps)
        st = check_gradient(gx.cpu(), rx, mdx, 0.99)
        sw = check_gradient(gw.cpu(), rw, mdw)
        # max_ulp / exact_match: dx (the sweep table's columns); dw separately
        out["rms_norm_backward"] = {"max_ulp": st.max_ulp, "exact_match": round(st.exact_rate, 6),
                                    "dw_max_ulp": sw.max_ulp, "dw_exact_match": round(sw.exact_rate, 6)}
        return out
    if "softmax" in wl.ops:
        y = ks.softmax(inp["x"].cuda())
        torch.cuda.synchronize()
        ref = oracle_mod.softmax(pick(inp["x"]))
        st = check_normalised(pick(y.cpu()), ref, 0.999)
        out["softmax"] = {"max_ulp": st.max_ulp, "exact_match": round(st.exact_rate, 6)}
        return out
    w = inp["weight"].cuda()
    if "rms_norm" in wl.ops:
        y = ks.rms_norm(inp["x"].cuda(), w, wl.eps)
        torch.cuda.synchronize()
        r = ref_inputs()
        ref = oracle_mod.rms_norm(r["x"], r["weight"], wl.eps)
        st = check_normalised(pick(y.cpu()), ref, 0.999)
        out["rms_norm"] = {"max_ulp": st.max_ulp, "exact_match": round(st.exact_rate, 6)}
        del y
    if "rms_norm_residual" in wl.ops:
        y = ks.rms_norm_residual(inp["x"].cuda(), inp["residual"].cuda(), w, wl.eps)
        torch.cuda.synchronize()
        r = ref_inputs()
        ref = oracle_mod.rms_norm_residual(r["x"], r["residual"], r["weight"], wl.eps)
        st = check_normalised(pick(y.cpu()), ref, 0.999)
        out["rms_norm_residual"] = {"max_ulp": st.max_ulp, "exact_match": round(st.exact_rate, 6)}
        del y
    if "fused_add_rms_norm" in wl.ops:
        xf, rf = inp["x"].cuda(), inp["residual"].cuda()
        ks.fused_add_rms_norm(xf, rf, w, wl.eps)
        torch.cuda.synchronize()
        r = ref_inputs()
        rx, rr = oracle_mod.fused_add_rms_norm(r["x"], r["residual"], r["weight"], wl.eps)
        check_bitexact(pick(rf.cpu()), rr)
        st = check_normalised(pick(xf.cpu()), rx, 0.999)
        out["fused_add_rms_norm"] = {"max_ulp": st.max_ulp, "exact_match": round(st.exact_rate, 6),
                                     "residual": "bit-exact"}
        del xf, rf
    return out


# ---------------------------------------------------------------------------
# timing
# ---------------------------------------------------------------------------
class Rig:
    """Rotating HBM-resident copies of a workload's batch and graph-timed launches."""

    def __init__(self, wl, inp, ks, rotate_mib: int):
        self.wl, self.ks = wl, ks
        esize = torch.empty(0, dtype=wl.torch_dtype).element_size()
        self.tensor_bytes = wl.rows * wl.hidden * esize
        footprint = {"rms_norm": 2.0, "fused_add_rms_norm": 2.0, "silu_and_mul": 1.5, "softmax": 2.0,
                     "rms_norm_residual": 3.0, "rms_norm_backward": 3.0}
        per_set = int(sum(footprint[op] for op in wl.ops) * self.tensor_bytes)
        # enough copies to pass through more than the last-level cache between
        # two uses of one copy; capped for tiny (launch-bound) batches
        self.nsets = min(MAX_SETS, max(2, -(-rotate_mib * (1 << 20) // per_set)))
        x0 = inp["x"].cuda()
        r0 = inp["residual"].cuda() if "residual" in inp else None
        self.w = inp["weight"].cuda() if "weight" in inp else None
        self.sets = []
        for _ in range(self.nsets):
            s = {}
            if "silu_and_mul" in wl.ops:
                s["sx"] = x0.clone()
                s["sout"] = torch.empty(wl.rows, wl.hidden // 2, dtype=x0.dtype, device=x0.device)
            if "rms_norm_backward" in wl.ops:
                s["bx"] = x0.clone()
                s["bdy"] = r0.clone()
                s["bdx"] = torch.empty_like(x0)
                s["bdw"] = torch.empty_like(self.w)
            if "rms_norm_residual" in wl.ops:
                s["ox"] = x0.clone()
                s["or"] = r0.clone()
                s["oout"] = torch.empty_like(x0)
            if "softmax" in wl.ops:
                s["mx"] = x0.clone()
                s["mout"] = torch.empty_like(x0)
            if "rms_norm" in wl.ops:
                s["x"] = x0.clone()
                s["out"] = torch.empty_like(x0)
            if "fused_add_rms_norm" in wl.ops:
                s["fx"] = x0.clone()
                s["fr"] = r0.clone()
            self.sets.append(s)
        del x0, r0
        if "rms_norm_backward" in wl.ops:
            self.workspace = torch.empty(ks.ks_rms_norm_backward_workspace_size(wl.rows, wl.hidden),
                                         dtype=torch.uint8, device="cuda")
        if "softmax" in wl.ops:          # split plans keep per-chunk statistics here
            need = ks.ks_softmax_workspace_size(wl.rows, wl.hidden, ks.KS_DTYPE[wl.torch_dtype])
            self.softmax_workspace = torch.empty(max(need, 1), dtype=torch.uint8, device="cuda")
        self.rotation_mib = self.nsets * per_set / 2**20
        self.stream = torch.cuda.Stream()
        torch.cuda.synchronize()

    def launch(self, op: str, i: int) -> None:
        s = self.sets[i % self.nsets]
        if op == "rms_norm":
            self.ks.rms_norm(s["x"], self.w, self.wl.eps, out=s["out"])
        elif op == "fused_add_rms_norm":
            self.ks.fused_add_rms_norm(s["fx"], s["fr"], self.w, self.wl.eps)
        elif op == "softmax":
            self.ks.softmax(s["mx"], out=s["mout"], workspace=self.softmax_workspace)
        elif op == "rms_norm_residual":
            self.ks.rms_norm_residual(s["ox"], s["or"], self.w, self.wl.eps, out=s["oout"])
        elif op == "rms_norm_backward":
            self.ks.rms_norm_backward(s["bdy"], s["bx"], self.w, self.wl.eps, workspace=self.workspace,
                                      dx=s["bdx"], dweight=s["bdw"])
        else:
            self.ks.silu_and_mul(s["sx"], out=s["sout"])

    def raw_call(self, op: str):
        """call(i): op on copy i through the C entry point itself, with every
        argument marshalled in advance (a few microseconds of host time per
        call, so a run of timed calls keeps the launch queue ahead of the GPU).
        Returns the status."""
        lib = self.ks.lib()
        wl, n = self.wl, self.nsets
        code = self.ks.KS_DTYPE[wl.torch_dtype]
        rows, hidden = wl.rows, wl.hidden
        eps = ctypes.c_float(wl.eps)
        st = self.stream.cuda_stream
        w = self.w.data_ptr() if self.w is not None else None
        P = [{k: v.data_ptr() for k, v in s.items()} for s in self.sets]
        if op == "rms_norm":
            return lambda i: lib.ks_rms_norm(P[i % n]["out"], P[i % n]["x"], w, rows, hidden, eps, code, st)
        if op == "fused_add_rms_norm":
            return lambda i: lib.ks_fused_add_rms_norm(P[i % n]["fx"], P[i % n]["fr"], w, rows, hidden, eps, code, st)
        if op == "rms_norm_residual":
            return lambda i: lib.ks_rms_norm_residual(P[i % n]["oout"], P[i % n]["ox"], P[i % n]["or"], w, rows,
                                                      hidden, eps, code, st)
        if op == "softmax":
            ws, wsn = self.softmax_workspace.data_ptr(), self.softmax_workspace.numel()
            return lambda i: lib.ks_softmax_ws(P[i % n]["mout"], P[i % n]["mx"], rows, hidden, code, ws, wsn, st)
        if op == "rms_norm_backward":
            ws, wsn = self.workspace.data_ptr(), self.workspace.numel()
            return lambda i: lib.ks_rms_norm_backward(P[i % n]["bdx"], P[i % n]["bdw"], P[i % n]["bdy"],
                                                      P[i % n]["bx"], w, rows, hidden, eps, code, ws, wsn, st)
        return lambda i: lib.ks_silu_and_mul(P[i % n]["sout"], P[i % n]["sx"], rows, hidden // 2, code, st)

    def timed_graph(self, body, per_rotation: int, steps: int, repeats: int = 1) -> float:
        """Exactly `steps` calls of body(i): body(i) for i < per_rotation is
        captured into one HIP graph, body(i) for i < steps mod per_rotation into
        a second; steps // per_rotation replays of the first and one of the
        second run between two events on the launch stream.  Milliseconds
        (the median of `repeats` timed regions)."""
        reps, tail = divmod(steps, per_rotation)
        graphs = []
        with torch.cuda.stream(self.stream):
            for count, n in ((reps, per_rotation), (1 if tail else 0, tail)):
                if count == 0:
                    continue
                g = torch.cuda.CUDAGraph()
                with torch.cuda.graph(g, stream=self.stream):
                    for i in range(n):
                        body(i)
                g.replay()                                   # untimed
                graphs.append((g, count))
            torch.cuda.synchronize()
            times = []
            for _ in range(repeats):
                ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                ev0.record(self.stream)
                for g, count in graphs:
                    for _ in range(count):
                        g.replay()
                ev1.record(self.stream)
                torch.cuda.synchronize()
                times.append(ev0.elapsed_time(ev1))
        return float(np.median(times))

    def warmup(self, n: int) -> None:
        with torch.cuda.stream(self.stream):
            for i in range(n):
                for op in self.wl.ops:
                    self.launch(op, i)
        torch.cuda.synchronize()


# ---------------------------------------------------------------------------
# HIP runtime calls the bench makes itself: events and versions
# ---------------------------------------------------------------------------
def _hip_runtime_path() -> str:
    """The HIP runtime library this process already uses (torch's), so that the
    events the bench creates are the ones the library records."""
    try:
        with open("/proc/self/maps") as f:
            for line in f:
                parts = line.split()
                if len(parts) >= 6 and os.path.basename(parts[-1]).startswith("libamdhip64.so"):
                    return parts[-1]
    except OSError:
        pass
    return "libamdhip64.so.7"


class Hip:
    def __init__(self):
        torch.cuda.init()
        self.h = ctypes.CDLL(_hip_runtime_path())
        vp, ci = ctypes.c_void_p, ctypes.c_int
        self.h.hipEventCreate.argtypes = [ctypes.POINTER(vp)]
        self.h.hipEventDestroy.argtypes = [vp]
        self.h.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), vp, vp]
        self.h.hipEventRecord.argtypes = [vp, vp]
        self.h.hipEventQuery.argtypes = [vp]
        self.h.hipRuntimeGetVersion.argtypes = [ctypes.POINTER(ci)]
        self.h.hipDriverGetVersion.argtypes = [ctypes.POINTER(ci)]

    def event(self) -> int:
        e = ctypes.c_void_p()
        rc = self.h.hipEventCreate(ctypes.byref(e))
        if rc != 0 or not e.value:
            raise RuntimeError(f"hipEventCreate failed ({rc})")
        return e.value

    def destroy(self, e: int) -> None:
        self.h.hipEventDestroy(ctypes.c_void_p(e))

    def record(self, e: int, stream: int) -> None:
        rc = self.h.hipEventRecord(ctypes.c_void_p(e), ctypes.c_void_p(stream))
        if rc != 0:
            raise RuntimeError(f"hipEventRecord failed ({rc})")

    def done(self, e: int) -> bool:
        """Whether the stream has reached event e (hipEventQuery)."""
        rc = self.h.hipEventQuery(ctypes.c_void_p(e))
        if rc not in (0, 600):   # hipSuccess, hipErrorNotReady
            raise RuntimeError(f"hipEventQuery failed ({rc})")
        return rc == 0

    def elapsed_us(self, a: int, b: int) -> float:
        ms = ctypes.c_float()
        rc = self.h.hipEventElapsedTime(ctypes.byref(ms), ctypes.c_void_p(a), ctypes.c_void_p(b))
        if rc != 0:
            raise RuntimeError(f"hipEventElapsedTime failed ({rc})")
        return ms.value * 1e3

    def versions(self) -> dict:
        rt, drv = ctypes.c_int(0), ctypes.c_int(0)
        self.h.hipRuntimeGetVersion(ctypes.byref(rt))
        self.h.hipDriverGetVersion(ctypes.byref(drv))
        return {"hip_runtime": rt.value, "hip_driver": drv.value, "hip_runtime_library": _hip_runtime_path()}


def distribution(vals: list[float]) -> dict:
    """n, mean, min, p50, p95, p99 and max of a sample (nearest-rank percentiles), rounded to ns."""
    v = sorted(vals)
    n = len(v)

    def q(p: float) -> float:
        return v[min(n - 1, max(0, int(np.ceil(p * n)) - 1))]

    return {"n": n, "mean": round(float(np.mean(v)), 3), "min": round(v[0], 3), "p50": round(q(0.50), 3),
            "p95": round(q(0.95), 3), "p99": round(q(0.99), 3), "max": round(v[-1], 3)}


HEAD_START_US = 1000     # the first spin kernel queued ahead of a run of timed calls
HEAD_START_MAX_US = 20000
HEAD_START_CALLS = 32    # timed calls enqueued behind one spin kernel


def kernel_durations(hip: Hip, call, n: int, stream: torch.cuda.Stream, timed_call=None,
                     info: dict | None = None) -> list[float]:
    """n calls of call(i) (a raw C entry point on `stream`, returning its status),
    each timed by the runtime's kernel-dispatch events (from the start of the
    call's first kernel to the end of its last): microseconds.  The calls go in
    runs of HEAD_START_CALLS behind a spin kernel, so the host has enqueued a
    run before it starts and its calls execute back to back, as they would in
    a steady stream of work.  The first spin lasts HEAD_START_US; each later
    one at least twice the host time the previous run took to enqueue (10-20
    us per call from Python, several times that under a tracer), up to
    HEAD_START_MAX_US.  A run is late when its spin had already ended by the
    time its last call was enqueued (the GPU may then have idled between
    calls); `info`, if given, receives runs, late_runs and the last spin's
    length.  Each run opens with one untimed call on the previous copy: the
    first call after the idle spin runs slower (about 0.8 us for rms_norm at
    2048x4096), and every timed call should follow another one as in a
    stream.  `timed_call(i, start, stop)` replaces the request through
    ks_time_next_call for callers that take the events themselves (start and
    stop None: untimed)."""
    import rmsnorm_row_normalisation_amd as ks

    lib = ks.lib()
    ref = StreamRef()
    evs = [(hip.event(), hip.event()) for _ in range(n)]
    marks: list[int] = []
    spin_us, late, t_run = HEAD_START_US, 0, None

    def close_run() -> None:
        nonlocal spin_us, late
        enqueue_us = (time.perf_counter() - t_run) * 1e6
        if hip.done(marks[-1]):
            late += 1
        spin_us = min(HEAD_START_MAX_US, max(spin_us, int(2 * enqueue_us)))

    try:
        torch.cuda.synchronize()
        for i, (a, b) in enumerate(evs):
            if i % HEAD_START_CALLS == 0:
                if t_run is not None:
                    close_run()
                StreamRef.check(ref.h.ksref_spin(spin_us, stream.cuda_stream), "ksref_spin")
                marks.append(hip.event())
                hip.record(marks[-1], stream.cuda_stream)
                if timed_call is not None:     # the untimed lead call
                    timed_call(i - 1, None, None)
                else:
                    rc = call(i - 1)
                    if rc != 0:
                        raise RuntimeError(f"lead call failed: {lib.ks_status_string(rc).decode()}")
                t_run = time.perf_counter()
            if timed_call is not None:
                timed_call(i, a, b)
            else:
                lib.ks_time_next_call(a, b)
                rc = call(i)
                if rc != 0:
                    raise RuntimeError(f"timed call failed: {lib.ks_status_string(rc).decode()}")
        if t_run is not None:
            close_run()
        torch.cuda.synchronize()
        if info is not None:
            info.update({"runs": len(marks), "late_runs": late, "head_start_us": spin_us})
        return [hip.elapsed_us(a, b) for a, b in evs]
    finally:
        for a, b in evs:
            hip.destroy(a)
            hip.destroy(b)
        for e in marks:
            hip.destroy(e)


KERNEL_TIMED_MAX = 2048


def measure(wl, inp, ks, args, hip: Hip) -> dict:
    """Whole-step throughput and, per op, the launch period and the kernel durations."""
    esize = torch.empty(0, dtype=wl.torch_dtype).element_size()
    op_bytes = {op: algorithmic_bytes(op, wl.rows, wl.hidden, esize) for op in wl.ops}
    rig = Rig(wl, inp, ks, args.rotate_mib)
    log(f"{wl.name}: {rig.nsets} rotating copies, {rig.rotation_mib:.0f} MiB")
    steps = args.steps
    rig.warmup(args.warmup)
    total_ms = rig.timed_graph(lambda i: [rig.launch(op, i) for op in wl.ops], rig.nsets, steps)
    per_op = {}
    for op in wl.ops:
        # launch period: median of three timed regions (run-to-run spread is a few %)
        ms = rig.timed_graph(lambda i, op=op: rig.launch(op, i), rig.nsets, steps, repeats=3)
        us = ms * 1e3 / steps
        timing: dict = {}
        kus = distribution(kernel_durations(hip, rig.raw_call(op), min(steps, KERNEL_TIMED_MAX), rig.stream,
                                            info=timing))
        kus.update(timing)
        gbps = op_bytes[op] / (kus["mean"] * 1e-6) / 1e9
        per_op[op] = {"us_per_call": round(us, 3), "kernel_us": kus, "bytes": op_bytes[op], "gbps": round(gbps, 1),
                      "frac_of_peak": round(gbps / HBM_PEAK_GBPS, 4),
                      "gbps_per_call": round(op_bytes[op] / (us * 1e-6) / 1e9, 1),
                      "plan": ks.get_plan(op, wl.torch_dtype, wl.hidden // 2 if op == "silu_and_mul" else wl.hidden,
                                          wl.rows, workspace=op == "softmax").as_dict()}
    ms_per_step = total_ms / steps
    result = {"steps": steps, "nsets": rig.nsets, "rotation_mib": rig.rotation_mib,
              "ms_per_step": ms_per_step, "step_bytes": sum(op_bytes.values()),
              "value": sum(op_bytes.values()) / (ms_per_step * 1e-3) / 1e9, "per_op": per_op,
              "tensor_bytes": rig.tensor_bytes}
    del rig
    torch.cuda.empty_cache()
    return result


# ---------------------------------------------------------------------------
# reference streams (libks_streamref.so)
# ---------------------------------------------------------------------------
class StreamRef:
    """The benchmark's reference streams: an empty kernel, reads, writes and
    copies of 16-byte pieces (rmsnorm_row_normalisation_amd/streamref)."""

    def __init__(self):
        if not os.path.exists(STREAMREF_LIB):
            raise RuntimeError(f"{STREAMREF_LIB} is not built; run __graft_entry__.build() first")
        h = ctypes.CDLL(STREAMREF_LIB)
        vp, u64, ci, cu = ctypes.c_void_p, ctypes.c_uint64, ctypes.c_int, ctypes.c_uint
        h.ksref_read.argtypes = [vp, u64, vp, vp, vp, vp]
        h.ksref_write.argtypes = [vp, u64, ci, vp, vp, vp]
        h.ksref_copy.argtypes = [vp, vp, u64, ci, vp, vp, vp]
        h.ksref_copy_rows.argtypes = [vp, vp, u64, ci, vp, vp, vp]
        h.ksref_inplace4.argtypes = [vp, vp, u64, ci, vp, vp, vp]
        h.ksref_empty.argtypes = [cu, vp, vp, vp]
        h.ksref_spin.argtypes = [cu, vp]
        h.ksref_timeline.argtypes = [vp, vp, u64, ci, ci, vp, u64, vp, vp, vp]
        h.ksref_wall_clock_khz.argtypes = [ctypes.POINTER(ci)]
        self.h = h

    @staticmethod
    def check(rc: int, what: str) -> None:
        if rc != 0:
            raise RuntimeError(f"{what} failed ({rc})")


# name -> (bytes moved per byte of buffer, launcher(ref, src, dst, nbytes, sink, stream, e0, e1))
STREAMS = {
    "read": (1, lambda r, a, b, n, k, s, e0, e1: r.h.ksref_read(a, n, k, s, e0, e1)),
    "write": (1, lambda r, a, b, n, k, s, e0, e1: r.h.ksref_write(b, n, 0, s, e0, e1)),
    "write nt": (1, lambda r, a, b, n, k, s, e0, e1: r.h.ksref_write(b, n, 1, s, e0, e1)),
    "write sc0 sc1": (1, lambda r, a, b, n, k, s, e0, e1: r.h.ksref_write(b, n, 2, s, e0, e1)),
    "copy": (2, lambda r, a, b, n, k, s, e0, e1: r.h.ksref_copy(a, b, n, 0, s, e0, e1)),
    "copy nt": (2, lambda r, a, b, n, k, s, e0, e1: r.h.ksref_copy(a, b, n, 1, s, e0, e1)),
    "copy sc0 sc1": (2, lambda r, a, b, n, k, s, e0, e1: r.h.ksref_copy(a, b, n, 2, s, e0, e1)),
    "rows 1": (2, lambda r, a, b, n, k, s, e0, e1: r.h.ksref_copy_rows(a, b, n, 1, s, e0, e1)),
    "rows 2": (2, lambda r, a, b, n, k, s, e0, e1: r.h.ksref_copy_rows(a, b, n, 2, s, e0, e1)),
    "rows 4": (2, lambda r, a, b, n, k, s, e0, e1: r.h.ksref_copy_rows(a, b, n, 4, s, e0, e1)),
    "rows 8": (2, lambda r, a, b, n, k, s, e0, e1: r.h.ksref_copy_rows(a, b, n, 8, s, e0, e1)),
    "in place x+r 1": (4, lambda r, a, b, n, k, s, e0, e1: r.h.ksref_inplace4(a, b, n, 1, s, e0, e1)),
    "in place x+r 2": (4, lambda r, a, b, n, k, s, e0, e1: r.h.ksref_inplace4(a, b, n, 2, s, e0, e1)),
    "in place x+r 8": (4, lambda r, a, b, n, k, s, e0, e1: r.h.ksref_inplace4(a, b, n, 8, s, e0, e1)),
}
STREAM_DESCRIPTIONS = {
    "read": "one 16-byte load per lane", "write": "one 16-byte store per lane, default cache bits",
    "write nt": "the same, non-temporal", "write sc0 sc1": "the same, system scope (sc0 sc1)",
    "copy": "one load and one store per lane", "copy nt": "the same, non-temporal stores",
    "copy sc0 sc1": "the same, system-scope stores",
    "rows 1": "the row kernels' layout: a wave owns N KiB (N pieces per lane at a 1 KiB stride), loads, "
              "a wave-wide sum and double rsqrt, then stores",
    "rows 2": "", "rows 4": "", "rows 8": "",
    "in place x+r 1": "the fused form's four streams: read x and r, write both back in place (row layout, "
                      "N pieces per lane)",
    "in place x+r 2": "", "in place x+r 8": "",
}


def stream_times(hip: Hip, ref: StreamRef, name: str, nbytes: int, launches: int, graph_calls: int) -> dict:
    """One reference stream over rotating buffers of nbytes (at least 1 GiB of
    buffers in the rotation, so every call reads data last touched more than a
    cache's worth of traffic ago): kernel durations from the kernel-dispatch
    events, and the launch period of graph-captured back-to-back calls."""
    mult, fn = STREAMS[name]
    nsets = max(1, -(-GIB // nbytes)) if nbytes < GIB else 1
    bufs = [(torch.empty(nbytes, dtype=torch.uint8, device="cuda").random_(0, 255),
             torch.empty(nbytes, dtype=torch.uint8, device="cuda")) for _ in range(nsets)]
    sink = torch.zeros(256, dtype=torch.int32, device="cuda")
    stream = torch.cuda.Stream()

    def call(i: int, e0=None, e1=None) -> None:
        a, b = bufs[i % nsets]
        StreamRef.check(fn(ref, a.data_ptr(), b.data_ptr(), nbytes, sink.data_ptr(), stream.cuda_stream, e0, e1), name)

    for i in range(2 * nsets):
        call(i)
    torch.cuda.synchronize()
    kus = distribution(kernel_durations(hip, None, launches, stream, timed_call=lambda i, a, b: call(i, a, b)))
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(stream):
        with torch.cuda.graph(g, stream=stream):
            for i in range(graph_calls):
                call(i)
        g.replay()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        g.replay()
        e1.record(stream)
        torch.cuda.synchronize()
    period = e0.elapsed_time(e1) * 1e3 / graph_calls
    moved = mult * nbytes
    del bufs, g
    torch.cuda.empty_cache()
    return {"stream": name, "buffer_bytes": nbytes, "bytes_moved": moved, "kernel_us": kus,
            "gbps": round(moved / (kus["mean"] * 1e-6) / 1e9, 1),
            "frac_of_peak": round(moved / (kus["mean"] * 1e-6) / 1e9 / HBM_PEAK_GBPS, 4),
            "us_per_call": round(period, 3), "gbps_per_call": round(moved / (period * 1e-6) / 1e9, 1)}


def empty_kernel_floor(hip: Hip, ref: StreamRef, launches: int = 512) -> dict:
    """A kernel that does nothing (REF_FLOOR_GROUPS workgroups of 256 threads):
    its launch period back to back in a graph (the per-launch floor of a
    captured sequence), and its kernel-dispatch event interval (which, for a
    kernel this short, is mostly the events' own overhead)."""
    stream = torch.cuda.Stream()

    def call(a=None, b=None) -> None:
        StreamRef.check(ref.h.ksref_empty(REF_FLOOR_GROUPS, stream.cuda_stream, a, b), "ksref_empty")

    kus = distribution(kernel_durations(hip, None, launches, stream, timed_call=lambda i, a, b: call(a, b)))
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(stream):
        with torch.cuda.graph(g, stream=stream):
            for _ in range(launches):
                call()
        g.replay()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        g.replay()
        e1.record(stream)
        torch.cuda.synchronize()
    return {"groups": REF_FLOOR_GROUPS, "us_per_call": round(e0.elapsed_time(e1) * 1e3 / launches, 3),
            "event_interval_us": kus}


def stream_reference(hip: Hip, tensor_bytes: int) -> dict:
    """The bench line's context: the per-launch floor, and a plain copy (one
    load and store per lane, system-scope stores: the fastest copy measured)
    of one batch-sized tensor and of 1 GiB."""
    ref = StreamRef()
    size = max(4096, tensor_bytes // 4096 * 4096)
    return {"empty_kernel": empty_kernel_floor(hip, ref),
            "copy_tensor": stream_times(hip, ref, "copy sc0 sc1", size, 256 if size <= 64 << 20 else 16, 16),
            "copy_1gib": stream_times(hip, ref, "copy sc0 sc1", GIB, 16, 4)}


def stream_reference_table(hip: Hip) -> None:
    """Every reference stream at 16 MiB and at 1 GiB, one markdown table (and
    the JSON cases with --json-out)."""
    ref = StreamRef()
    floor = empty_kernel_floor(hip, ref)
    lines = [f"Empty kernel ({REF_FLOOR_GROUPS} workgroups of 256 threads): {floor['us_per_call']:.2f} us per call "
             f"back to back in a graph; its kernel-dispatch event interval p50 "
             f"{floor['event_interval_us']['p50']:.2f} us (mostly the events' own overhead at this length).", "",
             "| Stream | Buffer | Bytes moved | Kernel p50 us | Kernel mean us | GB/s (mean) | % of 8 TB/s "
             "| Graph us/call | What it is |",
             "|---|---|---|---|---|---|---|---|---|"]
    cases = []
    for nbytes, launches, graph_calls in ((16 << 20, 256, 64), (GIB, 16, 4)):
        for name in STREAMS:
            r = stream_times(hip, ref, name, nbytes, launches, graph_calls)
            cases.append(r)
            lines.append(f"| {name} | {nbytes >> 20} MiB | {r['bytes_moved'] >> 20} MiB | {r['kernel_us']['p50']:.2f} "
                         f"| {r['kernel_us']['mean']:.2f} | {r['gbps']:.0f} | {100 * r['frac_of_peak']:.1f} "
                         f"| {r['us_per_call']:.2f} | {STREAM_DESCRIPTIONS[name]} |")
            log(lines[-1])
    print("\n".join(lines), flush=True)
    return {"empty_kernel": floor, "cases": cases}


TIMELINE_BYTES = 16 << 20       # one 2048 x 4096 bf16 tensor
TIMELINE_CALLS = 64
TIMELINE_STAMPS = ("start", "first", "loaded", "scaled", "issued", "acked", "hw_id", "xcc_id")
# (layout, store policy, name, what it is, histogram in the summary); the
# kernels' own stores are non-temporal (policy 1)
TIMELINE_LAYOUTS = (
    (2, 0, "stamps only", "no loads or stores: the launch and the waves alone", False),
    (0, 1, "rows 8", "rms_norm's layout: read x, write y, non-temporal stores", True),
    (0, 2, "rows 8 sc0 sc1", "the same with stores written through (system scope)", False),
    (1, 1, "in place x+r 8", "the fused form's: read x and r, write both in place, non-temporal stores", True),
    (1, 2, "in place x+r 8 sc0 sc1", "the same with stores written through", False),
)


def timeline_call_stats(st: np.ndarray, tick_us: float, event_us: float) -> dict:
    """One call's wave records (waves x 8 words) reduced to where its time went:
    offsets from the first wave's start, per-wave phase lengths, residency."""
    t0, tf, t1, t2, t3, t4 = (st[:, k].astype(np.int64) for k in range(6))
    base = t0.min()
    us = lambda v: v.astype(np.float64) * tick_us  # noqa: E731
    load, reduce_, issue, ack = us(t1 - t0), us(t2 - t1), us(t3 - t2), us(t4 - t3)
    span = float(us(t4.max() - base))
    edges = np.concatenate([t0, t4])
    order = np.argsort(edges, kind="stable")
    alive = np.cumsum(np.where(order < len(t0), 1, -1))
    return {
        "event_us": event_us, "span_us": span, "outside_waves_us": event_us - span,
        "start_ramp_us": float(us(t0.max() - base)),
        "first_data_us": float(us(tf.min() - base)), "first_data_p50_us": float(np.median(us(tf - base))),
        "first_loaded_us": float(us(t1.min() - base)), "last_loaded_us": float(us(t1.max() - base)),
        "first_issued_us": float(us(t3.min() - base)), "last_issued_us": float(us(t3.max() - base)),
        "last_acked_us": span,
        "first_load_p50_us": float(np.median(us(tf - t0))), "load_p50_us": float(np.median(load)), "load_p90_us": float(np.quantile(load, 0.9)),
        "load_max_us": float(load.max()), "reduce_p50_us": float(np.median(reduce_)),
        "issue_p50_us": float(np.median(issue)), "ack_p50_us": float(np.median(ack)),
        "ack_max_us": float(ack.max()), "max_resident_waves": int(alive.max()),
    }


def timeline_histogram(st: np.ndarray, tick_us: float, bucket_us: float = 0.5) -> list[dict]:
    """Waves that started, had their loads arrive, issued their last store and
    had their stores acknowledged in each bucket of time from the first start."""
    base = st[:, 0].astype(np.int64).min()
    rel = (st[:, :6].astype(np.int64) - base) * tick_us
    nb = int(rel.max() // bucket_us) + 1
    rows = []
    for b in range(nb):
        lo, hi = b * bucket_us, (b + 1) * bucket_us
        n = lambda k: int(((rel[:, k] >= lo) & (rel[:, k] < hi)).sum())  # noqa: E731
        rows.append({"from_us": lo, "started": n(0), "first": n(1), "loaded": n(2), "issued": n(4), "acked": n(5)})
    return rows


def wave_timeline(hip: Hip) -> dict:
    """ksref_timeline over rotating 16 MiB buffers (1 GiB in the rotation, every
    call cold), TIMELINE_CALLS calls back to back behind a head-start spin, each
    also timed by its kernel-dispatch events; per layout the medians over calls
    of each call's statistics, the spread of the dispatch events, the waves per
    XCD and compute unit, and the histogram of the median call."""
    ref = StreamRef()
    khz = ctypes.c_int(0)
    StreamRef.check(ref.h.ksref_wall_clock_khz(ctypes.byref(khz)), "ksref_wall_clock_khz")
    if khz.value <= 0:
        raise RuntimeError("the device reports no wall clock rate")
    tick_us = 1e3 / khz.value
    nbytes, calls = TIMELINE_BYTES, TIMELINE_CALLS
    waves = nbytes // 8192
    nsets = GIB // nbytes
    stream = torch.cuda.Stream()
    out = {"bytes_per_tensor": nbytes, "waves": waves, "calls": calls, "wall_clock_khz": khz.value, "layouts": []}
    for layout, policy, name, what, hist in TIMELINE_LAYOUTS:
        bufs = [(torch.empty(nbytes, dtype=torch.uint8, device="cuda").random_(0, 255),
                 torch.empty(nbytes, dtype=torch.uint8, device="cuda").random_(0, 255)) for _ in range(nsets)]
        stamps = torch.zeros(calls, waves, len(TIMELINE_STAMPS), dtype=torch.int64, device="cuda")

        def call(i: int, e0=None, e1=None) -> None:
            x, y = bufs[i % nsets]
            row = stamps[i % calls]
            StreamRef.check(ref.h.ksref_timeline(x.data_ptr(), y.data_ptr(), nbytes, layout, policy, row.data_ptr(),
                                                 row.numel() * row.element_size(), stream.cuda_stream, e0, e1),
                            "ksref_timeline")

        for i in range(2 * nsets):
            call(i)
        torch.cuda.synchronize()
        ev = kernel_durations(hip, None, calls, stream, timed_call=lambda i, a, b: call(i, a, b))
        st = stamps.cpu().numpy()
        per_call = [timeline_call_stats(st[c], tick_us, ev[c]) for c in range(calls)]
        med = {k: round(float(np.median([p[k] for p in per_call])), 3) for k in per_call[0]}
        mid = int(np.argsort([p["event_us"] for p in per_call])[calls // 2])
        hw = st[:, :, 6].astype(np.int64)
        cu_key = (st[:, :, 7].astype(np.int64) << 16) | (((hw >> 13) & 7) << 8) | (((hw >> 12) & 1) << 4) | ((hw >> 8) & 15)
        xcc = st[mid, :, 7].astype(np.int64)
        start_by_xcc = {int(x): round(float(np.median((st[mid, xcc == x, 0] - st[mid, :, 0].min()) * tick_us)), 3)
                        for x in np.unique(xcc)}
        out["layouts"].append({
            "stream": name, "what": what, "bytes_moved": {0: 2, 1: 4, 2: 0}[layout] * nbytes,
            "event_us": distribution(ev), "median": med,
            "distinct_cus": int(len(np.unique(cu_key[mid]))), "waves_per_xcc": {int(x): int((xcc == x).sum())
                                                                             for x in np.unique(xcc)},
            "median_start_by_xcc_us": start_by_xcc, "median_call": mid,
            "histogram": timeline_histogram(st[mid], tick_us) if hist else None})
        del bufs, stamps
        torch.cuda.empty_cache()
    return out


def wave_timeline_markdown(res: dict) -> str:
    L = ["| Quantity (median over calls; µs from the first wave's start) | " +
         " | ".join(f"{l['stream']}" for l in res["layouts"]) + " |",
         "|---|" + "---|" * len(res["layouts"])]
    rows = [("kernel-dispatch events (whole kernel)", "event_us"), ("waves' span: first start to last ack", "span_us"),
            ("outside the waves (events minus span)", "outside_waves_us"),
            ("wave starts spread over", "start_ramp_us"), ("first data back (any wave's first load)", "first_data_us"),
            ("waves' first load back, p50", "first_data_p50_us"), ("first wave's loads all arrived", "first_loaded_us"),
            ("last wave's loads all arrived", "last_loaded_us"), ("first wave's stores all issued", "first_issued_us"),
            ("last wave's stores all issued", "last_issued_us"), ("last wave's stores acknowledged", "last_acked_us"),
            ("per wave: start to first load back, p50", "first_load_p50_us"),
            ("per wave: start to loads arrived, p50", "load_p50_us"), ("per wave: the same, p90", "load_p90_us"),
            ("per wave: the same, max", "load_max_us"), ("per wave: sum, shuffles and rsqrt, p50", "reduce_p50_us"),
            ("per wave: store issue, p50", "issue_p50_us"), ("per wave: issue to acknowledged, p50", "ack_p50_us"),
            ("per wave: the same, max", "ack_max_us"), ("most waves resident at once", "max_resident_waves")]
    for label, key in rows:
        L.append(f"| {label} | " + " | ".join(f"{l['median'][key]}" for l in res["layouts"]) + " |")
    L.append("| kernel-dispatch events p50 / p95 / max | " + " | ".join(
        f"{l['event_us']['p50']} / {l['event_us']['p95']} / {l['event_us']['max']}" for l in res["layouts"]) + " |")
    L.append("| distinct compute units (one call) | " + " | ".join(str(l["distinct_cus"]) for l in res["layouts"]) + " |")
    L.append("| median wave start by XCD (one call) | " + " | ".join(
        ", ".join(f"{x}: {v}" for x, v in l["median_start_by_xcc_us"].items()) for l in res["layouts"]) + " |")
    out = ["# Wave timeline: the row kernels' layouts at 16 MiB (`bench.py --wave-timeline`)", "",
           "Command (from the repository root, on an MI355X):", "", "```",
           "python bench.py --wave-timeline --out <this file> --json-out <stamps summary JSON>", "```", "",
           "ksref_timeline (rmsnorm_row_normalisation_amd/streamref) runs the reference streams' row layouts with "
           "lane 0 of every wave reading the device's constant-rate wall clock at the wave's start, when its first "
           "load is back, when all its loads are back, when the row's scale is ready, when its last store has "
           "issued and when its stores are acknowledged; the kernel-dispatch events time the whole kernel.  "
           "Times are from the first wave's start.",
           "", f"{res['waves']} waves of one 8 KiB row each, 16 MiB per tensor, {res['calls']} calls back to back "
           f"(each cold: 1 GiB of buffers in the rotation); wall clock {res['wall_clock_khz']} kHz.", ""] + L
    for l in res["layouts"]:
        if l["histogram"] is None:
            continue
        out += ["", f"Waves per 0.5 µs of the median call (#{l['median_call']}), {l['stream']} ({l['what']}):", "",
                "| from µs | started | first load back | all loads back | last store issued | stores acknowledged |",
                "|---|---|---|---|---|---|"]
        out += [f"| {h['from_us']:.1f} | {h['started']} | {h['first']} | {h['loaded']} | {h['issued']} | {h['acked']} |"
                for h in l["histogram"]]
    return "\n".join(out) + "\n"


# ---------------------------------------------------------------------------
# CPU baseline
# ---------------------------------------------------------------------------
def cpu_baseline(wl, inp, oracle_mod, budget_s: float, step_bytes: int) -> dict:
    """The oracle as it stands, single-threaded on a host core, on whole steps of
    the workload, repeated for about budget_s seconds: the median step time."""
    times = []
    t_start = time.perf_counter()
    while True:
        t0 = time.perf_counter()
        if "rms_norm" in wl.ops:
            oracle_mod.rms_norm(inp["x"], inp["weight"], wl.eps)
        if "fused_add_rms_norm" in wl.ops:
            oracle_mod.fused_add_rms_norm(inp["x"], inp["residual"], inp["weight"], wl.eps)
        if "silu_and_mul" in wl.ops:
            oracle_mod.silu_and_mul(inp["x"])
        if "softmax" in wl.ops:
            oracle_mod.softmax(inp["x"])
        if "rms_norm_residual" in wl.ops:
            oracle_mod.rms_norm_residual(inp["x"], inp["residual"], inp["weight"], wl.eps)
        if "rms_norm_backward" in wl.ops:
            oracle_mod.rms_norm_backward(inp["residual"], inp["x"], inp["weight"], wl.eps)
        times.append(time.perf_counter() - t0)
        if time.perf_counter() - t_start >= budget_s and len(times) >= 3:
            break
    med = float(np.median(times))
    return {"value": round(step_bytes / med / 1e9, 4), "unit": "GB/s", "cores": 1, "kind": "oracle",
            "sample": f"{len(times)} full steps ({' + '.join(wl.ops)} on the whole [{wl.rows},{wl.hidden}] batch), "
                      f"timed one by one, single thread; value from the median step",
            "us_per_step": {"median": round(med * 1e6, 1), "min": round(min(times) * 1e6, 1),
                            "max": round(max(times) * 1e6, 1)},
            "host_cpus": os.cpu_count(), "host_cpu": _cpu_model()}


def memory_interface() -> dict | None:
    """The device's reported memory bus width and clock (hipDeviceGetAttribute)
    and their product (bytes per reported clock), as context next to the
    8 TB/s spec peak that the fractions use.  The product is not a peak: the
    HBM3E interface moves several transfers per reported clock (8 TB/s over
    2048 GB/s is about 4)."""
    try:
        hip = ctypes.CDLL(_hip_runtime_path())
    except OSError:
        return None
    bus, clk = ctypes.c_int(0), ctypes.c_int(0)
    bus_width_attr, mem_clock_attr = 59, 60          # hipDeviceAttributeMemoryBusWidth / ...MemoryClockRate
    if (hip.hipDeviceGetAttribute(ctypes.byref(bus), bus_width_attr, 0) != 0
            or hip.hipDeviceGetAttribute(ctypes.byref(clk), mem_clock_attr, 0) != 0):
        return None
    gbps = clk.value * 1e3 * bus.value / 8 / 1e9
    return {"bus_width_bits": bus.value, "memory_clock_khz": clk.value, "clock_x_bus_gbps": round(gbps, 1),
            "spec_peak_gbps": HBM_PEAK_GBPS}


def source_commit() -> str | None:
    """The checkout's commit (None where there is no git metadata, as on a
    machine that received a copy of the tree without it)."""
    import subprocess

    try:
        res = subprocess.run(["git", "-C", ROOT, "rev-parse", "HEAD"], capture_output=True, text=True, timeout=20)
    except (OSError, subprocess.SubprocessError):
        return None
    return res.stdout.strip() if res.returncode == 0 else None


def environment(hip: Hip, ks) -> dict:
    """Software versions and the source the library was built from."""
    rocm = None
    try:
        with open("/opt/rocm/.info/version") as f:
            rocm = f.read().strip()
    except OSError:
        pass
    return {"python": platform.python_version(), "torch": torch.__version__, "torch_hip": torch.version.hip,
            "rocm": rocm, **hip.versions(), "library": ks.ks_version(), "commit": source_commit(),
            "host_cpu": _cpu_model(), "host_cpus": os.cpu_count()}


def seeds(wl) -> dict:
    return {k: v for k, v in (("x", wl.seed_x), ("residual", wl.seed_r), ("weight", wl.seed_w),
                              ("outliers", wl.seed_outlier)) if v is not None}


def _cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return platform.processor()


# ---------------------------------------------------------------------------
# HBM traffic from counters
# ---------------------------------------------------------------------------
def load_traffic(workload: str) -> dict | None:
    """Counter-derived HBM bytes per launch, if taken on the current kernel sources."""
    try:
        with open(TRAFFIC_FILE) as f:
            data = json.load(f)
    except (OSError, ValueError):
        return None
    if data.get("kernel_source_hash") != kernel_source_hash():
        return None
    return data.get("workloads", {}).get(workload)


def copy_calibration(mib: int) -> None:
    """Plain device-to-device copies of a known size: the reference the HBM
    counters are scaled by (bytes read = bytes written = MIB MiB per copy)."""
    n = mib << 20
    src = torch.empty(n, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    src.fill_(1)
    torch.cuda.synchronize()
    for _ in range(COPY_REPS):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration_bytes": n, "copies": COPY_REPS}), flush=True)


def _counter_rows(directory: str) -> list[dict]:
    import csv
    import glob

    rows = []
    for path in glob.glob(os.path.join(directory, "**", "*counter_collection.csv"), recursive=True):
        with open(path) as f:
            rows.extend(csv.DictReader(f))
    if not rows:
        raise SystemExit(f"no counter_collection.csv under {directory}")
    return rows


def _per_kernel_kib(directory: str, counter: str) -> dict[str, list[float]]:
    out: dict[str, list[float]] = {}
    for r in _counter_rows(directory):
        if r.get("Counter_Name") == counter:
            out.setdefault(r["Kernel_Name"], []).append(float(r["Counter_Value"]))
    return out


def _median(vals: list[float]) -> float:
    vals = sorted(vals)
    return vals[len(vals) // 2]


def kernel_op(name: str) -> str | None:
    """The operation a demangled kernel name belongs to (None for other kernels)."""
    if "ks::" not in name:
        return None
    for op in ("fused_add_rms_norm", "rms_norm_residual", "rms_norm_backward", "rms_norm", "silu_and_mul", "softmax"):
        if op in name:
            return op
    return None


def traffic_summary(workload: str, fetch_dir: str, write_dir: str, copy_fetch_dir: str, copy_write_dir: str,
                    out: str | None = None) -> None:
    """Counter-derived HBM bytes per launch of each kernel of one workload,
    scaled so that the calibration copy reads and writes exactly its own size,
    into profiles/hbm_traffic.json (entries of other workloads taken on the
    same kernel sources are kept); with `out`, also a markdown summary there."""
    fetch = _per_kernel_kib(fetch_dir, "FETCH_SIZE")
    write = _per_kernel_kib(write_dir, "WRITE_SIZE")
    cf = _per_kernel_kib(copy_fetch_dir, "FETCH_SIZE")
    cw = _per_kernel_kib(copy_write_dir, "WRITE_SIZE")

    def copy_kib(d: dict) -> float:
        return _median([v for k, vs in d.items() if "copy" in k.lower() for v in vs])

    calib_path = os.path.join(copy_fetch_dir, "calibration.json")
    calib_bytes = 256 << 20
    if os.path.exists(calib_path):
        with open(calib_path) as f:
            calib_bytes = json.loads(f.readline())["copy_calibration_bytes"]
    fetch_scale = calib_bytes / (copy_kib(cf) * 1024)
    write_scale = calib_bytes / (copy_kib(cw) * 1024)
    wl = workloads.WORKLOADS[workload]
    esize = wl.torch_dtype.itemsize
    kernels = {}
    for name in fetch:
        op = kernel_op(name)
        if op is None or op not in wl.ops:
            continue
        f = _median(fetch[name]) * 1024 * fetch_scale
        w = _median(write.get(name, [0.0])) * 1024 * write_scale
        alg = algorithmic_bytes(op, wl.rows, wl.hidden, esize)
        kernels[name] = {"op": op, "dispatches": len(fetch[name]), "fetch_bytes": round(f),
                         "write_bytes": round(w), "traffic_bytes": round(f + w), "algorithmic_bytes": alg,
                         "traffic_over_algorithmic": round((f + w) / alg, 4)}
    data = {}
    try:
        with open(TRAFFIC_FILE) as f:
            data = json.load(f)
    except (OSError, ValueError):
        pass
    if data.get("kernel_source_hash") != kernel_source_hash():
        data = {"kernel_source_hash": kernel_source_hash(), "workloads": {}, "kernels": {}}
    data.setdefault("calibration", {})[workload] = {"fetch_scale": round(fetch_scale, 5),
                                                    "write_scale": round(write_scale, 5),
                                                    "copy_bytes": calib_bytes}
    data.setdefault("kernels", {})[workload] = kernels
    per_op: dict[str, int] = {}
    for k in kernels.values():           # an op of several kernels moves their sum
        per_op[k["op"]] = per_op.get(k["op"], 0) + k["traffic_bytes"]
    data.setdefault("workloads", {})[workload] = per_op
    with open(TRAFFIC_FILE, "w") as f:
        json.dump(data, f, indent=1)
    print(json.dumps({"workload": workload, "calibration": data["calibration"][workload], "kernels": kernels},
                     indent=1))
    if out:
        with open(out, "w") as f:
            f.write(traffic_markdown(wl, data["calibration"][workload], kernels, data["kernel_source_hash"],
                                     (fetch_dir, write_dir, copy_fetch_dir, copy_write_dir)))


def traffic_markdown(wl, cal: dict, kernels: dict, source_hash: str, dirs: tuple) -> str:
    fetch_dir, write_dir, cfetch_dir, cwrite_dir = dirs
    run = f"python3 $REPO/bench.py --workload {wl.name} --no-cpu-baseline --steps 64 --warmup 2"
    L = [f"# HBM traffic from counters: {' + '.join(wl.ops)}, {wl.dtype} [{wl.rows},{wl.hidden}]", "",
         f"Workload `{wl.name}`: {wl.describe()}.", "",
         "Four `rocprofv3 --pmc` passes, one counter each (from /tmp with TMPDIR=/tmp), and the summary:", "", "```",
         f"rocprofv3 --pmc FETCH_SIZE --output-format csv -d $REPO/{fetch_dir} -o fetch -- {run}",
         f"rocprofv3 --pmc WRITE_SIZE --output-format csv -d $REPO/{write_dir} -o write -- {run}",
         f"rocprofv3 --pmc FETCH_SIZE --output-format csv -d $REPO/{cfetch_dir} -o cfetch -- python3 $REPO/bench.py "
         "--copy-calibration 256",
         f"rocprofv3 --pmc WRITE_SIZE --output-format csv -d $REPO/{cwrite_dir} -o cwrite -- python3 $REPO/bench.py "
         "--copy-calibration 256",
         f"python bench.py --workload {wl.name} --traffic-summary {fetch_dir} {write_dir} {cfetch_dir} {cwrite_dir} "
         "--out <this file>",
         "```", "",
         f"Calibration: a plain device-to-device copy of {cal['copy_bytes'] >> 20} MiB (`__amd_rocclr_copyBuffer`) "
         f"reads FETCH_SIZE = {cal['copy_bytes'] / 1024 / cal['fetch_scale']:.0f} KiB and WRITE_SIZE = "
         f"{cal['copy_bytes'] / 1024 / cal['write_scale']:.0f} KiB per dispatch, so FETCH_SIZE is scaled by "
         f"{cal['fetch_scale']} and WRITE_SIZE by {cal['write_scale']}.", "",
         "Per launch (median over the profiled dispatches), scaled:", "",
         "| Kernel | Dispatches | Fetch bytes | Write bytes | Traffic bytes | Algorithmic bytes | Traffic / algorithmic |",
         "|---|---|---|---|---|---|---|"]
    for name, k in kernels.items():
        L.append(f"| `{name}` | {k['dispatches']} | {k['fetch_bytes']} | {k['write_bytes']} | {k['traffic_bytes']} | "
                 f"{k['algorithmic_bytes']} | {k['traffic_over_algorithmic']} |")
    models = {"silu_and_mul": "silu_and_mul reads the [R, 2D] input once and writes the [R, D] output, 3 R D elements.",
              "rms_norm_backward": "rms_norm_backward reads x and dy and writes dx, reads the weight and writes its "
                                   "gradient, (3 R H + 2 H) elements; each kernel's row compares its own traffic with "
                                   "the whole op's algorithmic bytes, and the op's traffic is the sum over its two "
                                   "kernels (the row kernel also writes fp32 partial sums of dw, one row per "
                                   "workgroup, which the dw kernel reads back).",
              "rms_norm_residual": "rms_norm_residual reads x and residual and writes out, (3 R H + H) elements "
                                   "with the weight.",
              "softmax": "softmax reads the [R, H] input once and writes the [R, H] output, 2 R H elements."}
    model = next((v for k, v in models.items() if k in wl.ops),
                 "rms_norm reads x and writes out, (2 R H + H) elements; the fused form reads x and residual and "
                 "writes both, (4 R H + H) elements.")
    L += ["", "Algorithmic bytes: " + model, "",
          f"`profiles/hbm_traffic.json` holds these figures with the hash of the kernel sources they were taken on "
          f"(`{source_hash}`, comments and whitespace removed); bench.py reports them as `roofline.traffic` only "
          "while the sources still hash the same."]
    return "\n".join(L) + "\n"


# ---------------------------------------------------------------------------
# kernel-trace summaries (rocprofv3 --kernel-trace output of a bench run)
# ---------------------------------------------------------------------------
def trace_dispatches(directory: str) -> dict[str, dict]:
    """Per kernel name (and grid, where one kernel ran at several sizes): the
    dispatch durations (us) and the first dispatch's resources."""
    import csv
    import glob

    out: dict[str, dict] = {}
    paths = glob.glob(os.path.join(directory, "**", "*kernel_trace.csv"), recursive=True)
    if not paths:
        raise SystemExit(f"no *kernel_trace.csv under {directory}")
    for path in paths:
        with open(path) as f:
            rows = list(csv.DictReader(f))
            grids: dict[str, set] = {}
            for r in rows:
                grids.setdefault(r["Kernel_Name"], set()).add(r.get("Grid_Size_X", ""))
            for r in rows:
                name = r["Kernel_Name"]
                if len(grids[name]) > 1:
                    name = f"{name} [grid {r.get('Grid_Size_X', '')}]"
                k = out.setdefault(name, {
                    "us": [], "resources": {key: r.get(col, "") for key, col in (
                        ("vgpr", "VGPR_Count"), ("agpr", "Accum_VGPR_Count"), ("sgpr", "SGPR_Count"),
                        ("lds", "LDS_Block_Size"), ("scratch", "Scratch_Size"), ("workgroup", "Workgroup_Size_X"),
                        ("grid", "Grid_Size_X"))}})
                k["us"].append((int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1000.0)
    return out


def _dispatch_kind(name: str) -> str:
    op = kernel_op(name)
    if op is not None:
        return op
    for key, kind in (("spin_kernel", "spin (head start)"), ("empty_kernel", "empty (reference)"),
                      ("copy", "copy (setup, reference)")):
        if key in name:
            return kind
    return "other"


def trace_contexts(directory: str) -> dict[str, dict]:
    """The library's dispatches per op, grouped by the kind of dispatch that
    ran just before on the device and by the idle gap between the two (under
    2 us: back to back, as in a graph replay; else the host or the tracer
    kept the device waiting): n, mean and p50 (us)."""
    import csv
    import glob

    rows = []
    for path in glob.glob(os.path.join(directory, "**", "*kernel_trace.csv"), recursive=True):
        with open(path) as f:
            rows += [(int(r["Start_Timestamp"]), int(r["End_Timestamp"]), r["Kernel_Name"]) for r in csv.DictReader(f)]
    rows.sort()
    groups: dict[tuple, list] = {}
    for (_, e0, n0), (s1, e1, n1) in zip(rows, rows[1:]):
        op = kernel_op(n1)
        if op is None:
            continue
        gap = "< 2 us" if (s1 - e0) < 2000 else ">= 2 us"
        groups.setdefault((op, _dispatch_kind(n0), gap), []).append((e1 - s1) / 1000.0)
    return {k: {"n": len(v), "mean": float(np.mean(v)), "p50": float(np.median(v))} for k, v in sorted(groups.items())}


def trace_summary(wl, directory: str, bench_json: str | None, command: str | None) -> str:
    """Markdown summary of a kernel trace of a bench run of workload `wl` (None:
    of a --stream-reference run)."""
    disp = trace_dispatches(directory)
    if wl is None:
        L = ["# Kernel trace: the reference streams (`bench.py --stream-reference`)", ""]
    else:
        L = [f"# Kernel trace: {' + '.join(wl.ops)}, {wl.dtype} [{wl.rows},{wl.hidden}]", "",
             f"Workload `{wl.name}`: {wl.describe()}.", ""]
    if command:
        L += ["Command (from the repository root, on an MI355X; the summary is rendered from its output by "
              "`python bench.py --trace-summary`):", "", "```", "cd /tmp && export TMPDIR=/tmp", command, "```", ""]
    L += ["Per-dispatch kernel durations (us, end minus start timestamp of each dispatch in the trace) and each "
          "kernel's resources:", "",
          "| Kernel | Dispatches | min | p50 | mean | p95 | p99 | max | VGPR | AGPR | SGPR | LDS B | scratch B "
          "| workgroup | grid threads |", "|---|---|---|---|---|---|---|---|---|---|---|---|---|---|---|"]
    per_op: dict[str, dict] = {}
    for name, k in sorted(disp.items(), key=lambda kv: (kernel_op(kv[0]) is None, kv[0])):
        d = distribution(k["us"])
        short = name if len(name) < 130 else name[:100] + "..." + name[name.rfind(" ["):] if " [grid" in name else \
            name if len(name) < 110 else name[:100] + "..."
        res = k["resources"]
        L.append(f"| `{short}` | {d['n']} | {d['min']:.2f} | {d['p50']:.2f} | {d['mean']:.2f} | {d['p95']:.2f} | "
                 f"{d['p99']:.2f} | {d['max']:.2f} | {res['vgpr']} | {res['agpr']} | {res['sgpr']} | {res['lds']} | "
                 f"{res['scratch']} | {res['workgroup']} | {res['grid']} |")
        op = kernel_op(name)
        if wl is not None and op is not None and op in wl.ops:
            per_op.setdefault(op, {"mean": 0.0, "p50": 0.0, "kernels": 0})
            per_op[op]["mean"] += d["mean"]   # an op of several kernels takes their sum
            per_op[op]["p50"] += d["p50"]
            per_op[op]["kernels"] += 1
    L += ["", "The library's kernels come first; the rest are the bench's own setup and reference kernels "
          "(input copies, the empty, spin and copy reference streams)."]
    if wl is None:
        return "\n".join(L) + "\n"
    esize = wl.torch_dtype.itemsize
    line = None
    if bench_json:
        with open(bench_json) as f:
            line = json.loads(f.read().strip().splitlines()[-1])
    L += ["", "Per op: the trace's durations against the uninstrumented bench run of the same command "
          "(kernel-dispatch events per call, and the graph launch period):", "",
          "| Op | algorithmic bytes | trace mean us | trace p50 us | GB/s (trace mean) | bench kernel mean us "
          "| bench kernel p50 us | bench graph us/call | GB/s (bench kernel mean) | bench vs trace mean |",
          "|---|---|---|---|---|---|---|---|---|---|"]
    for op in wl.ops:
        alg = algorithmic_bytes(op, wl.rows, wl.hidden, esize)
        t = per_op.get(op)
        if t is None:
            continue
        row = f"| {op} | {alg} | {t['mean']:.3f} | {t['p50']:.3f} | {alg / t['mean'] / 1e3:.0f} |"
        if line is not None and op in line.get("per_op", {}):
            b = line["per_op"][op]
            km = b["kernel_us"]["mean"]
            row += (f" {km:.3f} | {b['kernel_us']['p50']:.3f} | {b['us_per_call']:.3f} | {alg / km / 1e3:.0f} | "
                    f"{100 * (km - t['mean']) / t['mean']:+.1f}% |")
        else:
            row += " | | | | |"
        L.append(row)
    ctx = trace_contexts(directory)
    if line is not None:
        rf = line["roofline"]
        alg = algorithmic_bytes(rf["kernel"], wl.rows, wl.hidden, esize)
        text = (f"The bench line's roofline: dominant kernel {rf['kernel']}, {rf['achieved']} GB/s, frac "
                f"{rf['frac']} (algorithmic bytes over the mean of the per-call kernel-dispatch event durations).  "
                f"The same bytes over the trace's mean duration give frac "
                f"{alg / per_op[rf['kernel']]['mean'] / 1e3 / HBM_PEAK_GBPS:.4f}.")
        timed = ctx.get((rf["kernel"], rf["kernel"], ">= 2 us"))
        kernels = [n for n in disp if kernel_op(n) == rf["kernel"]]
        if timed is not None and timed["n"] >= 8 and len(kernels) == 1:   # an op of one kernel per call
            text += (f"  Over the dispatches of the kind the bench times (a call after a call of the same op, "
                     f"with an idle gap of 2 us or more: {timed['n']} dispatches, mean {timed['mean']:.3f} us) "
                     f"they give frac {alg / timed['mean'] / 1e3 / HBM_PEAK_GBPS:.4f}.")
        text += ("  The tracer adds a little to each dispatch, so its durations run slightly longer than the "
                 "uninstrumented ones.")
        L += ["", text]
    if ctx:
        L += ["", "The library's dispatches by what ran just before them on the device (a kernel of an op, the "
              "head-start spin, the setup and reference kernels) and by the idle gap in between.  The graph "
              "replays run back to back (gap under 2 us); the per-call timed calls follow another call of the "
              "same op, with the gaps the tracer's own work adds; the untimed lead call of each timed run "
              "follows the spin and reads a copy that is still in the Infinity Cache.  The trace's mean mixes "
              "these; the bench's kernel mean is the timed calls alone:", "",
              "| Op | after | gap | dispatches | mean us | p50 us |", "|---|---|---|---|---|---|"]
        L += [f"| {op} | {prev} | {gap} | {v['n']} | {v['mean']:.3f} | {v['p50']:.3f} |"
              for (op, prev, gap), v in ctx.items() if v["n"] >= 8]
    if line is not None:
        L += ["", f"Library: {line.get('env', {}).get('library', '?')}; kernel sources hash "
              f"`{line.get('kernel_source_hash', '?')}`."]
    return "\n".join(L) + "\n"


# ---------------------------------------------------------------------------
# regression gate: cases matched by (op, dtype, rows, hidden)
# ---------------------------------------------------------------------------
def case_key(case: dict) -> tuple:
    return (case["op"], case["dtype"], int(case["rows"]), int(case["hidden"]))


def cases_from(wl, per_op: dict) -> list[dict]:
    return [{"op": op, "dtype": wl.dtype, "rows": wl.rows, "hidden": wl.hidden,
             "us_per_call": v["us_per_call"], "gbps": v["gbps"]} for op, v in per_op.items()]


def regressions(current: list[dict], baseline: list[dict], max_percent: float) -> list[dict]:
    """Cases present in both lists whose time per call grew by more than max_percent."""
    base = {case_key(c): c for c in baseline}
    out = []
    for c in current:
        b = base.get(case_key(c))
        if b is None or b["us_per_call"] <= 0:
            continue
        pct = 100.0 * (c["us_per_call"] - b["us_per_call"]) / b["us_per_call"]
        if pct > max_percent:
            out.append({"case": list(case_key(c)), "baseline_us": b["us_per_call"], "us": c["us_per_call"],
                        "regression_percent": round(pct, 2)})
    return out


def finish_cases(args, cases: list[dict]) -> None:
    """Write the per-case JSON and apply the regression gate (exit status 2)."""
    if args.json_out:
        with open(args.json_out, "w") as f:
            json.dump({"cases": cases, "kernel_source_hash": kernel_source_hash()}, f, indent=1)
    if args.baseline:
        with open(args.baseline) as f:
            base = json.load(f)["cases"]
        bad = regressions(cases, base, args.max_regression_percent)
        matched = sum(1 for c in cases if case_key(c) in {case_key(b) for b in base})
        log(f"regression gate: {matched} matching cases, {len(bad)} slower by more than "
            f"{args.max_regression_percent:g}%")
        for r in bad:
            log("  regression", r)
        if bad:
            sys.exit(2)


# ---------------------------------------------------------------------------
# modes
# ---------------------------------------------------------------------------
def sweep_set(dtypes: list[str]) -> list:
    """Every workload, plus the RMSNorm workloads C1, C2 and C3b in the other
    requested dtypes (same shapes, distributions and seeds) where no workload
    already covers that (op, dtype, shape)."""
    out = list(workloads.WORKLOADS.values())
    keys = {(wl.ops, wl.dtype, wl.rows, wl.hidden) for wl in out}
    for name in ("C1", "C2", "C3b"):
        for tag in dtypes:
            v = workloads.with_dtype(workloads.WORKLOADS[name], tag)
            key = (v.ops, v.dtype, v.rows, v.hidden)
            if key not in keys:
                keys.add(key)
                out.append(v)
    return out


def sweep_workloads(args, ks, oracle_mod, hip: Hip) -> None:
    """Every workload of the pages' benchmark set (and the dtype variants):
    parity, then per-op timing."""
    cases = []
    lines = ["| Workload | Op | dtype | rows x hidden | us/call (graph) | kernel p50 us | GB/s (kernel mean) "
             "| % of 8 TB/s | rotation MiB | plan (team x pieces, hints) | max ulp | exact |",
             "|---|---|---|---|---|---|---|---|---|---|---|---|"]
    for wl in sweep_set([t for t in args.sweep_dtypes.split(",") if t]):
        log("generating", wl.name, wl.describe())
        inp = workloads.make_inputs(wl)
        parity = parity_gate(wl, inp, ks, oracle_mod)
        res = measure(wl, inp, ks, args, hip)
        cases.extend(cases_from(wl, res["per_op"]))
        for op in wl.ops:
            p = res["per_op"][op]
            pl = p["plan"]
            path = {0: "", 1: "generic ", 2: "split "}.get(pl["path"], "?")
            plan = (f"{path}{pl['threads_per_row']}x{pl['vectors_per_thread']} "
                    f"nt{pl['load_nt']}{pl['store_nt']} lds{pl['weight_lds']}")
            lines.append(f"| {wl.name} | {op} | {DTYPE_TAG[wl.dtype]} | {wl.rows}x{wl.hidden} | {p['us_per_call']:.3f} | "
                         f"{p['kernel_us']['p50']:.2f} | {p['gbps']:.0f} | {100 * p['frac_of_peak']:.1f} | "
                         f"{res['rotation_mib']:.0f} | {plan} | {parity[op]['max_ulp']} | "
                         f"{parity[op]['exact_match']:.6f} |")
            log(lines[-1])
        del inp
    table = "\n".join(lines)
    print(table, flush=True)
    if args.out:
        with open(args.out, "w") as f:
            f.write(table + "\n")
    finish_cases(args, cases)


def main() -> None:
    args = parse()
    if args.trace_summary:
        wl = None if args.stream_reference else workloads.WORKLOADS[args.workload]
        if wl is not None and args.dtype:
            wl = workloads.with_dtype(wl, args.dtype)
        text = trace_summary(wl, args.trace_summary, args.trace_bench, args.trace_command)
        if args.out:
            with open(args.out, "w") as f:
                f.write(text)
        else:
            print(text, end="")
        return
    if args.traffic_summary:
        traffic_summary(args.workload, *args.traffic_summary, out=args.out)
        return
    if args.gpus != 1:
        print(f"bench.py measures one GPU; --gpus {args.gpus} is not supported "
              "(rows shard across GPUs with no communication; see the design notes).", file=sys.stderr)
        sys.exit(2)
    if not torch.cuda.is_available():
        fail("no HIP device visible")
    if args.copy_calibration:
        copy_calibration(args.copy_calibration)
        return

    import oracle
    import rmsnorm_row_normalisation_amd as ks

    dev = torch.cuda.get_device_properties(0)
    log("device", dev.name, getattr(dev, "gcnArchName", "?"), "CUs", dev.multi_processor_count)
    if args.steps < 1:
        fail("--steps must be at least 1")
    hip = Hip()
    if args.stream_reference:
        table = stream_reference_table(hip)
        if args.json_out:
            with open(args.json_out, "w") as f:
                json.dump(table, f, indent=1)
        return
    if args.wave_timeline:
        res = wave_timeline(hip)
        text = wave_timeline_markdown(res)
        print(text, end="", flush=True)
        if args.out:
            with open(args.out, "w") as f:
                f.write(text)
        if args.json_out:
            with open(args.json_out, "w") as f:
                json.dump(res, f, indent=1)
        return
    if args.sweep_workloads:
        sweep_workloads(args, ks, oracle, hip)
        return

    wl = workloads.WORKLOADS[args.workload]
    if args.dtype:
        wl = workloads.with_dtype(wl, args.dtype)
    if args.op:
        if args.op not in wl.ops:
            fail(f"workload {wl.name} has no op {args.op} (its ops: {', '.join(wl.ops)})", 2)
        wl = workloads.with_ops(wl, (args.op,))
    log("generating inputs", wl.describe())
    inp = workloads.make_inputs(wl)
    try:
        parity = parity_gate(wl, inp, ks, oracle)
    except AssertionError as exc:
        fail(f"parity gate failed, nothing timed: {exc}")
    log("parity", parity)
    res = measure(wl, inp, ks, args, hip)
    per_op = res["per_op"]
    log("per op", per_op)

    dominant = max(wl.ops, key=lambda op: per_op[op]["kernel_us"]["mean"])
    traffic = load_traffic(wl.name)
    kus = per_op[dominant]["kernel_us"]
    roofline = {"bound": "hbm", "kernel": dominant,
                "achieved": per_op[dominant]["gbps"], "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                "frac": round(per_op[dominant]["gbps"] / HBM_PEAK_GBPS, 4),
                "traffic": (traffic or {}).get(dominant),
                "bytes": per_op[dominant]["bytes"], "kernel_us_mean": kus["mean"], "kernel_us_p50": kus["p50"],
                "method": f"algorithmic bytes / mean kernel duration over {kus['n']} calls, each timed by the "
                          "runtime's kernel-dispatch events (ks_time_next_call) on the launch stream"}
    reps, tail = divmod(res["steps"], res["nsets"])
    timing_mode = (f"exactly {res['steps']} steps: HIP graph of {res['nsets']} steps replayed {reps} times"
                   + (f" plus a graph of {tail}" if tail else "")
                   + "; per op: the same with that op's launches alone (median of three timed regions) and "
                     "per-call kernel-dispatch events")
    line = {
        "metric": METRIC, "value": round(res["value"], 1), "unit": "GB/s", "n_gpus": 1, "steps": res["steps"],
        "warmup": args.warmup, "ms_per_step": round(res["ms_per_step"], 6), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": DTYPE_TAG[wl.dtype], "data": "synthetic",
        "config": {"workload": wl.describe(), "name": wl.name, "ops": list(wl.ops), "rows": wl.rows,
                   "hidden": wl.hidden, "eps": wl.eps, "seeds": seeds(wl), "timing": timing_mode,
                   "cache": f"cold: {res['nsets']} rotating copies ({res['rotation_mib']:.0f} MiB)"},
        "frac_of_peak": round(res["value"] / HBM_PEAK_GBPS, 4),
        "per_op": per_op,
        "roofline": roofline,
        "stream_reference": stream_reference(hip, res["tensor_bytes"]),
        "parity": parity,
        "device": {"name": dev.name, "arch": getattr(dev, "gcnArchName", "?"), "cus": dev.multi_processor_count,
                   "memory": memory_interface()},
        "env": environment(hip, ks),
        "kernel_source_hash": kernel_source_hash(),
    }
    if not args.no_cpu_baseline:
        log(f"timing the CPU oracle for about {args.cpu_seconds:.0f} s")
        line["cpu_baseline"] = cpu_baseline(wl, inp, oracle, args.cpu_seconds, res["step_bytes"])
    else:
        line["cpu_baseline"] = None
    print(json.dumps(line), flush=True)
    finish_cases(args, cases_from(wl, per_op))


if __name__ == "__main__":
    main()
