"""Benchmark: RMSNorm and fused residual-add RMSNorm on one MI355X (the
default workload), and the SwiGLU (S*) and softmax (X*) workloads.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload C3b]
    python bench.py --sweep-workloads [--out FILE]      # every workload, one table

One step is one pass of the whole path over one batch: ks_rms_norm on the
batch, then ks_fused_add_rms_norm on it (both at 2048 x 4096 bf16 by
default; x ~ N(0,1) with 1% of elements x100, residual ~ N(0,0.5), weight ~
U(0.5,1.5), eps = 1e-5).  The inputs are resident in HBM before timing.

Cache state: the 256 MiB Infinity Cache and the L2s would hold a 64 MiB
working set, so the steps rotate over enough copies of the batch (1 GiB by
default) that every step reads data last touched more than a cache's worth
of traffic ago.  Numbers are therefore HBM numbers, not cache numbers.

Timing:
  * whole job (``value``): one rotation of steps over the copies is captured
    into a HIP graph (no host launch overhead inside the timed region) and
    replayed until K steps have run, between a synchronize and two events on
    the launch stream;
  * per kernel (``per_op``, ``roofline``): the same, with a graph holding only
    that op's launches, back to back (the median of three timed regions); the
    average launch period includes the short gap between consecutive kernels,
    so it is an upper bound on the kernel's own duration (rocprofv3's kernel
    trace of the same run gives the duration alone);
  * ``copy_reference``: one batch-sized tensor streamed through the runtime's
    elementwise kernel (out = -x: one read, one write), timed the same way:
    what a plain read+write stream of that size achieves on this GPU;
  * ``copy_ceiling``: a 1 GiB read + 1 GiB write stream by the runtime's
    elementwise kernel (out = -x), where launch costs vanish: what a plain
    read+write stream reaches on this GPU (context, not the denominator:
    fractions are of the 8 TB/s spec).
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
    ap.add_argument("--rotate-mib", type=int, default=1024, help="total size of the rotating input copies")
    ap.add_argument("--cpu-seconds", type=float, default=10.0, help="budget for the CPU oracle baseline")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--sweep-workloads", action="store_true",
                    help="measure every workload (per op) and print a markdown table instead of the bench line")
    ap.add_argument("--out", default=None, help="with --sweep-workloads: also write the table to this file")
    ap.add_argument("--json-out", default=None, help="also write the per-case results (JSON) to this file")
    ap.add_argument("--baseline", default=None,
                    help="a previous --json-out file: exit with status 2 if any matching case got slower "
                         "by more than --max-regression-percent")
    ap.add_argument("--max-regression-percent", type=float, default=10.0)
    ap.add_argument("--copy-calibration", type=int, metavar="MIB", default=0,
                    help="only run device-to-device copies of MIB MiB (the counter calibration run) and exit")
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

    def timed_graph(self, body, per_rotation: int, reps: int, repeats: int = 1) -> float:
        """Capture body(i) for i in range(per_rotation) into a HIP graph and replay
        it `reps` times between two events on the launch stream; milliseconds.
        With repeats > 1 the timed region runs that many times and the median
        is returned."""
        graph = torch.cuda.CUDAGraph()
        times = []
        with torch.cuda.stream(self.stream):
            with torch.cuda.graph(graph, stream=self.stream):
                for i in range(per_rotation):
                    body(i)
            graph.replay()                                   # untimed
            torch.cuda.synchronize()
            for _ in range(repeats):
                ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                ev0.record(self.stream)
                for _ in range(reps):
                    graph.replay()
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

    def copy_reference(self, reps: int) -> dict:
        """A read+write stream of one batch-sized tensor per launch by the
        runtime's elementwise kernel (out = -x; the DMA copy behind
        ``Tensor.copy_`` is slower)."""
        n = self.nsets
        srcs = [s.get("x", s.get("fx", s.get("sx", s.get("mx", s.get("ox", s.get("bx")))))) for s in self.sets]
        dsts = [torch.empty_like(t) for t in srcs]
        ms = self.timed_graph(lambda i: torch.neg(srcs[i % n], out=dsts[i % n]), n, reps)
        del dsts
        us = ms * 1e3 / (n * reps)
        gbps = 2 * self.tensor_bytes / (us * 1e-6) / 1e9
        return {"bytes": 2 * self.tensor_bytes, "us_per_copy": round(us, 3), "gbps": round(gbps, 1),
                "frac_of_peak": round(gbps / HBM_PEAK_GBPS, 4)}


def measure(wl, inp, ks, args) -> dict:
    """Whole-step and per-op throughput of one workload."""
    esize = torch.empty(0, dtype=wl.torch_dtype).element_size()
    op_bytes = {op: algorithmic_bytes(op, wl.rows, wl.hidden, esize) for op in wl.ops}
    rig = Rig(wl, inp, ks, args.rotate_mib)
    log(f"{wl.name}: {rig.nsets} rotating copies, {rig.rotation_mib:.0f} MiB")
    reps = max(1, -(-args.steps // rig.nsets))
    steps = reps * rig.nsets
    rig.warmup(args.warmup)
    total_ms = rig.timed_graph(lambda i: [rig.launch(op, i) for op in wl.ops], rig.nsets, reps)
    per_op = {}
    for op in wl.ops:
        # per-op figures: median of three timed regions (run-to-run spread is a few %)
        ms = rig.timed_graph(lambda i, op=op: rig.launch(op, i), rig.nsets, reps, repeats=3)
        us = ms * 1e3 / steps
        gbps = op_bytes[op] / (us * 1e-6) / 1e9
        per_op[op] = {"us_per_call": round(us, 3), "bytes": op_bytes[op], "gbps": round(gbps, 1),
                      "frac_of_peak": round(gbps / HBM_PEAK_GBPS, 4),
                      "plan": ks.get_plan(op, wl.torch_dtype, wl.hidden // 2 if op == "silu_and_mul" else wl.hidden,
                                          wl.rows, workspace=op == "softmax").as_dict()}
    copy = rig.copy_reference(reps)
    ms_per_step = total_ms / steps
    result = {"steps": steps, "reps": reps, "nsets": rig.nsets, "rotation_mib": rig.rotation_mib,
              "ms_per_step": ms_per_step, "step_bytes": sum(op_bytes.values()),
              "value": sum(op_bytes.values()) / (ms_per_step * 1e-3) / 1e9, "per_op": per_op,
              "copy_reference": copy}
    del rig
    torch.cuda.empty_cache()
    return result


# ---------------------------------------------------------------------------
# CPU baseline
# ---------------------------------------------------------------------------
def cpu_baseline(wl, inp, oracle_mod, budget_s: float, step_bytes: int) -> dict:
    """The oracle as it stands, single-threaded on a host core, on whole steps of the workload."""
    t0 = time.perf_counter()
    steps = 0
    while True:
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
        steps += 1
        el = time.perf_counter() - t0
        if el >= budget_s:
            break
    return {"value": round(steps * step_bytes / el / 1e9, 4), "unit": "GB/s", "cores": 1, "kind": "oracle",
            "sample": f"{steps} full steps ({' + '.join(wl.ops)} on the whole [{wl.rows},{wl.hidden}] batch) "
                      f"in {el:.1f} s, single thread",
            "us_per_step": round(el / steps * 1e6, 1), "host_cpus": os.cpu_count(),
            "host_cpu": _cpu_model()}


def memory_interface() -> dict | None:
    """The device's reported memory bus width and clock (hipDeviceGetAttribute)
    and their product (bytes per reported clock), as context next to the
    8 TB/s spec peak that the fractions use.  The product is not a peak: the
    HBM3E interface moves several transfers per reported clock (8 TB/s over
    2048 GB/s is about 4)."""
    try:
        hip = ctypes.CDLL("libamdhip64.so")
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


def copy_ceiling(mib: int = 1024, reps: int = 8) -> dict:
    """A read+write stream of MIB MiB each way by the runtime's elementwise
    kernel (out = -x over bf16, a shader kernel: the DMA copy behind
    ``Tensor.copy_`` is slower), on the same clock as the kernels, at a size
    where launch costs vanish: what a plain read+write stream reaches on this
    device.  Context for the fractions of the 8 TB/s spec, never their
    denominator."""
    n = mib << 20
    src = torch.ones(n // 2, dtype=torch.bfloat16, device="cuda")
    dst = torch.empty_like(src)
    torch.neg(src, out=dst)
    torch.cuda.synchronize()
    times = []
    for _ in range(3):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            torch.neg(src, out=dst)
        e1.record()
        torch.cuda.synchronize()
        times.append(e0.elapsed_time(e1) / reps)
    ms = float(np.median(times))
    del src, dst
    torch.cuda.empty_cache()
    gbps = 2 * n / (ms * 1e-3) / 1e9
    return {"op": "torch.neg, bf16", "bytes": 2 * n, "ms_per_pass": round(ms, 4), "gbps": round(gbps, 1),
            "frac_of_peak": round(gbps / HBM_PEAK_GBPS, 4)}


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


def traffic_summary(workload: str, fetch_dir: str, write_dir: str, copy_fetch_dir: str, copy_write_dir: str) -> None:
    """Counter-derived HBM bytes per launch of each kernel of one workload,
    scaled so that the calibration copy reads and writes exactly its own size.
    Entries of other workloads taken on the same kernel sources are kept."""
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
def sweep_workloads(args, ks, oracle_mod) -> None:
    """Every workload of the pages' benchmark set: parity, then per-op timing."""
    cases = []
    lines = ["| Workload | Op | dtype | rows x hidden | us/call | GB/s | % of 8 TB/s | copy ref GB/s | rotation MiB "
             "| plan (team x pieces, hints) | max ulp | exact |",
             "|---|---|---|---|---|---|---|---|---|---|---|---|"]
    for name, wl in workloads.WORKLOADS.items():
        log("generating", name, wl.describe())
        inp = workloads.make_inputs(wl)
        parity = parity_gate(wl, inp, ks, oracle_mod)
        res = measure(wl, inp, ks, args)
        cases.extend(cases_from(wl, res["per_op"]))
        for op in wl.ops:
            p = res["per_op"][op]
            pl = p["plan"]
            path = {0: "", 1: "generic ", 2: "split "}.get(pl["path"], "?")
            plan = (f"{path}{pl['threads_per_row']}x{pl['vectors_per_thread']} "
                    f"nt{pl['load_nt']}{pl['store_nt']} lds{pl['weight_lds']}")
            lines.append(f"| {name} | {op} | {DTYPE_TAG[wl.dtype]} | {wl.rows}x{wl.hidden} | {p['us_per_call']:.3f} | "
                         f"{p['gbps']:.0f} | {100 * p['frac_of_peak']:.1f} | {res['copy_reference']['gbps']:.0f} | "
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
    if args.traffic_summary:
        traffic_summary(args.workload, *args.traffic_summary)
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
    if args.sweep_workloads:
        sweep_workloads(args, ks, oracle)
        return

    wl = workloads.WORKLOADS[args.workload]
    log("generating inputs", wl.describe())
    inp = workloads.make_inputs(wl)
    try:
        parity = parity_gate(wl, inp, ks, oracle)
    except AssertionError as exc:
        fail(f"parity gate failed, nothing timed: {exc}")
    log("parity", parity)
    res = measure(wl, inp, ks, args)
    per_op = res["per_op"]
    log("per op", per_op)

    dominant = max(wl.ops, key=lambda op: per_op[op]["us_per_call"])
    traffic = load_traffic(args.workload)
    roofline = {"bound": "hbm", "kernel": dominant,
                "achieved": per_op[dominant]["gbps"], "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                "frac": round(per_op[dominant]["gbps"] / HBM_PEAK_GBPS, 4),
                "traffic": (traffic or {}).get(dominant)}
    timing_mode = (f"HIP graph replay, {res['reps']} replays of {res['nsets']} steps; per op: graphs of "
                   "back-to-back launches of that op, median of three timed regions")
    line = {
        "metric": METRIC, "value": round(res["value"], 1), "unit": "GB/s", "n_gpus": 1, "steps": res["steps"],
        "warmup": args.warmup, "ms_per_step": round(res["ms_per_step"], 6), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": DTYPE_TAG[wl.dtype], "data": "synthetic",
        "config": {"workload": wl.describe(), "ops": list(wl.ops), "rows": wl.rows, "hidden": wl.hidden,
                   "eps": wl.eps, "timing": timing_mode,
                   "cache": f"cold: {res['nsets']} rotating copies ({res['rotation_mib']:.0f} MiB)"},
        "frac_of_peak": round(res["value"] / HBM_PEAK_GBPS, 4),
        "per_op": per_op,
        "roofline": roofline,
        "copy_reference": res["copy_reference"],
        "copy_ceiling": copy_ceiling(),
        "parity": parity,
        "device": {"name": dev.name, "arch": getattr(dev, "gcnArchName", "?"), "cus": dev.multi_processor_count,
                   "memory": memory_interface()},
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
