"""Helpers for GPU parity tests: run the HIP path and the CPU oracle on the
same seeded inputs and compare them with the gates in compare.py."""
from __future__ import annotations

import sys

import torch

import oracle
import rmsnorm_row_normalisation_amd as ks
from compare import FP32_MAX_ULP, check_bitexact, check_normalised

# Below this many elements a single 1-ulp difference already breaks a 99.9%
# exact-match rate, so small cases rely on the 1-ulp bound alone.
EXACT_RATE_MIN_ELEMS = 20000
EXACT_RATE = 0.999


def say(*parts) -> None:
    print("[gpu-case]", *parts, file=sys.stderr, flush=True)


def require_gpu() -> None:
    import pytest

    if not torch.cuda.is_available():
        pytest.skip("no HIP device visible")
    ks.lib()   # fails loudly when the library is not built


def gpu_run(op: str, inp: dict, eps: float, plan=None, stream: torch.cuda.Stream | None = None,
            offset: int = 0):
    """Run one op on cuda:0.  offset > 0 places every tensor `offset` elements into a
    larger allocation, so the buffers are not 16-byte aligned.  Returns CPU tensors."""
    def dev(t):
        if offset == 0:
            return t.cuda()
        buf = torch.empty(t.numel() + offset, dtype=t.dtype, device="cuda")
        view = buf[offset:].view(t.shape)
        view.copy_(t.cuda())
        return view

    x, w = dev(inp["x"]), dev(inp["weight"])
    ctx = torch.cuda.stream(stream) if stream is not None else torch.cuda.stream(torch.cuda.current_stream())
    with ctx:
        if op == "rms_norm":
            y = ks.rms_norm(x, w, eps, plan=plan)
            res = None
        else:
            r = dev(inp["residual"])
            ks.fused_add_rms_norm(x, r, w, eps, plan=plan)
            y, res = x, r
    torch.cuda.synchronize()
    return y.cpu(), (res.cpu() if res is not None else None)


def oracle_run(op: str, inp: dict, eps: float):
    if op == "rms_norm":
        return oracle.rms_norm(inp["x"], inp["weight"], eps), None
    return oracle.fused_add_rms_norm(inp["x"], inp["residual"], inp["weight"], eps)


def check_outputs(op: str, got, ref, exact_rate: bool | None = None):
    y, r = got
    ry, rr = ref
    if exact_rate is None:
        exact_rate = y.numel() >= EXACT_RATE_MIN_ELEMS
    st = check_normalised(y, ry, EXACT_RATE if exact_rate else None, fp32_max_ulp=FP32_MAX_ULP)
    if op != "rms_norm":
        check_bitexact(r, rr)
    return st


def check_case(name: str, op: str, inp: dict, eps: float, plan=None, offset: int = 0,
               stream: torch.cuda.Stream | None = None, exact_rate: bool | None = None):
    say(name, op, tuple(inp["x"].shape), inp["x"].dtype, "plan" if plan is not None else "policy",
        f"offset={offset}")
    got = gpu_run(op, inp, eps, plan=plan, offset=offset, stream=stream)
    ref = oracle_run(op, inp, eps)
    return check_outputs(op, got, ref, exact_rate)


HINTS = ((0, 0, 0), (1, 1, 0), (0, 1, 0), (1, 1, 1))   # compiled (load_nt, store_nt, weight_lds)


WIDE_VPT = 16            # the 16-piece builds (RMSNorm and its residual forms, teams of 32..128 lanes)
WIDE_VPT_TPRS = (32, 64, 128)


def all_plans(dtype: torch.dtype, hidden: int, aligned: bool = True) -> list:
    """Every compiled plan of rms_norm and the fused form that covers rows of
    this size (the library rejects the rest)."""
    es = torch.empty(0, dtype=dtype).element_size()
    row_bytes = hidden * es
    vec_elems = 16 // es
    plans = []
    if aligned and row_bytes % 16 == 0:
        tpr = 8
        while tpr <= 1024:
            maxv = 8
            for vpt in list(range(1, maxv + 1)) + ([WIDE_VPT] if tpr in WIDE_VPT_TPRS else []):
                if tpr * vpt * 16 >= row_bytes:
                    block = max(256, tpr)
                    for lnt, snt, wlds in HINTS:
                        plans.append(ks.Plan(path=0, threads_per_row=tpr, vectors_per_thread=vpt,
                                             elems_per_access=vec_elems, rows_per_block=block // tpr,
                                             block_threads=block, load_nt=lnt, store_nt=snt, weight_lds=wlds))
            tpr *= 2
    for tpr in (8, 64, 256, 1024):
        block = 1024 if tpr == 1024 else 256
        epas = [1] + ([vec_elems] if aligned and row_bytes % 16 == 0 else [])
        for epa in epas:
            plans.append(ks.Plan(path=1, threads_per_row=tpr, vectors_per_thread=0, elems_per_access=epa,
                                 rows_per_block=block // tpr, block_threads=block))
    return plans
