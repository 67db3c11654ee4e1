"""Seeded synthetic inputs shared by the tests, the smoke check and the benchmark.

RMSNorm workloads (C*), SwiGLU workloads (S*: 512x8192 -> 512x4096 bf16 as in
the kernscope SwiGLU baseline, and the 7B-model FFN width 11008 at sequence
2048 from the Triton Kernels benchmark table) and softmax workloads (X*: the
kernscope softmax measurements at 512 rows of 1024, 128 and 8192 bf16, its
65536-column fp16 accumulation case, and the RMSNorm headline shape 2048x4096
as an HBM-bound softmax batch) and out-of-place residual RMSNorm workloads
(R*: the Triton Kernels README usage example, fp16 [2048, 4096] with unit
weight, and the headline shape in bf16) and the RMSNorm backward at the
headline shape (B1; its incoming gradient dy ~ N(0, 1), drawn as "residual").  The softmax pages state no input
distribution; N(0, 1) logits are used, as in their usage example.

This module draws random numbers and nothing else: it holds none of the
normalisation's arithmetic, so both the CPU oracle and the GPU path can take
their inputs from it without sharing any of the method.

Recipe: one ``numpy.random.default_rng(seed)`` stream per tensor; values are
drawn in fp32, scaled and shifted in fp32, optional outliers are applied in
fp32, and the result is rounded ONCE to the storage dtype by torch's CPU cast
(round to nearest, ties to even).  Both sides therefore see identical bits.

The shapes and distributions are the ones the benchmark pages use for this
operator: random-normal activations with hidden sizes 1024, 1536, 4096, 8192
and 16384, and row counts from one decode token up to long prefills.
"""
from __future__ import annotations

from dataclasses import dataclass, field, replace

import numpy as np
import torch

DTYPES = {"float32": torch.float32, "float16": torch.float16, "bfloat16": torch.bfloat16}


@dataclass(frozen=True)
class Dist:
    """A value distribution: ``normal`` (mean, std) or ``uniform`` (low, high)."""

    kind: str
    a: float
    b: float

    def draw(self, rng: np.random.Generator, n: int) -> np.ndarray:
        if self.kind == "normal":
            return rng.standard_normal(n, dtype=np.float32) * np.float32(self.b) + np.float32(self.a)
        if self.kind == "uniform":
            return rng.random(n, dtype=np.float32) * np.float32(self.b - self.a) + np.float32(self.a)
        raise ValueError(self.kind)

    def __str__(self) -> str:
        return f"N({self.a:g},{self.b:g})" if self.kind == "normal" else f"U({self.a:g},{self.b:g})"


def normal(mean: float, std: float) -> Dist:
    return Dist("normal", mean, std)


def uniform(low: float, high: float) -> Dist:
    return Dist("uniform", low, high)


@dataclass(frozen=True)
class Workload:
    name: str
    ops: tuple[str, ...]
    dtype: str
    rows: int
    hidden: int
    x: Dist
    weight: Dist | None
    eps: float
    seed_x: int
    seed_w: int | None
    residual: Dist | None = None
    seed_r: int | None = None
    outlier_frac: float = 0.0
    outlier_scale: float = 1.0
    seed_outlier: int | None = None
    note: str = field(default="", compare=False)

    @property
    def torch_dtype(self) -> torch.dtype:
        return DTYPES[self.dtype]

    def describe(self) -> str:
        ops = " + ".join(self.ops)
        parts = [f"{ops} {self.dtype} [{self.rows},{self.hidden}]", f"x ~{self.x}"]
        if self.outlier_frac:
            parts[-1] += f" with {self.outlier_frac:.0%} of elements x{self.outlier_scale:g}"
        if self.residual is not None and ("fused_add_rms_norm" in self.ops or "rms_norm_residual" in self.ops):
            parts.append(f"residual ~{self.residual}")
        if self.residual is not None and "rms_norm_backward" in self.ops:
            parts.append(f"dy ~{self.residual}")
        if self.weight is not None:
            parts.append(f"weight ~{self.weight}")
            parts.append(f"eps={self.eps:g}")
        return ", ".join(parts)


RMS, FUSED, SWIGLU, SOFTMAX = "rms_norm", "fused_add_rms_norm", "silu_and_mul", "softmax"
RESIDUAL, BACKWARD = "rms_norm_residual", "rms_norm_backward"

WORKLOADS: dict[str, Workload] = {
    # small case the oracle finishes in milliseconds
    "C1": Workload("C1", (RMS,), "bfloat16", 128, 1024, normal(0, 1), normal(1, 0.1), 1e-6, 1001, 1003),
    "C2": Workload("C2", (RMS, FUSED), "bfloat16", 512, 4096, normal(0, 1), normal(1, 0.1), 1e-6, 2001, 2003,
                   residual=normal(0, 1), seed_r=2002),
    "C3": Workload("C3", (RMS, FUSED), "float16", 2048, 4096, normal(0, 1), uniform(0.5, 1.5), 1e-5, 3001, 3003,
                   residual=normal(0, 0.5), seed_r=3002, outlier_frac=0.01, outlier_scale=100.0,
                   seed_outlier=3004),
    # the headline shape in bf16 (same distributions as C3)
    "C3b": Workload("C3b", (RMS, FUSED), "bfloat16", 2048, 4096, normal(0, 1), uniform(0.5, 1.5), 1e-5, 3101,
                    3103, residual=normal(0, 0.5), seed_r=3102, outlier_frac=0.01, outlier_scale=100.0,
                    seed_outlier=3104),
    # decode-shaped, launch-bound
    "C4a": Workload("C4a", (FUSED,), "bfloat16", 4, 1536, normal(0, 1), normal(1, 0.1), 1e-6, 4001, 4003,
                    residual=normal(0, 1), seed_r=4002),
    "C4b": Workload("C4b", (FUSED,), "bfloat16", 1, 8192, normal(0, 1), normal(1, 0.1), 1e-6, 4101, 4103,
                    residual=normal(0, 1), seed_r=4102),
    # large prefill (wide rows); the residual distribution is not stated, taken as that of x
    "C5f": Workload("C5f", (FUSED,), "bfloat16", 32768, 8192, normal(0, 2), normal(1, 0.1), 1e-6, 5001, 5003,
                    residual=normal(0, 2), seed_r=5002),
    "C5r": Workload("C5r", (RMS,), "bfloat16", 8192, 16384, normal(0, 2), normal(1, 0.1), 1e-6, 5101, 5103),
    # SwiGLU: `hidden` is the input width 2D (gate half, then up half)
    "S1": Workload("S1", (SWIGLU,), "bfloat16", 512, 2 * 4096, normal(0, 1), None, 0.0, 6001, None),
    "S2": Workload("S2", (SWIGLU,), "bfloat16", 2048, 2 * 11008, normal(0, 1), None, 0.0, 6101, None),
    "S3": Workload("S3", (SWIGLU,), "float16", 2048, 2 * 4096, normal(0, 1), None, 0.0, 6201, None),
    # out-of-place RMSNorm(x + residual) * w: the Triton Kernels README example
    # (fp16 [2048, 4096], randn x and residual, unit weight) and the headline
    # shape with the C3b distributions
    "R1": Workload("R1", (RESIDUAL,), "float16", 2048, 4096, normal(0, 1), normal(1, 0), 1e-6, 8001, 8003,
                   residual=normal(0, 1), seed_r=8002),
    "R2": Workload("R2", (RESIDUAL,), "bfloat16", 2048, 4096, normal(0, 1), uniform(0.5, 1.5), 1e-5, 8101, 8103,
                   residual=normal(0, 0.5), seed_r=8102, outlier_frac=0.01, outlier_scale=100.0,
                   seed_outlier=8104),
    # RMSNorm backward at the headline shape; the incoming gradient dy is drawn
    # through the residual fields
    "B1": Workload("B1", (BACKWARD,), "bfloat16", 2048, 4096, normal(0, 1), uniform(0.5, 1.5), 1e-5, 9001, 9003,
                   residual=normal(0, 1), seed_r=9002),
    # softmax over the last dimension
    "X1": Workload("X1", (SOFTMAX,), "bfloat16", 512, 1024, normal(0, 1), None, 0.0, 7001, None),
    "X2": Workload("X2", (SOFTMAX,), "bfloat16", 512, 128, normal(0, 1), None, 0.0, 7101, None),
    "X3": Workload("X3", (SOFTMAX,), "bfloat16", 512, 8192, normal(0, 1), None, 0.0, 7201, None),
    "X4": Workload("X4", (SOFTMAX,), "float16", 8, 65536, normal(0, 1), None, 0.0, 7301, None),
    "X5": Workload("X5", (SOFTMAX,), "bfloat16", 2048, 4096, normal(0, 1), None, 0.0, 7401, None),
}


DTYPE_TAGS = {"bf16": "bfloat16", "fp16": "float16", "fp32": "float32"}


def with_dtype(wl: Workload, dtype: str) -> Workload:
    """The same workload (shape, distributions, seeds) stored in another dtype;
    named e.g. ``C1-fp32``.  ``dtype`` is a torch name or a tag (bf16, fp16, fp32)."""
    dtype = DTYPE_TAGS.get(dtype, dtype)
    if dtype not in DTYPES:
        raise ValueError(f"unknown dtype {dtype}")
    if dtype == wl.dtype:
        return wl
    tag = {v: k for k, v in DTYPE_TAGS.items()}[dtype]
    return replace(wl, name=f"{wl.name}-{tag}", dtype=dtype)


def with_ops(wl: Workload, ops: tuple[str, ...]) -> Workload:
    """The same workload restricted to some of its ops (same inputs and seeds);
    named e.g. ``C3b/rms_norm``."""
    if not set(ops) <= set(wl.ops) or not ops:
        raise ValueError(f"{wl.name} has ops {wl.ops}, not {ops}")
    if tuple(ops) == wl.ops:
        return wl
    return replace(wl, name=f"{wl.name}/{'+'.join(ops)}", ops=tuple(ops))


def _to_dtype(values: np.ndarray, dtype: torch.dtype, shape: tuple[int, ...]) -> torch.Tensor:
    return torch.from_numpy(values).reshape(shape).to(dtype)


def make_inputs(wl: Workload, rows: int | None = None) -> dict[str, torch.Tensor]:
    """CPU tensors ``x``, ``weight`` and (if the workload has one) ``residual`` in the workload's dtype.

    ``rows`` may truncate the batch (the first rows of the full draw are NOT
    reproduced then: a shorter draw is a different sample); default is the
    workload's own row count.
    """
    rows = wl.rows if rows is None else rows
    n = rows * wl.hidden
    x = wl.x.draw(np.random.default_rng(wl.seed_x), n)
    if wl.outlier_frac:
        k = int(round(wl.outlier_frac * n))
        idx = np.random.default_rng(wl.seed_outlier).choice(n, size=k, replace=False)
        x[idx] *= np.float32(wl.outlier_scale)
    out = {"x": _to_dtype(x, wl.torch_dtype, (rows, wl.hidden))}
    if wl.weight is not None:
        out["weight"] = _to_dtype(wl.weight.draw(np.random.default_rng(wl.seed_w), wl.hidden), wl.torch_dtype,
                                  (wl.hidden,))
    if wl.residual is not None:
        r = wl.residual.draw(np.random.default_rng(wl.seed_r), n)
        out["residual"] = _to_dtype(r, wl.torch_dtype, (rows, wl.hidden))
    return out


def random_case(shape: tuple[int, ...], dtype: str, seed: int, x: Dist = normal(0, 1),
                residual: Dist = normal(0, 1), weight: Dist = normal(1, 0.1)) -> dict[str, torch.Tensor]:
    """Inputs of any shape (..., H) for edge-case tests."""
    n = int(np.prod(shape)) if len(shape) else 1
    hidden = shape[-1]
    tdt = DTYPES[dtype]
    rng = np.random.default_rng(seed)
    return {
        "x": _to_dtype(x.draw(rng, n), tdt, shape),
        "residual": _to_dtype(residual.draw(rng, n), tdt, shape),
        "weight": _to_dtype(weight.draw(rng, hidden), tdt, (hidden,)),
    }
