"""CPU oracle for RMSNorm (forward and backward), fused residual-add RMSNorm
(in place and out of place), SwiGLU and softmax.

TEST INFRASTRUCTURE ONLY.  The tests, ``__graft_entry__.smoke()`` and the
benchmark's ``cpu_baseline`` leg may import this package; the GPU product path
never does, and the two share no code.

``ks_oracle.c`` holds all arithmetic (kernscope README, "Numerical contract":
"RMSNorm", "Fused residual-add RMSNorm", "SwiGLU activation" and "Softmax";
Triton Kernels README, "Kernels": the out-of-place residual-fused RMSNorm).  This module
only builds and loads that library and marshals torch CPU tensors (used as
plain byte containers) to it.  ``brute64`` is a second, independent fp64 / exact-rational
check for tiny inputs.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "ks_oracle.c")
_LIB = os.path.join(_HERE, "libks_oracle.so")

# Flags that keep every C float operation a single IEEE operation.
CFLAGS = ["-O2", "-std=c11", "-ffp-contract=off", "-fno-fast-math", "-fPIC", "-shared"]

_DTYPE_CODE = {torch.float32: 0, torch.float16: 1, torch.bfloat16: 2}


def build(src: str = _SRC, out: str = _LIB, defines: tuple[str, ...] = ()) -> str:
    """Compile the oracle with gcc into ``out`` and return its path."""
    cmd = ["gcc", *CFLAGS, *[f"-D{d}" for d in defines], src, "-o", out + ".tmp", "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(out + ".tmp", out)
    return out


def _configure(lib: ctypes.CDLL) -> ctypes.CDLL:
    i64, vp, c_int, c_float = ctypes.c_int64, ctypes.c_void_p, ctypes.c_int, ctypes.c_float
    lib.oracle_rms_norm.argtypes = [c_int, vp, vp, vp, i64, i64, c_float]
    lib.oracle_rms_norm.restype = c_int
    lib.oracle_fused_add_rms_norm.argtypes = [c_int, vp, vp, vp, i64, i64, c_float]
    lib.oracle_fused_add_rms_norm.restype = c_int
    lib.oracle_round_f32_array.argtypes = [c_int, vp, vp, i64]
    lib.oracle_round_f32_array.restype = c_int
    lib.oracle_widen_array.argtypes = [c_int, vp, vp, i64]
    lib.oracle_widen_array.restype = c_int
    lib.oracle_silu_and_mul.argtypes = [c_int, vp, vp, i64, i64]
    lib.oracle_silu_and_mul.restype = c_int
    lib.oracle_softmax.argtypes = [c_int, vp, vp, i64, i64]
    lib.oracle_rms_norm_residual.argtypes = [c_int, vp, vp, vp, vp, i64, i64, c_float]
    lib.oracle_rms_norm_residual.restype = c_int
    lib.oracle_rms_norm_backward.argtypes = [c_int, vp, vp, vp, vp, vp, i64, i64, c_float]
    lib.oracle_rms_norm_backward.restype = c_int
    lib.oracle_softmax.restype = c_int
    return lib


_lib: ctypes.CDLL | None = None


def load(path: str | None = None) -> ctypes.CDLL:
    """Load the oracle library (building it first if it is not there)."""
    global _lib
    if path is not None:
        return _configure(ctypes.CDLL(path))
    if _lib is None:
        if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
            build()
        _lib = _configure(ctypes.CDLL(_LIB))
    return _lib


def _check_rows(x: torch.Tensor, w: torch.Tensor) -> tuple[int, int]:
    if x.device.type != "cpu" or w.device.type != "cpu":
        raise ValueError("oracle works on CPU tensors")
    if x.dtype not in _DTYPE_CODE or w.dtype != x.dtype:
        raise TypeError(f"unsupported dtypes {x.dtype}, {w.dtype}")
    if not (x.is_contiguous() and w.is_contiguous()):
        raise ValueError("oracle needs contiguous tensors")
    hidden = x.shape[-1] if x.dim() > 0 else 0
    if hidden <= 0 or w.shape != (hidden,):
        raise ValueError("bad hidden size or weight shape")
    return x.numel() // hidden, hidden


def rms_norm(x: torch.Tensor, w: torch.Tensor, eps: float = 1e-6, lib: ctypes.CDLL | None = None) -> torch.Tensor:
    """Return a new tensor: the contract's RMSNorm of x (CPU, any shape (..., H))."""
    lib = lib or load()
    rows, hidden = _check_rows(x, w)
    out = torch.empty_like(x)
    st = lib.oracle_rms_norm(_DTYPE_CODE[x.dtype], x.data_ptr(), w.data_ptr(), out.data_ptr(), rows, hidden, eps)
    if st != 0:
        raise ValueError(f"oracle_rms_norm failed with status {st}")
    return out


def fused_add_rms_norm(x: torch.Tensor, residual: torch.Tensor, w: torch.Tensor, eps: float = 1e-6,
                       lib: ctypes.CDLL | None = None) -> tuple[torch.Tensor, torch.Tensor]:
    """Return (x_out, residual_out) as new tensors; the inputs are left unchanged."""
    lib = lib or load()
    rows, hidden = _check_rows(x, w)
    if residual.shape != x.shape or residual.dtype != x.dtype or not residual.is_contiguous():
        raise ValueError("residual must match x")
    xo, ro = x.clone(), residual.clone()
    st = lib.oracle_fused_add_rms_norm(_DTYPE_CODE[x.dtype], xo.data_ptr(), ro.data_ptr(), w.data_ptr(),
                                       rows, hidden, eps)
    if st != 0:
        raise ValueError(f"oracle_fused_add_rms_norm failed with status {st}")
    return xo, ro


def rms_norm_residual(x: torch.Tensor, residual: torch.Tensor, w: torch.Tensor, eps: float = 1e-6,
                      lib: ctypes.CDLL | None = None) -> torch.Tensor:
    """Out of place: a new tensor RMSNorm(x + residual) * w; the inputs are unchanged."""
    lib = lib or load()
    rows, hidden = _check_rows(x, w)
    if residual.shape != x.shape or residual.dtype != x.dtype or not residual.is_contiguous():
        raise ValueError("residual must match x")
    out = torch.empty_like(x)
    st = lib.oracle_rms_norm_residual(_DTYPE_CODE[x.dtype], x.data_ptr(), residual.data_ptr(), w.data_ptr(),
                                      out.data_ptr(), rows, hidden, eps)
    if st != 0:
        raise ValueError(f"oracle_rms_norm_residual failed with status {st}")
    return out


def rms_norm_backward(dy: torch.Tensor, x: torch.Tensor, w: torch.Tensor, eps: float = 1e-6,
                      lib: ctypes.CDLL | None = None) -> tuple[torch.Tensor, torch.Tensor]:
    """Gradients (dx, dw) of rms_norm(x, w, eps) for the incoming gradient dy."""
    lib = lib or load()
    rows, hidden = _check_rows(x, w)
    if dy.shape != x.shape or dy.dtype != x.dtype or not dy.is_contiguous() or dy.device.type != "cpu":
        raise ValueError("dy must match x")
    dx = torch.empty_like(x)
    dw = torch.empty_like(w)
    st = lib.oracle_rms_norm_backward(_DTYPE_CODE[x.dtype], dy.data_ptr(), x.data_ptr(), w.data_ptr(),
                                      dx.data_ptr(), dw.data_ptr(), rows, hidden, eps)
    if st != 0:
        raise ValueError(f"oracle_rms_norm_backward failed with status {st}")
    return dx, dw


def silu_and_mul(x: torch.Tensor, lib: ctypes.CDLL | None = None) -> torch.Tensor:
    """SwiGLU of x with shape (..., 2D): returns a new (..., D) tensor."""
    lib = lib or load()
    if x.device.type != "cpu" or x.dtype not in _DTYPE_CODE or not x.is_contiguous():
        raise ValueError("oracle needs a contiguous CPU tensor of a supported dtype")
    if x.dim() == 0 or x.shape[-1] == 0 or x.shape[-1] % 2:
        raise ValueError("the last dimension must be nonempty and even")
    d = x.shape[-1] // 2
    rows = x.numel() // x.shape[-1]
    out = torch.empty(*x.shape[:-1], d, dtype=x.dtype)
    st = lib.oracle_silu_and_mul(_DTYPE_CODE[x.dtype], x.data_ptr(), out.data_ptr(), rows, d)
    if st != 0:
        raise ValueError(f"oracle_silu_and_mul failed with status {st}")
    return out


def softmax(x: torch.Tensor, lib: ctypes.CDLL | None = None) -> torch.Tensor:
    """Softmax of x with shape (..., H) over the last dimension: a new tensor."""
    lib = lib or load()
    if x.device.type != "cpu" or x.dtype not in _DTYPE_CODE or not x.is_contiguous():
        raise ValueError("oracle needs a contiguous CPU tensor of a supported dtype")
    if x.dim() == 0 or x.shape[-1] == 0:
        raise ValueError("the last dimension must be nonempty")
    hidden = x.shape[-1]
    out = torch.empty_like(x)
    st = lib.oracle_softmax(_DTYPE_CODE[x.dtype], x.data_ptr(), out.data_ptr(), x.numel() // hidden, hidden)
    if st != 0:
        raise ValueError(f"oracle_softmax failed with status {st}")
    return out


def round_f32(values: torch.Tensor, dtype: torch.dtype, lib: ctypes.CDLL | None = None) -> torch.Tensor:
    """Round fp32 values to a 16-bit dtype with the oracle's cast; returns int16 bit patterns."""
    lib = lib or load()
    v = values.contiguous().to(torch.float32)
    out = torch.empty(v.shape, dtype=torch.int16)
    st = lib.oracle_round_f32_array(_DTYPE_CODE[dtype], v.data_ptr(), out.data_ptr(), v.numel())
    if st != 0:
        raise ValueError("bad dtype")
    return out


def widen(bits: torch.Tensor, dtype: torch.dtype, lib: ctypes.CDLL | None = None) -> torch.Tensor:
    """Widen int16 bit patterns of a 16-bit dtype to fp32 with the oracle's decoder."""
    lib = lib or load()
    b = bits.contiguous().to(torch.int16)
    out = torch.empty(b.shape, dtype=torch.float32)
    st = lib.oracle_widen_array(_DTYPE_CODE[dtype], b.data_ptr(), out.data_ptr(), b.numel())
    if st != 0:
        raise ValueError("bad dtype")
    return out
