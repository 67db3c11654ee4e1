"""ctypes binding of libks_norm.so: argument marshalling only.

The ``ks_*`` functions mirror the C ABI in ``include/ks_norm.h`` one to one
(raw device pointers as ints).  ``rms_norm``, ``fused_add_rms_norm``,
``rms_norm_residual``, ``rms_norm_backward``, ``silu_and_mul`` and ``softmax``
are the tensor-level calls with the kernscope API shape
(README, "API contract" and "Inputs"): they check devices, dtypes, shapes, contiguity and
``requires_grad`` (the accelerator kernels are inference-only), then pass the
tensors' device pointers and torch's current HIP stream to the library.
Every step of the computation runs in the library's kernels; there is no
fallback.
"""
from __future__ import annotations

import ctypes
import os
import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
DEFAULT_LIB = os.path.join(_PKG, "libks_norm.so")

(KS_SUCCESS, KS_ERROR_INVALID_VALUE, KS_ERROR_UNSUPPORTED_DTYPE, KS_ERROR_OVERLAP, KS_ERROR_HIP,
 KS_ERROR_SCRATCH_LIMIT) = range(6)
KS_NOALLOC_SCRATCH_BYTES = 1 << 20
KS_DTYPE = {torch.float32: 0, torch.float16: 1, torch.bfloat16: 2}
(KS_OP_RMS_NORM, KS_OP_FUSED_ADD_RMS_NORM, KS_OP_SILU_AND_MUL, KS_OP_SOFTMAX, KS_OP_RMS_NORM_RESIDUAL,
 KS_OP_RMS_NORM_BACKWARD) = range(6)
KS_PATH_VECTOR, KS_PATH_GENERIC, KS_PATH_SPLIT = 0, 1, 2


class KsError(RuntimeError):
    """A non-success ks_status_t."""

    def __init__(self, status: int, message: str, hip_error: int = 0):
        super().__init__(message)
        self.status = status
        self.hip_error = hip_error


class KsValueError(KsError, ValueError):
    pass


class KsTypeError(KsError, TypeError):
    pass


class Plan(ctypes.Structure):
    """ks_plan_t."""

    _fields_ = [
        ("path", ctypes.c_int32),
        ("threads_per_row", ctypes.c_int32),
        ("vectors_per_thread", ctypes.c_int32),
        ("elems_per_access", ctypes.c_int32),
        ("rows_per_block", ctypes.c_int32),
        ("block_threads", ctypes.c_int32),
        ("load_nt", ctypes.c_int32),
        ("store_nt", ctypes.c_int32),
        ("weight_lds", ctypes.c_int32),
    ]

    def as_dict(self) -> dict:
        return {name: int(getattr(self, name)) for name, _ in self._fields_}

    @classmethod
    def from_dict(cls, d: dict) -> "Plan":
        return cls(**{k: int(d.get(k, 0)) for k, _ in cls._fields_})


_lib: ctypes.CDLL | None = None


def library_path() -> str:
    return os.environ.get("KS_NORM_LIB", DEFAULT_LIB)


def lib() -> ctypes.CDLL:
    """The loaded library.  Raises if it has not been built: there is no fallback."""
    global _lib
    if _lib is None:
        path = library_path()
        if not os.path.exists(path):
            raise RuntimeError(f"{path} is not built; run `python -m rmsnorm_row_normalisation_amd.build` "
                               "(or __graft_entry__.build()) first")
        h = ctypes.CDLL(path)
        i64, vp, f32, i32 = ctypes.c_int64, ctypes.c_void_p, ctypes.c_float, ctypes.c_int
        h.ks_rms_norm.argtypes = [vp, vp, vp, i64, i64, f32, i32, vp]
        h.ks_fused_add_rms_norm.argtypes = [vp, vp, vp, i64, i64, f32, i32, vp]
        h.ks_rms_norm_ex.argtypes = [vp, vp, vp, i64, i64, f32, i32, ctypes.POINTER(Plan), vp]
        h.ks_fused_add_rms_norm_ex.argtypes = [vp, vp, vp, i64, i64, f32, i32, ctypes.POINTER(Plan), vp]
        h.ks_get_plan.argtypes = [i32, i32, i64, i64, i32, ctypes.POINTER(Plan)]
        h.ks_get_plan_cus.argtypes = [i32, i32, i64, i64, i32, i32, ctypes.POINTER(Plan)]
        h.ks_time_next_call.argtypes = [vp, vp]
        h.ks_silu_and_mul.argtypes = [vp, vp, i64, i64, i32, vp]
        h.ks_silu_and_mul_ex.argtypes = [vp, vp, i64, i64, i32, ctypes.POINTER(Plan), vp]
        h.ks_softmax.argtypes = [vp, vp, i64, i64, i32, vp]
        h.ks_rms_norm_residual.argtypes = [vp, vp, vp, vp, i64, i64, f32, i32, vp]
        sz = ctypes.c_size_t
        h.ks_rms_norm_backward_workspace_size.argtypes = [i64, i64, ctypes.POINTER(sz)]
        h.ks_rms_norm_backward.argtypes = [vp, vp, vp, vp, vp, i64, i64, f32, i32, vp, sz, vp]
        h.ks_rms_norm_backward_ex.argtypes = [vp, vp, vp, vp, vp, i64, i64, f32, i32, vp, sz, ctypes.POINTER(Plan),
                                              vp]
        h.ks_rms_norm_residual_ex.argtypes = [vp, vp, vp, vp, i64, i64, f32, i32, ctypes.POINTER(Plan), vp]
        h.ks_softmax_ex.argtypes = [vp, vp, i64, i64, i32, ctypes.POINTER(Plan), vp]
        h.ks_softmax_workspace_size.argtypes = [i64, i64, i32, ctypes.POINTER(Plan), ctypes.POINTER(sz)]
        h.ks_softmax_ws.argtypes = [vp, vp, i64, i64, i32, vp, sz, vp]
        h.ks_softmax_ws_ex.argtypes = [vp, vp, i64, i64, i32, vp, sz, ctypes.POINTER(Plan), vp]
        h.ks_softmax_noalloc.argtypes = [vp, vp, i64, i64, i32, vp]
        h.ks_status_string.argtypes = [i32]
        h.ks_status_string.restype = ctypes.c_char_p
        h.ks_last_hip_error.argtypes = []
        h.ks_version.argtypes = []
        h.ks_version.restype = ctypes.c_char_p
        for name in ("ks_rms_norm", "ks_fused_add_rms_norm", "ks_rms_norm_ex", "ks_fused_add_rms_norm_ex",
                     "ks_get_plan", "ks_last_hip_error", "ks_silu_and_mul", "ks_silu_and_mul_ex", "ks_softmax",
                     "ks_softmax_ex", "ks_rms_norm_residual", "ks_rms_norm_residual_ex",
                     "ks_rms_norm_backward_workspace_size", "ks_rms_norm_backward", "ks_rms_norm_backward_ex",
                     "ks_softmax_workspace_size", "ks_softmax_ws", "ks_softmax_ws_ex", "ks_softmax_noalloc",
                     "ks_get_plan_cus", "ks_time_next_call"):
            getattr(h, name).restype = ctypes.c_int
        _lib = h
    return _lib


def _check(status: int, what: str) -> None:
    if status == KS_SUCCESS:
        return
    msg = f"{what}: {lib().ks_status_string(status).decode()}"
    if status == KS_ERROR_UNSUPPORTED_DTYPE:
        raise KsTypeError(status, msg)
    if status in (KS_ERROR_INVALID_VALUE, KS_ERROR_OVERLAP, KS_ERROR_SCRATCH_LIMIT):
        raise KsValueError(status, msg)
    hip = int(lib().ks_last_hip_error())
    raise KsError(status, f"{msg} (hipError {hip})", hip)


# ---------------------------------------------------------------------------
# Raw C-ABI mirrors (device pointers as ints; return the status code).
# ---------------------------------------------------------------------------
def ks_rms_norm(out: int, x: int, weight: int, rows: int, hidden: int, eps: float, dtype: int,
                stream: int) -> int:
    return lib().ks_rms_norm(out, x, weight, rows, hidden, eps, dtype, stream)


def ks_fused_add_rms_norm(x: int, residual: int, weight: int, rows: int, hidden: int, eps: float, dtype: int,
                          stream: int) -> int:
    return lib().ks_fused_add_rms_norm(x, residual, weight, rows, hidden, eps, dtype, stream)


def ks_rms_norm_ex(out: int, x: int, weight: int, rows: int, hidden: int, eps: float, dtype: int,
                   plan: Plan | None, stream: int) -> int:
    return lib().ks_rms_norm_ex(out, x, weight, rows, hidden, eps, dtype,
                                ctypes.byref(plan) if plan is not None else None, stream)


def ks_fused_add_rms_norm_ex(x: int, residual: int, weight: int, rows: int, hidden: int, eps: float, dtype: int,
                             plan: Plan | None, stream: int) -> int:
    return lib().ks_fused_add_rms_norm_ex(x, residual, weight, rows, hidden, eps, dtype,
                                          ctypes.byref(plan) if plan is not None else None, stream)


def ks_rms_norm_residual(out: int, x: int, residual: int, weight: int, rows: int, hidden: int, eps: float,
                         dtype: int, stream: int) -> int:
    return lib().ks_rms_norm_residual(out, x, residual, weight, rows, hidden, eps, dtype, stream)


def ks_rms_norm_residual_ex(out: int, x: int, residual: int, weight: int, rows: int, hidden: int, eps: float,
                            dtype: int, plan: Plan | None, stream: int) -> int:
    return lib().ks_rms_norm_residual_ex(out, x, residual, weight, rows, hidden, eps, dtype,
                                         ctypes.byref(plan) if plan is not None else None, stream)


def ks_rms_norm_backward_workspace_size(rows: int, hidden: int) -> int:
    n = ctypes.c_size_t()
    _check(lib().ks_rms_norm_backward_workspace_size(rows, hidden, ctypes.byref(n)),
           "ks_rms_norm_backward_workspace_size")
    return n.value


def ks_rms_norm_backward(dx: int, dw: int, dy: int, x: int, weight: int, rows: int, hidden: int, eps: float,
                         dtype: int, workspace: int, workspace_bytes: int, stream: int) -> int:
    return lib().ks_rms_norm_backward(dx, dw, dy, x, weight, rows, hidden, eps, dtype, workspace, workspace_bytes,
                                      stream)


def ks_rms_norm_backward_ex(dx: int, dw: int, dy: int, x: int, weight: int, rows: int, hidden: int, eps: float,
                            dtype: int, workspace: int, workspace_bytes: int, plan: Plan | None, stream: int) -> int:
    return lib().ks_rms_norm_backward_ex(dx, dw, dy, x, weight, rows, hidden, eps, dtype, workspace,
                                         workspace_bytes, ctypes.byref(plan) if plan is not None else None, stream)


def ks_silu_and_mul(out: int, x: int, rows: int, d: int, dtype: int, stream: int) -> int:
    return lib().ks_silu_and_mul(out, x, rows, d, dtype, stream)


def ks_silu_and_mul_ex(out: int, x: int, rows: int, d: int, dtype: int, plan: Plan | None, stream: int) -> int:
    return lib().ks_silu_and_mul_ex(out, x, rows, d, dtype, ctypes.byref(plan) if plan is not None else None, stream)


def ks_softmax(out: int, x: int, rows: int, hidden: int, dtype: int, stream: int) -> int:
    return lib().ks_softmax(out, x, rows, hidden, dtype, stream)


def ks_softmax_ex(out: int, x: int, rows: int, hidden: int, dtype: int, plan: Plan | None, stream: int) -> int:
    return lib().ks_softmax_ex(out, x, rows, hidden, dtype, ctypes.byref(plan) if plan is not None else None, stream)


def ks_softmax_workspace_size(rows: int, hidden: int, dtype: int, plan: Plan | None = None) -> int:
    n = ctypes.c_size_t(0)
    _check(lib().ks_softmax_workspace_size(rows, hidden, dtype, ctypes.byref(plan) if plan is not None else None,
                                           ctypes.byref(n)), "ks_softmax_workspace_size")
    return n.value


def ks_softmax_ws(out: int, x: int, rows: int, hidden: int, dtype: int, workspace: int, workspace_bytes: int,
                  stream: int) -> int:
    return lib().ks_softmax_ws(out, x, rows, hidden, dtype, workspace, workspace_bytes, stream)


def ks_softmax_ws_ex(out: int, x: int, rows: int, hidden: int, dtype: int, workspace: int, workspace_bytes: int,
                     plan: Plan | None, stream: int) -> int:
    return lib().ks_softmax_ws_ex(out, x, rows, hidden, dtype, workspace, workspace_bytes,
                                  ctypes.byref(plan) if plan is not None else None, stream)


def ks_softmax_noalloc(out: int, x: int, rows: int, hidden: int, dtype: int, stream: int) -> int:
    return lib().ks_softmax_noalloc(out, x, rows, hidden, dtype, stream)


KS_PLAN_ALIGNED = 1
KS_PLAN_WORKSPACE = 2


def ks_get_plan(op: int, dtype: int, rows: int, hidden: int, aligned: bool = True, workspace: bool = False,
                compute_units: int | None = None) -> Plan:
    """ks_get_plan (the current device's compute units), or ks_get_plan_cus when
    compute_units is given."""
    plan = Plan()
    flags = (KS_PLAN_ALIGNED if aligned else 0) | (KS_PLAN_WORKSPACE if workspace else 0)
    if compute_units is None:
        _check(lib().ks_get_plan(op, dtype, rows, hidden, flags, ctypes.byref(plan)), "ks_get_plan")
    else:
        _check(lib().ks_get_plan_cus(op, dtype, rows, hidden, flags, compute_units, ctypes.byref(plan)),
               "ks_get_plan_cus")
    return plan


def ks_time_next_call(start: int | None, stop: int | None) -> int:
    """Attach two hipEvent_t handles (ints, or None) to the calling thread's next call."""
    return lib().ks_time_next_call(start, stop)


def ks_version() -> str:
    return lib().ks_version().decode()


# ---------------------------------------------------------------------------
# Tensor-level API.
# ---------------------------------------------------------------------------
def _check_tensors(op: str, x: torch.Tensor, weight: torch.Tensor, *others: torch.Tensor) -> tuple[int, int]:
    if x.dtype not in KS_DTYPE:
        raise TypeError(f"{op}: unsupported dtype {x.dtype}")
    for t in (weight, *others):
        if t.dtype != x.dtype:
            raise TypeError(f"{op}: all tensors must share dtype {x.dtype}, got {t.dtype}")
        if t.device != x.device:
            raise ValueError(f"{op}: all tensors must be on {x.device}, got {t.device}")
    if x.device.type != "cuda":
        raise ValueError(f"{op}: tensors must be on a HIP device, got {x.device}")
    for t in (x, weight, *others):
        if not t.is_contiguous():
            raise ValueError(f"{op}: tensors must be contiguous")
        if t.requires_grad:
            raise ValueError(f"{op}: inference-only kernel; got a tensor that requires grad")
    if x.dim() == 0 or x.shape[-1] == 0:
        raise ValueError(f"{op}: the last dimension must be nonempty")
    hidden = x.shape[-1]
    if weight.shape != (hidden,):
        raise ValueError(f"{op}: weight must have shape ({hidden},), got {tuple(weight.shape)}")
    return x.numel() // hidden, hidden


def _stream(x: torch.Tensor) -> int:
    return int(torch.cuda.current_stream(x.device).cuda_stream)


def rms_norm(x: torch.Tensor, weight: torch.Tensor, eps: float = 1e-6, *, out: torch.Tensor | None = None,
             plan: Plan | None = None) -> torch.Tensor:
    """RMSNorm over the last dimension; returns ``out`` (a new tensor unless given; may be ``x``)."""
    rows, hidden = _check_tensors("rms_norm", x, weight)
    if out is None:
        out = torch.empty_like(x)
    else:
        _check_tensors("rms_norm", out, weight)
        if out.shape != x.shape:
            raise ValueError("rms_norm: out must have the shape of x")
    with torch.cuda.device(x.device):
        st = ks_rms_norm_ex(out.data_ptr(), x.data_ptr(), weight.data_ptr(), rows, hidden, float(eps),
                            KS_DTYPE[x.dtype], plan, _stream(x))
    _check(st, "ks_rms_norm")
    return out


def fused_add_rms_norm(x: torch.Tensor, residual: torch.Tensor, weight: torch.Tensor, eps: float = 1e-6, *,
                       plan: Plan | None = None) -> None:
    """In place: residual <- cast(x + residual); x <- RMSNorm of the fp32 sum.  Returns None."""
    rows, hidden = _check_tensors("fused_add_rms_norm", x, weight, residual)
    if residual.shape != x.shape:
        raise ValueError("fused_add_rms_norm: residual must have the shape of x")
    with torch.cuda.device(x.device):
        st = ks_fused_add_rms_norm_ex(x.data_ptr(), residual.data_ptr(), weight.data_ptr(), rows, hidden,
                                      float(eps), KS_DTYPE[x.dtype], plan, _stream(x))
    _check(st, "ks_fused_add_rms_norm")


def rms_norm_residual(x: torch.Tensor, residual: torch.Tensor, weight: torch.Tensor, eps: float = 1e-6, *,
                      out: torch.Tensor | None = None, plan: Plan | None = None) -> torch.Tensor:
    """Out of place: RMSNorm(x + residual) * weight with the fp32 sum (Triton Kernels
    README, "Kernels"); returns ``out`` (a new tensor unless given; may be x or residual)."""
    rows, hidden = _check_tensors("rms_norm_residual", x, weight, residual)
    if residual.shape != x.shape:
        raise ValueError("rms_norm_residual: residual must have the shape of x")
    if out is None:
        out = torch.empty_like(x)
    else:
        _check_tensors("rms_norm_residual", out, weight)
        if out.shape != x.shape:
            raise ValueError("rms_norm_residual: out must have the shape of x")
    with torch.cuda.device(x.device):
        st = ks_rms_norm_residual_ex(out.data_ptr(), x.data_ptr(), residual.data_ptr(), weight.data_ptr(), rows,
                                     hidden, float(eps), KS_DTYPE[x.dtype], plan, _stream(x))
    _check(st, "ks_rms_norm_residual")
    return out


def rms_norm_backward(dy: torch.Tensor, x: torch.Tensor, weight: torch.Tensor, eps: float = 1e-6, *,
                      weight_grad: bool = True, plan: Plan | None = None, workspace: torch.Tensor | None = None,
                      dx: torch.Tensor | None = None,
                      dweight: torch.Tensor | None = None) -> tuple[torch.Tensor, torch.Tensor | None]:
    """Gradients (dx, dweight) of rms_norm(x, weight, eps) for the incoming gradient dy.
    dweight is None when ``weight_grad`` is False.  The fp32 workspace the weight
    gradient needs is allocated through torch unless given (a uint8 device tensor
    of at least ks_rms_norm_backward_workspace_size bytes)."""
    rows, hidden = _check_tensors("rms_norm_backward", x, weight, dy)
    if dy.shape != x.shape:
        raise ValueError("rms_norm_backward: dy must have the shape of x")
    if dx is None:
        dx = torch.empty_like(x)
    else:
        _check_tensors("rms_norm_backward", dx, weight)
        if dx.shape != x.shape:
            raise ValueError("rms_norm_backward: dx must have the shape of x")
    if not weight_grad:
        dw = None
    elif dweight is None:
        dw = torch.empty_like(weight)
    else:
        _check_tensors("rms_norm_backward", x, dweight)
        dw = dweight
    need = ks_rms_norm_backward_workspace_size(rows, hidden) if weight_grad else 0
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=x.device)
    elif workspace.device != x.device or not workspace.is_contiguous() or workspace.numel() * workspace.element_size() < need:
        raise ValueError(f"rms_norm_backward: workspace must be a contiguous tensor of >= {need} bytes on {x.device}")
    with torch.cuda.device(x.device):
        st = ks_rms_norm_backward_ex(dx.data_ptr(), dw.data_ptr() if dw is not None else None, dy.data_ptr(),
                                     x.data_ptr(), weight.data_ptr(), rows, hidden, float(eps), KS_DTYPE[x.dtype],
                                     workspace.data_ptr(), workspace.numel() * workspace.element_size(), plan,
                                     _stream(x))
    _check(st, "ks_rms_norm_backward")
    return dx, dw


class _RMSNormFunction(torch.autograd.Function):
    """rms_norm with its gradients from ks_rms_norm_backward (the kernscope
    reference of rms_norm supports autograd; the kernels themselves see only
    detached tensors)."""

    @staticmethod
    def forward(ctx, x: torch.Tensor, weight: torch.Tensor, eps: float) -> torch.Tensor:
        xd, wd = x.detach(), weight.detach()
        ctx.save_for_backward(xd, wd)
        ctx.eps = eps
        return rms_norm(xd, wd, eps)

    @staticmethod
    def backward(ctx, dy: torch.Tensor):
        x, w = ctx.saved_tensors
        dx, dw = rms_norm_backward(dy.detach().contiguous(), x, w, ctx.eps, weight_grad=ctx.needs_input_grad[1])
        return (dx if ctx.needs_input_grad[0] else None), dw, None


def rms_norm_autograd(x: torch.Tensor, weight: torch.Tensor, eps: float = 1e-6) -> torch.Tensor:
    """rms_norm that records the autograd graph: the forward is ks_rms_norm, the
    backward ks_rms_norm_backward (first derivatives only)."""
    return _RMSNormFunction.apply(x, weight, eps)


def silu_and_mul(x: torch.Tensor, *, out: torch.Tensor | None = None, plan: Plan | None = None) -> torch.Tensor:
    """SwiGLU of x with shape (..., 2D): a new (..., D) tensor (kernscope "SwiGLU activation")."""
    if x.dtype not in KS_DTYPE:
        raise TypeError(f"silu_and_mul: unsupported dtype {x.dtype}")
    if x.device.type != "cuda":
        raise ValueError(f"silu_and_mul: tensors must be on a HIP device, got {x.device}")
    if not x.is_contiguous():
        raise ValueError("silu_and_mul: x must be contiguous")
    if x.requires_grad:
        raise ValueError("silu_and_mul: inference-only kernel; got a tensor that requires grad")
    if x.dim() == 0 or x.shape[-1] == 0 or x.shape[-1] % 2:
        raise ValueError("silu_and_mul: the last dimension must be nonempty and even")
    d = x.shape[-1] // 2
    rows = x.numel() // x.shape[-1]
    shape = (*x.shape[:-1], d)
    if out is None:
        out = torch.empty(shape, dtype=x.dtype, device=x.device)
    elif out.shape != shape or out.dtype != x.dtype or out.device != x.device or not out.is_contiguous():
        raise ValueError(f"silu_and_mul: out must be a contiguous {x.dtype} tensor of shape {shape}")
    with torch.cuda.device(x.device):
        st = ks_silu_and_mul_ex(out.data_ptr(), x.data_ptr(), rows, d, KS_DTYPE[x.dtype], plan, _stream(x))
    _check(st, "ks_silu_and_mul")
    return out


def softmax(x: torch.Tensor, *, out: torch.Tensor | None = None, plan: Plan | None = None, split: bool = True,
            workspace: torch.Tensor | None = None) -> torch.Tensor:
    """Softmax over the last dimension (kernscope "Softmax"): returns ``out`` (a new
    tensor unless given; may be ``x``).

    With ``split`` (the default) the call passes a workspace (ks_softmax_ws_ex),
    so wide rows in small batches may be split over many workgroups; the
    workspace is ``workspace`` (a contiguous tensor on x's device of at least
    ks_softmax_workspace_size bytes) or, when that is None and the plan needs
    one, a new tensor.  ``split=False`` (ks_softmax_ex) keeps to the one-pass
    plans, whose bits for a row never depend on the batch it is in."""
    if x.dtype not in KS_DTYPE:
        raise TypeError(f"softmax: unsupported dtype {x.dtype}")
    if x.device.type != "cuda":
        raise ValueError(f"softmax: tensors must be on a HIP device, got {x.device}")
    if not x.is_contiguous():
        raise ValueError("softmax: x must be contiguous")
    if x.requires_grad:
        raise ValueError("softmax: inference-only kernel; got a tensor that requires grad")
    if x.dim() == 0 or x.shape[-1] == 0:
        raise ValueError("softmax: the last dimension must be nonempty")
    hidden = x.shape[-1]
    rows = x.numel() // hidden
    if out is None:
        out = torch.empty_like(x)
    elif out.shape != x.shape or out.dtype != x.dtype or out.device != x.device or not out.is_contiguous():
        raise ValueError(f"softmax: out must be a contiguous {x.dtype} tensor of shape {tuple(x.shape)}")
    dt = KS_DTYPE[x.dtype]
    with torch.cuda.device(x.device):
        if not split:
            st = ks_softmax_ex(out.data_ptr(), x.data_ptr(), rows, hidden, dt, plan, _stream(x))
        else:
            need = ks_softmax_workspace_size(rows, hidden, dt, plan)
            if workspace is None:
                workspace = torch.empty(need, dtype=torch.uint8, device=x.device) if need else None
            elif (workspace.device != x.device or not workspace.is_contiguous()
                  or workspace.numel() * workspace.element_size() < need):
                raise ValueError(f"softmax: workspace must be a contiguous tensor of >= {need} bytes on {x.device}")
            wp = workspace.data_ptr() if workspace is not None else 0
            wb = workspace.numel() * workspace.element_size() if workspace is not None else 0
            st = ks_softmax_ws_ex(out.data_ptr(), x.data_ptr(), rows, hidden, dt, wp, wb, plan, _stream(x))
    _check(st, "ks_softmax")
    return out


def get_plan(op: str, dtype: torch.dtype, hidden: int, rows: int = 1, aligned: bool = True,
             workspace: bool = False, compute_units: int | None = None) -> Plan:
    """The plan the library picks for this op, dtype, row size and batch (ks_get_plan:
    on the current device, or on a device of ``compute_units`` compute units).
    For silu_and_mul, ``hidden`` is the output width D; ``workspace`` asks for the
    plan of a call that passes one (softmax: ``softmax(split=True)``)."""
    code = {"rms_norm": KS_OP_RMS_NORM, "fused_add_rms_norm": KS_OP_FUSED_ADD_RMS_NORM,
            "silu_and_mul": KS_OP_SILU_AND_MUL, "softmax": KS_OP_SOFTMAX,
            "rms_norm_residual": KS_OP_RMS_NORM_RESIDUAL, "rms_norm_backward": KS_OP_RMS_NORM_BACKWARD}[op]
    return ks_get_plan(code, KS_DTYPE[dtype], rows, hidden, aligned, workspace, compute_units)
