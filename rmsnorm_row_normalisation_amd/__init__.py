"""RMSNorm (forward and backward), fused residual-add RMSNorm (in place and out
of place), SwiGLU and softmax for MI355X (gfx950).

The computation lives in ``libks_norm.so`` (hand-written HIP kernels behind a
C ABI, ``include/ks_norm.h``); this package is its thin Python binding.
"""
from .binding import (  # noqa: F401
    KS_DTYPE,
    KsError,
    KsTypeError,
    KsValueError,
    Plan,
    fused_add_rms_norm,
    get_plan,
    ks_fused_add_rms_norm,
    ks_fused_add_rms_norm_ex,
    ks_get_plan,
    ks_time_next_call,
    ks_rms_norm,
    ks_rms_norm_ex,
    ks_silu_and_mul,
    ks_silu_and_mul_ex,
    ks_version,
    lib,
    library_path,
    rms_norm,
    silu_and_mul,
    softmax,
    ks_softmax,
    ks_softmax_ex,
    ks_softmax_workspace_size,
    ks_softmax_ws,
    ks_softmax_ws_ex,
    ks_softmax_noalloc,
    KS_NOALLOC_SCRATCH_BYTES,
    KS_PLAN_ALIGNED,
    KS_PLAN_WORKSPACE,
    rms_norm_residual,
    ks_rms_norm_residual,
    ks_rms_norm_residual_ex,
    rms_norm_backward,
    rms_norm_autograd,
    ks_rms_norm_backward,
    ks_rms_norm_backward_ex,
    ks_rms_norm_backward_workspace_size,
)

__version__ = "0.1.0"
