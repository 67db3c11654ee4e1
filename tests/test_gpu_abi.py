"""The C ABI itself on cuda:0, through ctypes with raw device pointers.

* ks_rms_norm and ks_fused_add_rms_norm (the plain entry points, no plan
  argument) on a stream other than the default one, at 2048 x 4096 bf16: the
  oracle's bar, and bit-identical to the same calls through the _ex entry
  points and the tensor API.
* ks_time_next_call: the kernel-dispatch events of one call, multi-kernel
  calls included; the request applies to one call only and changes no result.
* The launch policy reads the device's compute units: ks_get_plan on the
  device equals ks_get_plan_cus with the count the device reports.
"""
import ctypes

import pytest
import torch

import oracle
import rmsnorm_row_normalisation_amd as ks
import workloads
from compare import FP32_MAX_ULP, check_bitexact, check_normalised
from gpu_cases import require_gpu, say
from rmsnorm_row_normalisation_amd import binding as b

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _gpu():
    require_gpu()


def _hip():
    import bench

    return bench.Hip()


def test_plain_entry_points_on_a_side_stream():
    wl = workloads.WORKLOADS["C3b"]
    inp = workloads.make_inputs(wl)
    code = ks.KS_DTYPE[wl.torch_dtype]
    stream = torch.cuda.Stream()
    x, w = inp["x"].cuda(), inp["weight"].cuda()
    r = inp["residual"].cuda()
    out = torch.full_like(x, float("nan"))
    fx, fr = x.clone(), r.clone()
    torch.cuda.synchronize()
    say("plain ks_rms_norm / ks_fused_add_rms_norm", wl.name, "side stream")
    lib = ks.lib()
    st = lib.ks_rms_norm(out.data_ptr(), x.data_ptr(), w.data_ptr(), wl.rows, wl.hidden, ctypes.c_float(wl.eps),
                         code, stream.cuda_stream)
    assert st == b.KS_SUCCESS
    st = lib.ks_fused_add_rms_norm(fx.data_ptr(), fr.data_ptr(), w.data_ptr(), wl.rows, wl.hidden,
                                   ctypes.c_float(wl.eps), code, stream.cuda_stream)
    assert st == b.KS_SUCCESS
    stream.synchronize()
    ref = oracle.rms_norm(inp["x"], inp["weight"], wl.eps)
    check_normalised(out.cpu(), ref, 0.999, fp32_max_ulp=FP32_MAX_ULP)
    rx, rr = oracle.fused_add_rms_norm(inp["x"], inp["residual"], inp["weight"], wl.eps)
    check_bitexact(fr.cpu(), rr)
    check_normalised(fx.cpu(), rx, 0.999)
    # the _ex entry points with the policy's plan, and the tensor API, give the same bits
    out2 = torch.empty_like(x)
    assert b.ks_rms_norm_ex(out2.data_ptr(), x.data_ptr(), w.data_ptr(), wl.rows, wl.hidden, wl.eps, code, None,
                            stream.cuda_stream) == b.KS_SUCCESS
    stream.synchronize()
    check_bitexact(out2.cpu(), out.cpu())
    check_bitexact(ks.rms_norm(x, w, wl.eps).cpu(), out.cpu())
    gx, gr = x.clone(), r.clone()
    ks.fused_add_rms_norm(gx, gr, w, wl.eps)
    check_bitexact(gx.cpu(), fx.cpu())
    check_bitexact(gr.cpu(), fr.cpu())


def test_time_next_call_records_one_call():
    hip = _hip()
    x = workloads.random_case((2048, 4096), "bfloat16", 41)
    xd, wd = x["x"].cuda(), x["weight"].cuda()
    y_plain = ks.rms_norm(xd, wd, 1e-6)
    torch.cuda.synchronize()
    e0, e1 = hip.event(), hip.event()
    try:
        assert ks.ks_time_next_call(e0, e1) == b.KS_SUCCESS
        y_timed = ks.rms_norm(xd, wd, 1e-6)
        torch.cuda.synchronize()
        t = hip.elapsed_us(e0, e1)
        say("timed rms_norm 2048x4096 bf16:", f"{t:.2f} us")
        assert 0.5 < t < 5000.0
        check_bitexact(y_timed.cpu(), y_plain.cpu())
        # the request is spent: later calls leave both events where they were
        for _ in range(3):
            ks.rms_norm(xd, wd, 1e-6)
        torch.cuda.synchronize()
        assert hip.elapsed_us(e0, e1) == t
        # a call rejected by validation spends it too
        assert ks.ks_time_next_call(e0, e1) == b.KS_SUCCESS
        assert b.ks_rms_norm_ex(0, 0, 0, 4, 0, 1e-6, 2, None, 0) == b.KS_ERROR_INVALID_VALUE
        ks.rms_norm(xd, wd, 1e-6)
        torch.cuda.synchronize()
        assert hip.elapsed_us(e0, e1) == t
    finally:
        hip.destroy(e0)
        hip.destroy(e1)


def test_time_next_call_spans_every_kernel_of_a_call():
    """The backward with a weight gradient is two kernels (rows, then the dw
    column sums); the interval covers both and is longer than the row kernel's."""
    hip = _hip()
    inp = workloads.random_case((2048, 4096), "bfloat16", 42)
    x, dy, w = inp["x"].cuda(), inp["residual"].cuda(), inp["weight"].cuda()
    ws = torch.empty(b.ks_rms_norm_backward_workspace_size(2048, 4096), dtype=torch.uint8, device="cuda")
    dx0, dw0 = ks.rms_norm_backward(dy, x, w, 1e-5, workspace=ws)
    torch.cuda.synchronize()
    ev = [hip.event() for _ in range(4)]
    try:
        ks.ks_time_next_call(ev[0], ev[1])
        dx, dw = ks.rms_norm_backward(dy, x, w, 1e-5, workspace=ws)
        ks.ks_time_next_call(ev[2], ev[3])
        dx2, _ = ks.rms_norm_backward(dy, x, w, 1e-5, workspace=ws, weight_grad=False)
        torch.cuda.synchronize()
        both, rows_only = hip.elapsed_us(ev[0], ev[1]), hip.elapsed_us(ev[2], ev[3])
        say(f"backward 2048x4096 bf16: dx + dw {both:.2f} us, dx alone {rows_only:.2f} us")
        assert both > rows_only > 0.5
        check_bitexact(dx.cpu(), dx0.cpu())
        check_bitexact(dw.cpu(), dw0.cpu())
        check_bitexact(dx2.cpu(), dx0.cpu())
    finally:
        for e in ev:
            hip.destroy(e)


def test_policy_uses_the_device_compute_units():
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    say("device compute units", cus)
    for op in ("rms_norm", "fused_add_rms_norm", "softmax", "silu_and_mul", "rms_norm_residual"):
        for rows, hidden in ((1, 4096), (2048, 4096), (32768, 8192), (4, 65536)):
            for dtype in (torch.bfloat16, torch.float32):
                got = ks.get_plan(op, dtype, hidden, rows, workspace=op == "softmax").as_dict()
                want = ks.get_plan(op, dtype, hidden, rows, workspace=op == "softmax", compute_units=cus).as_dict()
                assert got == want, (op, rows, hidden, dtype)
