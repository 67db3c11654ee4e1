"""The seeded input generator: deterministic, right shapes and distributions."""
import numpy as np
import torch

import workloads


def test_deterministic_and_shaped():
    wl = workloads.WORKLOADS["C3b"]
    a = workloads.make_inputs(wl, rows=64)
    b = workloads.make_inputs(wl, rows=64)
    for k in ("x", "residual", "weight"):
        assert torch.equal(a[k].view(torch.int16), b[k].view(torch.int16))
    assert a["x"].shape == (64, 4096) and a["x"].dtype == torch.bfloat16
    assert a["weight"].shape == (4096,)


def test_outliers_and_distributions():
    wl = workloads.WORKLOADS["C3"]
    inp = workloads.make_inputs(wl, rows=256)
    x = inp["x"].float()
    n = x.numel()
    # ~1% of elements scaled by 100: their magnitude is far outside N(0,1)
    big = (x.abs() > 8).sum().item()
    assert 0.008 * n < big < 0.0101 * n
    w = inp["weight"].float()
    assert 0.5 <= w.min().item() and w.max().item() <= 1.5
    r = inp["residual"].float()
    assert abs(r.std().item() - 0.5) < 0.01


def test_every_workload_describes_itself():
    for wl in workloads.WORKLOADS.values():
        d = wl.describe()
        assert f"[{wl.rows},{wl.hidden}]" in d and wl.dtype in d


def test_random_case_shapes():
    inp = workloads.random_case((2, 3, 5), "float16", 1)
    assert inp["x"].shape == (2, 3, 5) and inp["weight"].shape == (5,)
    assert np.isfinite(inp["x"].float().numpy()).all()
