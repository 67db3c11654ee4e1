"""Measurement logic that runs without a GPU: the byte model, the kernel-source
hash, the counter post-processing and the regression gate (cases matched by
op, dtype and shape; exit status 2 past the threshold, as the Triton Kernel
Lab README's "Regression Gate" section describes)."""
import json
import os
import subprocess
import sys

import pytest

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_algorithmic_bytes():
    # rms_norm: read x, write out, read weight once; fused: x and residual both ways
    assert bench.algorithmic_bytes("rms_norm", 2048, 4096, 2) == 33562624
    assert bench.algorithmic_bytes("fused_add_rms_norm", 2048, 4096, 2) == 67117056
    assert bench.algorithmic_bytes("fused_add_rms_norm", 4, 1536, 2) == 52224


def test_source_hash_ignores_comments(tmp_path, monkeypatch):
    a = tmp_path / "a.hpp"
    a.write_text("int f() { return 1; } // one\n")
    monkeypatch.setattr(bench, "KERNEL_SOURCES", [str(a)])
    h1 = bench.kernel_source_hash()
    a.write_text("/* a comment */\nint  f()  {\n return 1;\n}\n")
    assert bench.kernel_source_hash() == h1
    a.write_text("int f() { return 2; }\n")
    assert bench.kernel_source_hash() != h1


def _counter_csv(path, rows):
    os.makedirs(path, exist_ok=True)
    with open(os.path.join(path, "x_counter_collection.csv"), "w") as f:
        f.write('"Kernel_Name","Counter_Name","Counter_Value"\n')
        for name, counter, value in rows:
            f.write(f'"{name}","{counter}",{value}\n')


def test_traffic_summary(tmp_path, monkeypatch):
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(tmp_path / "t.json"))
    k = "void ks::fused_add_rms_norm_vec<ks::bf16, 64, 8, 256, 2, 2, true>(ks::Params)"
    # FETCH_SIZE counts half of what a copy reads: the calibration copy fixes the scale
    _counter_csv(tmp_path / "f", [(k, "FETCH_SIZE", 16384.0)] * 3)
    _counter_csv(tmp_path / "w", [(k, "WRITE_SIZE", 32768.0)] * 3)
    _counter_csv(tmp_path / "cf", [("__amd_rocclr_copyBuffer", "FETCH_SIZE", 131072.0)])
    _counter_csv(tmp_path / "cw", [("__amd_rocclr_copyBuffer", "WRITE_SIZE", 262144.0)])
    (tmp_path / "cf" / "calibration.json").write_text(json.dumps({"copy_calibration_bytes": 256 << 20}))
    bench.traffic_summary("C3b", *(str(tmp_path / d) for d in ("f", "w", "cf", "cw")))
    data = json.load(open(tmp_path / "t.json"))
    entry = data["kernels"]["C3b"][k]
    cal = data["calibration"]["C3b"]
    assert cal["fetch_scale"] == pytest.approx(2.0) and cal["write_scale"] == pytest.approx(1.0)
    assert entry["fetch_bytes"] == 32 << 20 and entry["write_bytes"] == 32 << 20
    assert data["workloads"]["C3b"]["fused_add_rms_norm"] == 64 << 20
    assert bench.load_traffic("C3b") == {"fused_add_rms_norm": 64 << 20}
    # a second workload on the same sources is merged; SwiGLU kernels are recognised
    s = "void ks::silu_and_mul_vec<ks::bf16, 512, 3, 512, 2, 2>(ks::SwigluParams)"
    _counter_csv(tmp_path / "f2", [(s, "FETCH_SIZE", 1024.0), (k, "FETCH_SIZE", 1.0)])
    _counter_csv(tmp_path / "w2", [(s, "WRITE_SIZE", 512.0)])
    bench.traffic_summary("S2", *(str(tmp_path / d) for d in ("f2", "w2", "cf", "cw")))
    data = json.load(open(tmp_path / "t.json"))
    assert set(data["workloads"]) == {"C3b", "S2"}
    assert data["workloads"]["S2"] == {"silu_and_mul": (2 << 20) + (512 << 10)}
    assert bench.kernel_op(k) == "fused_add_rms_norm" and bench.kernel_op("__amd_rocclr_copyBuffer") is None


def test_regressions():
    base = [{"op": "rms_norm", "dtype": "bfloat16", "rows": 2048, "hidden": 4096, "us_per_call": 6.0},
            {"op": "fused_add_rms_norm", "dtype": "bfloat16", "rows": 2048, "hidden": 4096, "us_per_call": 12.0}]
    cur = [{"op": "rms_norm", "dtype": "bfloat16", "rows": 2048, "hidden": 4096, "us_per_call": 6.5},
           {"op": "fused_add_rms_norm", "dtype": "bfloat16", "rows": 2048, "hidden": 4096, "us_per_call": 14.0},
           {"op": "rms_norm", "dtype": "float16", "rows": 2048, "hidden": 4096, "us_per_call": 99.0}]
    bad = bench.regressions(cur, base, 10.0)
    assert [r["case"][0] for r in bad] == ["fused_add_rms_norm"]
    assert bad[0]["regression_percent"] == pytest.approx(16.67, abs=0.01)
    assert bench.regressions(cur, base, 20.0) == []


def test_gpus_above_one_exits_with_message():
    res = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                         text=True, cwd=ROOT)
    assert res.returncode == 2 and "one GPU" in res.stderr
