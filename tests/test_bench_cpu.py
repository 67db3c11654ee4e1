"""Measurement logic that runs without a GPU: the byte model, the kernel-source
hash, the counter post-processing and the regression gate (cases matched by
op, dtype and shape; exit status 2 past the threshold, as the Triton Kernel
Lab README's "Regression Gate" section describes)."""
import json
import os
import subprocess
import sys

import numpy as np
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


def test_distribution_nearest_rank():
    d = bench.distribution([float(v) for v in range(1, 101)])
    assert (d["n"], d["min"], d["p50"], d["p95"], d["p99"], d["max"]) == (100, 1, 50, 95, 99, 100)
    assert d["mean"] == pytest.approx(50.5)
    one = bench.distribution([3.25])
    assert one["p50"] == one["p99"] == one["min"] == one["max"] == 3.25


def test_sweep_set_adds_dtype_variants_once():
    wls = bench.sweep_set(["bf16", "fp16", "fp32"])
    names = [w.name for w in wls]
    for n in ("C1-fp16", "C1-fp32", "C2-fp16", "C2-fp32", "C3b-fp32"):
        assert n in names
    # C3 already covers fp16 at 2048x4096, so C3b's fp16 variant would repeat its cases
    assert "C3b-fp16" not in names
    keys = [(w.ops, w.dtype, w.rows, w.hidden) for w in wls]
    assert len(keys) == len(set(keys))
    v = next(w for w in wls if w.name == "C1-fp32")
    c1 = bench.workloads.WORKLOADS["C1"]
    assert (v.rows, v.hidden, v.seed_x, v.seed_w, v.eps, v.dtype) == (c1.rows, c1.hidden, c1.seed_x, c1.seed_w,
                                                                     c1.eps, "float32")


def test_streamref_library_exports_and_rejects_bad_sizes():
    """The reference streams check sizes before any launch (no GPU needed)."""
    ref = bench.StreamRef()
    for name in ("ksref_read", "ksref_write", "ksref_copy", "ksref_copy_rows", "ksref_inplace4", "ksref_empty",
                 "ksref_spin", "ksref_timeline", "ksref_wall_clock_khz"):
        assert hasattr(ref.h, name)
    a, b = 0x10000000, 0x20000000
    assert ref.h.ksref_copy(a, b, 4095, 0, None, None, None) == 1          # not a whole 4 KiB block
    assert ref.h.ksref_copy(a, b, 0, 0, None, None, None) == 1
    assert ref.h.ksref_copy(a, b, (1 << 31) + 4096, 0, None, None, None) == 1
    assert ref.h.ksref_copy(a, b, 4096, 3, None, None, None) == 1          # unknown store policy
    assert ref.h.ksref_write(b, 4096, 7, None, None, None) == 1
    assert ref.h.ksref_copy_rows(a, b, 4096, 2, None, None, None) == 1     # 2 pieces: blocks of 8 KiB
    assert ref.h.ksref_copy_rows(a, b, 8192, 3, None, None, None) == 1
    assert ref.h.ksref_inplace4(a, b, 4096 * 8 + 4096, 8, None, None, None) == 1
    assert ref.h.ksref_empty(0, None, None, None) == 1
    assert ref.h.ksref_spin(0, None) == 1 and ref.h.ksref_spin(100001, None) == 1
    st, need = 0x30000000, 4 * 64                                          # one 32 KiB block: 4 waves of 64 B
    assert ref.h.ksref_timeline(a, b, 32768, 0, 1, st, need - 8, None, None, None) == 1   # stamps too small
    assert ref.h.ksref_timeline(a, b, 32768, 0, 1, None, need, None, None, None) == 1
    assert ref.h.ksref_timeline(a, b, 32768, 0, 1, st + 4, need, None, None, None) == 1   # not 8-byte aligned
    assert ref.h.ksref_timeline(a, b, 32768, 3, 1, st, need, None, None, None) == 1       # unknown layout
    assert ref.h.ksref_timeline(a, b, 32768, 1, 3, st, need, None, None, None) == 1       # unknown store policy
    assert ref.h.ksref_timeline(a, b, 16384, 0, 1, st, need, None, None, None) == 1       # not a whole 32 KiB block
    assert ref.h.ksref_wall_clock_khz(None) == 1


def test_wave_timeline_statistics():
    """Per-call statistics of the wave records, on a hand-made call: 4 waves,
    clock ticks of 10 ns."""
    tick_us = 0.01
    st = np.zeros((4, 8), dtype=np.int64)
    #          start first loaded scaled issued acked
    st[:, :6] = [[100, 150, 200, 210, 215, 300],
                 [110, 240, 250, 260, 262, 330],
                 [120, 130, 220, 225, 230, 280],
                 [130, 300, 400, 402, 404, 500]]
    s = bench.timeline_call_stats(st, tick_us, 5.0)
    assert s["span_us"] == pytest.approx(4.0) and s["outside_waves_us"] == pytest.approx(1.0)
    assert s["start_ramp_us"] == pytest.approx(0.3)
    assert s["first_data_us"] == pytest.approx(0.3) and s["first_data_p50_us"] == pytest.approx((0.5 + 1.4) / 2)
    assert s["first_load_p50_us"] == pytest.approx((0.5 + 1.3) / 2)
    assert s["first_loaded_us"] == pytest.approx(1.0) and s["last_loaded_us"] == pytest.approx(3.0)
    assert s["first_issued_us"] == pytest.approx(1.15) and s["last_issued_us"] == pytest.approx(3.04)
    assert s["load_max_us"] == pytest.approx(2.7) and s["load_p50_us"] == pytest.approx(1.2)
    assert s["ack_p50_us"] == pytest.approx((0.68 + 0.85) / 2)
    assert s["max_resident_waves"] == 4
    h = bench.timeline_histogram(st, tick_us, bucket_us=1.0)
    assert [r["started"] for r in h] == [4, 0, 0, 0, 0]
    assert [r["first"] for r in h] == [2, 1, 1, 0, 0]
    assert [r["loaded"] for r in h] == [0, 3, 0, 1, 0]
    assert [r["acked"] for r in h] == [0, 1, 2, 0, 1]
    st[3, :6] = [400, 420, 450, 451, 452, 460]     # starts after the others have finished
    assert bench.timeline_call_stats(st, tick_us, 5.0)["max_resident_waves"] == 3


def test_streams_table_is_consistent():
    for name, (mult, _) in bench.STREAMS.items():
        assert name in bench.STREAM_DESCRIPTIONS
        assert mult == (1 if name.startswith(("read", "write")) else 4 if name.startswith("in place") else 2)


def test_trace_summary_renders_a_kernel_trace(tmp_path):
    d = tmp_path / "trace"
    d.mkdir()
    hdr = ('"Kind","Kernel_Name","Start_Timestamp","End_Timestamp","LDS_Block_Size","Scratch_Size","VGPR_Count",'
           '"Accum_VGPR_Count","SGPR_Count","Workgroup_Size_X","Grid_Size_X"\n')
    k = "void ks::fused_add_rms_norm_vec<ks::bf16, 64, 8, 256, 2, 2, true>(ks::Params)"
    r = "void ks::rms_norm_vec<ks::bf16, 64, 8, 256, 2, 2, false>(ks::Params)"
    lines = [f'"KERNEL_DISPATCH","{k}",{1000 * i},{1000 * i + 11000 + 10 * i},0,0,52,0,32,256,131072\n' for i in range(5)]
    lines += [f'"KERNEL_DISPATCH","{r}",{1000 * i},{1000 * i + 6000},0,0,52,0,48,256,131072\n' for i in range(5)]
    lines += ['"KERNEL_DISPATCH","copy_one<17>",0,7000,0,0,4,0,32,256,1048576\n',
              '"KERNEL_DISPATCH","copy_one<17>",0,325000,0,0,4,0,32,256,67108864\n']
    (d / "b_kernel_trace.csv").write_text(hdr + "".join(lines))
    wl = bench.workloads.WORKLOADS["C3b"]
    text = bench.trace_summary(wl, str(d), None, "rocprofv3 --kernel-trace -- python3 bench.py")
    assert "| fused_add_rms_norm | 67117056 | 11.020 | 11.020 |" in text
    assert "| rms_norm | 33562624 | 6.000 | 6.000 |" in text
    assert "[grid 1048576]" in text and "[grid 67108864]" in text


def test_trace_contexts_group_by_predecessor_and_gap(tmp_path):
    d = tmp_path / "trace"
    d.mkdir()
    hdr = '"Kind","Kernel_Name","Start_Timestamp","End_Timestamp"\n'
    r = "void ks::rms_norm_vec<ks::bf16, 64, 8, 256, 2, 2, false>(ks::Params)"
    f = "void ks::fused_add_rms_norm_vec<ks::bf16, 64, 8, 256, 2, 2, true>(ks::Params)"
    ev = [("spin_kernel(unsigned long)", 0, 300000),     # head start
          (r, 300500, 305500),                          # after the spin, 0.5 us gap: 5 us
          (r, 306000, 312000),                          # back to back: 6 us
          (r, 312500, 318500),                          # back to back: 6 us
          (r, 330000, 337000),                          # 11.5 us gap: 7 us
          (f, 337500, 348500),                          # fused after rms, back to back: 11 us
          (r, 349000, 355400)]                          # rms after fused: 6.4 us
    rows = [f'"KERNEL_DISPATCH","{n}",{s0},{e0}\n' for n, s0, e0 in ev]
    (d / "b_kernel_trace.csv").write_text(hdr + "".join(reversed(rows)))    # order comes from the timestamps
    ctx = bench.trace_contexts(str(d))
    assert ctx[("rms_norm", "spin (head start)", "< 2 us")] == {"n": 1, "mean": 5.0, "p50": 5.0}
    assert ctx[("rms_norm", "rms_norm", "< 2 us")]["n"] == 2 and ctx[("rms_norm", "rms_norm", "< 2 us")]["mean"] == 6.0
    assert ctx[("rms_norm", "rms_norm", ">= 2 us")]["mean"] == 7.0
    assert ctx[("fused_add_rms_norm", "rms_norm", "< 2 us")]["mean"] == 11.0
    assert ctx[("rms_norm", "fused_add_rms_norm", "< 2 us")]["mean"] == pytest.approx(6.4)
    assert len(ctx) == 5


def test_op_and_dtype_variants_keep_inputs():
    c3b = bench.workloads.WORKLOADS["C3b"]
    v = bench.workloads.with_ops(c3b, ("rms_norm",))
    assert v.ops == ("rms_norm",) and v.name == "C3b/rms_norm"
    assert (v.seed_x, v.seed_w, v.rows, v.hidden, v.dtype) == (c3b.seed_x, c3b.seed_w, c3b.rows, c3b.hidden, c3b.dtype)
    assert bench.workloads.with_ops(c3b, c3b.ops) is c3b
    with pytest.raises(ValueError):
        bench.workloads.with_ops(c3b, ("softmax",))
    res = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--op", "softmax"], capture_output=True,
                         text=True, cwd=ROOT)
    assert res.returncode != 0
