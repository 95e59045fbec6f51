"""Host-side checks of bench.py's measurement plumbing (no GPU): the traffic
calibration against a plain copy, the source hash gate, and the stats summary."""
import csv
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402

COLS = ["Correlation_Id", "Dispatch_Id", "Agent_Id", "Queue_Id", "Process_Id", "Thread_Id",
        "Grid_Size", "Kernel_Id", "Kernel_Name", "Workgroup_Size", "LDS_Block_Size",
        "Scratch_Size", "VGPR_Count", "Accum_VGPR_Count", "SGPR_Count", "Counter_Name",
        "Counter_Value", "Start_Timestamp", "End_Timestamp"]


def _csv(d, counter, entries):
    os.makedirs(d, exist_ok=True)
    with open(os.path.join(d, "x_counter_collection.csv"), "w", newline="") as f:
        w = csv.DictWriter(f, COLS)
        w.writeheader()
        for i, (name, val) in enumerate(entries):
            r = {c: 0 for c in COLS}
            r.update(Dispatch_Id=i, Kernel_Name=name, Counter_Name=counter, Counter_Value=val)
            w.writerow(r)


def test_traffic_calibration(tmp_path, monkeypatch):
    monkeypatch.setattr(bench, "TRAFFIC_DIR", str(tmp_path))
    out = tmp_path / "traffic_x.json"
    neg = "void at::native::vectorized_elementwise_kernel<4, at::native::neg_kernel_cuda(...)>"
    dw = "kd::(anonymous namespace)::dw_kernel(kd::DwArgs)"
    fwd = "void kd::(anonymous namespace)::logits_kernel<0>(kd::LogitsArgs)"
    # copy of 1024 MiB: the fetch counter reads 2x, the write counter reads exactly
    _csv(tmp_path / "f", "FETCH_SIZE", [(neg, 2 * 1024 * 1024.0), (dw, 100.0), (dw, 300.0),
                                        (fwd, 50.0)])
    _csv(tmp_path / "w", "WRITE_SIZE", [(neg, 1024 * 1024.0), (dw, 10.0), (dw, 30.0),
                                        (fwd, 4.0)])
    cfg = {"workload": "x"}
    bench.write_traffic(str(tmp_path / "f"), str(tmp_path / "w"), 1024, "cmd", cfg)
    doc = json.loads(out.read_text())
    assert doc["calibration"]["fetch_scale"] == pytest.approx(0.5)
    assert doc["calibration"]["write_scale"] == pytest.approx(1.0)
    e = doc["kernels"]["dw"]
    assert e["fetch_bytes_per_launch"] == pytest.approx(0.5 * 200.0 * 1024)
    assert e["write_bytes_per_launch"] == pytest.approx(20.0 * 1024)
    assert e["bytes_per_launch"] == pytest.approx((100.0 + 20.0) * 1024)
    assert doc["kernels"]["logits_fwd"]["bytes_per_launch"] == pytest.approx((25.0 + 4.0) * 1024)
    # the gate: same sources and workload -> reported; another workload -> None
    assert bench.measured_traffic("dw", cfg) == pytest.approx(120.0 * 1024)
    assert bench.measured_traffic("dw", {"workload": "y"}) is None
    doc["source_sha256"] = "0" * 64
    out.write_text(json.dumps(doc))
    assert bench.measured_traffic("dw", cfg) is None


def test_traffic_needs_copy_kernel(tmp_path, monkeypatch):
    monkeypatch.setattr(bench, "TRAFFIC_DIR", str(tmp_path))
    _csv(tmp_path / "f", "FETCH_SIZE", [("dw_kernel", 1.0)])
    _csv(tmp_path / "w", "WRITE_SIZE", [("dw_kernel", 1.0)])
    with pytest.raises(SystemExit):
        bench.write_traffic(str(tmp_path / "f"), str(tmp_path / "w"), 64, "", {"workload": "x"})


def test_kernel_classes():
    assert bench._kernel_class("kd::(anonymous namespace)::dh_reduce_kernel(float const*)") == "dh_reduce"
    assert bench._kernel_class("kd::(anonymous namespace)::dh_kernel(kd::DhArgs)") == "dh"
    assert bench._kernel_class("void kd::(anonymous namespace)::logits_kernel<1>(kd::LogitsArgs)") == \
        "logits_bwd"
    assert bench._kernel_class("at::native::whatever") is None


def test_stats_summary(tmp_path):
    d = tmp_path / "s"
    d.mkdir()
    with open(d / "x_kernel_stats.csv", "w", newline="") as f:
        w = csv.writer(f)
        w.writerow(["Name", "Calls", "TotalDurationNs", "AverageNs", "Percentage", "MinNs", "MaxNs",
                    "StdDev"])
        w.writerow(["kd::(anonymous namespace)::dw_kernel(kd::DwArgs)", 4, 8e6, 2e6, 60.0, 1.9e6,
                    2.1e6, 0])
        w.writerow(["kd::(anonymous namespace)::dh_kernel(kd::DhArgs)", 8, 4e6, 5e5, 40.0, 4e5, 6e5, 0])
    md = tmp_path / "s.md"
    bench.write_stats(str(d), str(md), "rocprofv3 ... -- python3 bench.py", '{"metric": "m"}\n')
    text = md.read_text()
    assert "| dw | 4 | 8.000 | 2.0000 |" in text and "rocprofv3 ... -- python3 bench.py" in text
    assert text.index("| dw |") < text.index("| dh |")


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2 and "one GPU" in r.stderr


def test_source_hash_ignores_comments_not_code():
    import bench
    a = "int f(int x) {\n  return x + 1;  // one more\n}\n/* block\n comment */\n"
    b = "int f(int x) {\n    return x + 1;\n}\n"
    c = "int f(int x) {\n  return x + 2;\n}\n"
    assert bench.code_text(a) == bench.code_text(b)
    assert bench.code_text(a) != bench.code_text(c)
    assert bench.source_hash() == bench.source_hash(
        lambda rel: open(os.path.join(ROOT, rel)).read() + "\n// a trailing comment\n")
