"""Host logic of bench.py: the counter summaries and the derived lines.

Fake rocprofv3 CSV files stand in for the counter runs; the summaries are
written to a temporary directory, never to profiles/.
"""
import csv
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402
import workloads as W  # noqa: E402

KERN = "void firols::ols_fused_kernel<12, false>(firols::FusedArgs)"
COPY = "void at::native::vectorized_elementwise_kernel<4, at::native::neg_kernel_cuda>(int)"


def write_counters(d, rows):
    os.makedirs(d, exist_ok=True)
    with open(os.path.join(d, "run_counter_collection.csv"), "w", newline="") as f:
        wr = csv.DictWriter(f, fieldnames=["Kernel_Name", "Counter_Name", "Counter_Value"])
        wr.writeheader()
        for k, c, v in rows:
            wr.writerow({"Kernel_Name": k, "Counter_Name": c, "Counter_Value": v})


def run_main(monkeypatch, argv):
    monkeypatch.setattr(sys, "argv", ["bench.py"] + argv)
    old = bench.PROFILES_DIR
    try:
        bench.main()
    finally:
        bench.PROFILES_DIR = old


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=60)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def test_valu_summary_and_line(tmp_path, monkeypatch):
    add, mul, fma, instr = 1.0e6, 3.0e5, 2.0e5, 1.6e6
    rows = []
    for disp in range(4):    # four dispatches, the mean is taken
        for c, v in (("SQ_INSTS_VALU", instr), ("SQ_INSTS_VALU_ADD_F32", add),
                     ("SQ_INSTS_VALU_MUL_F32", mul), ("SQ_INSTS_VALU_FMA_F32", fma),
                     ("SQ_ACTIVE_INST_VALU", 5000.0), ("SQ_BUSY_CYCLES", 9000.0),
                     ("SQ_WAVES", 1024.0)):
            rows.append((KERN, c, v + (disp - 1.5)))
    rows.append((COPY, "SQ_INSTS_VALU", 7.0))      # other kernels are ignored
    write_counters(tmp_path / "valu", rows)
    prof = tmp_path / "prof"
    prof.mkdir()
    run_main(monkeypatch, ["--workload", "cfg2", "--summarize-valu", str(tmp_path / "valu"),
                           "--profiles-dir", str(prof), "--command", "rocprofv3 --pmc ..."])
    rec = json.load(open(prof / "valu.json"))["cfg2"]
    want = 64.0 * (add + mul + 2 * fma)
    assert rec["fp32_flops_per_launch"] == pytest.approx(want)
    w = W.WORKLOADS["cfg2"]
    samples = w.nchan * w.samples / len(w.calls)
    assert rec["fp32_flops_per_sample"] == pytest.approx(want / samples, abs=0.01)
    assert rec["valu_instr_per_sample"] == pytest.approx(64 * instr / samples, abs=0.01)
    assert rec["source_hash"] == bench.kernel_source_hash("cfg2")
    assert (prof / "ols_fused_kernel_12_false_cfg2_valu.md").exists()

    monkeypatch.setattr(bench, "PROFILES_DIR", str(prof))
    line = bench.valu_line("cfg2", 0.01)            # 10 us per launch
    assert line["achieved"] == pytest.approx(want / 1e-5 / 1e12, rel=1e-3)
    assert line["frac"] == pytest.approx(line["achieved"] / bench.VALU_PEAK_TFLOPS, rel=1e-3)
    # a record taken with other kernel sources is not used
    db = json.load(open(prof / "valu.json"))
    db["cfg2"]["source_hash"] = "0" * 16
    json.dump(db, open(prof / "valu.json", "w"))
    assert bench.valu_line("cfg2", 0.01) is None


def test_traffic_summary_calibrates_against_the_copy(tmp_path, monkeypatch):
    w = W.WORKLOADS["cfg2"]
    copy_kib = w.nchan * w.samples * 8 / 1024.0
    # the counter reads half the copy's bytes for FETCH_SIZE, all for WRITE_SIZE
    write_counters(tmp_path / "f", [(COPY, "FETCH_SIZE", copy_kib / 2), (KERN, "FETCH_SIZE", 3000.0),
                                    (KERN, "FETCH_SIZE", 3000.0)])
    write_counters(tmp_path / "w", [(COPY, "WRITE_SIZE", copy_kib), (KERN, "WRITE_SIZE", 6000.0)])
    prof = tmp_path / "prof"
    prof.mkdir()
    run_main(monkeypatch, ["--workload", "cfg2", "--summarize-pmc", str(tmp_path / "f"),
                           str(tmp_path / "w"), "--profiles-dir", str(prof)])
    rec = json.load(open(prof / "traffic.json"))["cfg2"]
    assert rec["fetch_scale"] == pytest.approx(2.0)
    assert rec["write_scale"] == pytest.approx(1.0)
    assert rec["bytes_per_launch"] == pytest.approx((2 * 3000.0 + 6000.0) * 1024, abs=1)
    alg = w.nchan * w.samples / len(w.calls) * 16
    assert rec["ratio"] == pytest.approx((2 * 3000.0 + 6000.0) * 1024 / alg, abs=1e-4)


def test_trace_summary_names_the_top_kernel(tmp_path, monkeypatch):
    d = tmp_path / "t"
    d.mkdir()
    with open(d / "run_kernel_stats.csv", "w", newline="") as f:
        wr = csv.DictWriter(f, fieldnames=["Name", "Calls", "TotalDurationNs", "AverageNs",
                                           "MinNs", "MaxNs", "Percentage"])
        wr.writeheader()
        wr.writerow({"Name": COPY, "Calls": 3, "TotalDurationNs": 300, "AverageNs": 100,
                     "MinNs": 90, "MaxNs": 110, "Percentage": 1.0})
        wr.writerow({"Name": KERN, "Calls": 400, "TotalDurationNs": 3.6e6, "AverageNs": 9000,
                     "MinNs": 8000, "MaxNs": 20000, "Percentage": 99.0})
    prof = tmp_path / "prof"
    prof.mkdir()
    run_main(monkeypatch, ["--workload", "cfg2", "--summarize-trace", str(d),
                           "--profiles-dir", str(prof)])
    text = open(prof / "ols_fused_kernel_12_false_cfg2_kernel_trace.md").read()
    assert "| 400 | 9.000 |" in text


def test_trace_summary_timed_region_from_the_bench_line(tmp_path, monkeypatch):
    """With --trace-stdout the summary averages the last steps x calls
    dispatches of the kernel, the timed region of the traced bench run."""
    d = tmp_path / "t"
    d.mkdir()
    with open(d / "run_kernel_stats.csv", "w", newline="") as f:
        wr = csv.DictWriter(f, fieldnames=["Name", "Calls", "TotalDurationNs", "AverageNs",
                                           "MinNs", "MaxNs", "Percentage"])
        wr.writeheader()
        wr.writerow({"Name": KERN, "Calls": 20, "TotalDurationNs": 2.0e5, "AverageNs": 10000,
                     "MinNs": 8000, "MaxNs": 20000, "Percentage": 100.0})
    with open(d / "run_kernel_trace.csv", "w", newline="") as f:
        wr = csv.DictWriter(f, fieldnames=["Kernel_Name", "Start_Timestamp", "End_Timestamp"])
        wr.writeheader()
        t = 0
        for i in range(20):
            # 8 slow warm-up dispatches (20 us), then 12 timed ones (8 us)
            dur = 20000 if i < 8 else 8000
            wr.writerow({"Kernel_Name": KERN, "Start_Timestamp": t, "End_Timestamp": t + dur})
            t += dur + 1000
        wr.writerow({"Kernel_Name": COPY, "Start_Timestamp": t, "End_Timestamp": t + 500})
    out = tmp_path / "stdout.log"
    line = {"metric": "m", "configs": {"cfg2": {"steps": 3, "calls_per_step": 4,
                                                "avg_launch_us": 8.4}}}
    out.write_text("some log line\n" + json.dumps(line) + "\n")
    prof = tmp_path / "prof"
    prof.mkdir()
    run_main(monkeypatch, ["--workload", "cfg2", "--summarize-trace", str(d),
                           "--trace-stdout", str(out), "--profiles-dir", str(prof)])
    text = open(prof / "ols_fused_kernel_12_false_cfg2_kernel_trace.md").read()
    assert "its last 12 dispatches (3 steps x 4 calls) average 8.000 us" in text
    assert "avg_launch_us (HIP events around the same steps" in text
    assert "is 8.4." in text
