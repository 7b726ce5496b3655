"""bench.py: the one-line JSON contract, and the host-side arithmetic behind
its roofline fields.

The counter summary turns two rocprofv3 --pmc runs into HBM bytes per launch
by scaling each counter with what it reads for a copy of known size; the
bench then reports those bytes as roofline.traffic only while the kernel's
sources are unchanged. The CPU tests below feed that code synthetic counter
files whose answer is known. The GPU test runs a short bench and checks the
line it prints.
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

WORKLOAD = "B64_V262144_masked_quarters"
N_BYTES = 64 * 262144 * 4
KNAME = "ts_fused<8, true, 0>"


def _write_counters(d, counter, per_dispatch):
    """per_dispatch: {kernel name: [[value per XCD row, ...] per dispatch]}."""
    os.makedirs(d, exist_ok=True)
    with open(os.path.join(d, "x_counter_collection.csv"), "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"])
        w.writeheader()
        did = 0
        for name, dispatches in per_dispatch.items():
            for parts in dispatches:
                did += 1
                for v in parts:
                    w.writerow({"Dispatch_Id": did, "Kernel_Name": f"void tsk::{name}(args)",
                                "Counter_Name": counter, "Counter_Value": v})
        # a row of another counter must be ignored
        w.writerow({"Dispatch_Id": did + 1, "Kernel_Name": f"void tsk::{KNAME}(args)",
                    "Counter_Name": "SQ_WAVES", "Counter_Value": 1e9})


def test_more_than_one_gpu_is_refused(capsys):
    assert bench.main(["--gpus", "2"]) == 2
    assert "one GPU" in capsys.readouterr().err


def test_counter_summary_scales_by_the_copy(tmp_path, monkeypatch):
    monkeypatch.setattr(bench, "PROFILES", str(tmp_path / "profiles"))
    kib = N_BYTES / 1024.0
    # the copy's FETCH_SIZE reads half its bytes, WRITE_SIZE all of them; each
    # dispatch's value is split over several rows (one per XCD) and summed
    _write_counters(tmp_path / "f", "FETCH_SIZE", {
        "ts_copy_vec": [[kib / 4] * 2, [kib / 4] * 2],
        KNAME: [[0.3 * kib, 0.2 * kib], [0.45 * kib, 0.05 * kib]],
    })
    _write_counters(tmp_path / "w", "WRITE_SIZE", {
        "ts_copy_vec": [[kib / 2] * 2, [kib]],
        KNAME: [[1.02 * kib], [0.51 * kib, 0.51 * kib]],
    })
    out = bench.summarize_counters(str(tmp_path / "f"), str(tmp_path / "w"), WORKLOAD, KNAME, "ts_fused_c8192",
                                   "cmd")
    kv = dict(line.split("=", 1) for line in open(out).read().splitlines() if "=" in line and line[0] != "#")
    assert float(kv["fetch_factor"]) == pytest.approx(2.0)
    assert float(kv["write_factor"]) == pytest.approx(1.0)
    # the kernel fetched 0.5 of the copy's raw count (-> 1.0 N) and wrote 1.02 N
    assert float(kv["fetch_bytes_per_launch"]) == pytest.approx(1.00 * N_BYTES, rel=1e-6)
    assert float(kv["write_bytes_per_launch"]) == pytest.approx(1.02 * N_BYTES, rel=1e-6)
    assert int(kv["algorithmic_bytes_per_launch"]) == 2 * N_BYTES
    assert float(kv["traffic_over_algorithmic"]) == pytest.approx(1.01, abs=1e-4)
    assert int(kv["dispatches_fetch"]) == 2 and int(kv["dispatches_write"]) == 2
    # read back for roofline.traffic while the sources match, and not after
    assert bench.read_traffic("ts_fused_c8192", WORKLOAD) == pytest.approx(2.02 * N_BYTES, abs=1)
    monkeypatch.setattr(bench, "kernel_source_hash", lambda tag="": "changed")
    assert bench.read_traffic("ts_fused_c8192", WORKLOAD) is None


def test_counter_summary_refuses_missing_copy(tmp_path, monkeypatch):
    monkeypatch.setattr(bench, "PROFILES", str(tmp_path / "profiles"))
    _write_counters(tmp_path / "f", "FETCH_SIZE", {KNAME: [[1.0]]})
    _write_counters(tmp_path / "w", "WRITE_SIZE", {KNAME: [[1.0]]})
    with pytest.raises(SystemExit):
        bench.summarize_counters(str(tmp_path / "f"), str(tmp_path / "w"), WORKLOAD, KNAME, "ts_fused_c8192", "c")


def test_source_hash_families_are_separate():
    h_fused, h_draw = bench.kernel_source_hash("ts_fused_c8192"), bench.kernel_source_hash("ts_draw_partials")
    assert h_fused == bench.kernel_source_hash("ts_fused_c4096")
    assert h_fused != h_draw


def test_trace_summary_orders_by_total_time(tmp_path, monkeypatch):
    monkeypatch.setattr(bench, "PROFILES", str(tmp_path / "profiles"))
    d = tmp_path / "t" / "host"
    os.makedirs(d)
    with open(d / "x_kernel_stats.csv", "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=["Name", "Calls", "TotalDurationNs", "AverageNs", "MinNs", "MaxNs"])
        w.writeheader()
        w.writerow({"Name": "small", "Calls": 10, "TotalDurationNs": 1000, "AverageNs": 100, "MinNs": 90,
                    "MaxNs": 110})
        w.writerow({"Name": KNAME, "Calls": 2, "TotalDurationNs": 46000, "AverageNs": 23000, "MinNs": 22000,
                    "MaxNs": 24000})
    out = bench.summarize_trace(str(tmp_path / "t"), WORKLOAD, KNAME, "ts_fused_c8192", "cmd")
    rows = [l for l in open(out).read().splitlines() if not l.startswith("#")]
    assert rows[1].startswith(KNAME) and rows[2].startswith("small")
    assert rows[1].split()[-3:] == ["23.000", "22.000", "24.000"]


@pytest.mark.gpu
def test_bench_prints_one_json_line_with_the_contract_fields():
    print("[gpu] bench.py --steps 20 --warmup 5 --extras none --cpu-seconds 1", flush=True)
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--steps", "20", "--warmup", "5",
                        "--extras", "none", "--cpu-seconds", "1"],
                       capture_output=True, text=True, timeout=300, cwd=ROOT)
    assert r.returncode == 0, r.stderr[-2000:]
    lines = [l for l in r.stdout.splitlines() if l.startswith("{")]
    assert len(lines) == 1
    j = json.loads(lines[0])
    assert j["n_gpus"] == 1 and j["steps"] == 20 and j["warmup"] == 5
    assert j["unit"] == "GB/s" and j["higher_is_better"] is True and j["data"] == "synthetic"
    assert j["vs_baseline"] is None and j["dtype"] == "f32"
    assert j["config"]["workload"] == WORKLOAD
    assert j["ms_per_step"] == pytest.approx(j["us_per_call"] / 1000.0, rel=1e-3)
    assert j["value"] == pytest.approx(2 * N_BYTES / j["us_per_call"] / 1e3, rel=1e-3)
    rf = j["roofline"]
    assert rf["bound"] == "hbm" and rf["unit"] == "GB/s" and rf["peak"] == 8000.0
    assert rf["achieved"] == j["value"] and rf["frac"] == pytest.approx(rf["achieved"] / rf["peak"], abs=1e-4)
    assert rf["traffic"] is None or rf["traffic"] > 2 * N_BYTES * 0.99
    assert j["outputs_sane"] is True
    cb = j["cpu_baseline"]
    assert cb["kind"] == "oracle" and cb["unit"] == "GB/s" and cb["value"] > 0 and cb["cores"] >= 1
    assert cb["sample"]
