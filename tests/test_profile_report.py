"""The arithmetic behind `bench.py`'s roofline.traffic: profile_report turns
rocprofv3's FETCH_SIZE / WRITE_SIZE (KiB per dispatch) into bytes per launch,
scaled by what the same counters read for a plain 256 MiB device copy.  Run on
synthetic counter files with known values (CPU only)."""

import csv
import json
import os
import subprocess
import sys

import workloads

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
W = "prefill_b1h32n2048d64_f16"


def _counters(path, rows):
    os.makedirs(path, exist_ok=True)
    with open(os.path.join(path, "run_counter_collection.csv"), "w", newline="") as f:
        w = csv.writer(f)
        w.writerow(["Kernel_Name", "Counter_Name", "Counter_Value"])
        w.writerows(rows)


def test_warm_traffic_from_counters(tmp_path):
    g = tmp_path / "rocprof"
    kern = "_ZN2fa4mfma17fa_forward_kernelIDF16_Li64ELb0ELb0ELi8ELi1ELi1EEEvNS0_4ArgsE"
    # two dispatches each: means 1100 KiB fetched and 500 KiB written
    _counters(g / f"prof_FETCH_SIZE_{W}", [[kern, "FETCH_SIZE", 1000.0], [kern, "FETCH_SIZE", 1200.0]])
    _counters(g / f"prof_WRITE_SIZE_{W}", [[kern, "WRITE_SIZE", 500.0], [kern, "WRITE_SIZE", 500.0]])
    # the 256 MiB copy: FETCH_SIZE reads half the bytes (factor 0.5), WRITE_SIZE all of them (factor 1)
    _counters(g / "prof_FETCH_SIZE_copy256", [["__amd_rocclr_copyBuffer", "FETCH_SIZE", 131072.0]])
    _counters(g / "prof_WRITE_SIZE_copy256", [["__amd_rocclr_copyBuffer", "WRITE_SIZE", 262144.0]])
    os.makedirs(g / f"prof_trace_{W}")
    with open(g / f"prof_trace_{W}" / "run_kernel_stats.csv", "w", newline="") as f:
        w = csv.writer(f)
        w.writerow(["Name", "Calls", "TotalDurationNs", "AverageNs", "Percentage", "MinNs", "MaxNs", "StdDev"])
        w.writerow([kern, 10, 400000, 40000.0, 99.0, 39000, 41000, 10.0])
    rec = {"kernel_source_hash": "0123456789abcdef", "value": 850.0, "steps": 100,
           "roofline": {"kernel_us_mean": 40.4}}
    (g / f"prof_trace_{W}.log").write_text("log line\n" + json.dumps(rec) + "\n")
    out = tmp_path / "out"
    out.mkdir()
    subprocess.run([sys.executable, "-m", "tiled_attention_fa_amd.profile_report", "warm", "--workload", W,
                    "--dir", str(g), "--out-dir", str(out)], cwd=ROOT, check=True, capture_output=True)
    r = json.load(open(out / f"traffic_{W}.json"))
    assert r["copy_calibration"]["fetch_factor"] == 0.5 and r["copy_calibration"]["write_factor"] == 1.0
    assert r["hbm_read_bytes_per_launch"] == 1100 * 1024 * 2
    assert r["hbm_write_bytes_per_launch"] == 500 * 1024
    assert r["hbm_bytes_per_launch"] == 1100 * 1024 * 2 + 500 * 1024
    minb = workloads.min_bytes(workloads.get(W))
    assert r["min_bytes"] == minb
    assert abs(r["ratio_to_min"] - (1100 * 2048 + 500 * 1024) / minb) < 1e-4
    assert r["kernel_source_hash"] == "0123456789abcdef" and r["kernel"] == kern
    md = (out / f"fa_forward_{W}_hbm_bytes.md").read_text()
    assert "profile_report warm" in md and "FETCH_SIZE per dispatch (mean of 2)" in md
