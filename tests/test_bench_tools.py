"""CPU checks of the benchmark's measurement plumbing: the traffic summary made
from rocprofv3 counter files (calibration against the page copy, hash gate that
voids a summary once a kernel source changes) and the GPU-count guard."""
import csv
import os
import subprocess
import sys

import pytest

import bench

COPY = "kda::copy_kernel(kda::CopyArgs)"
SCAN = "void kda::scan_kernel<128, unsigned short, 1>(kda::ScanArgs)"
PREP = "void kda::prep2_kernel<128>(kda::PrepArgs, int)"


def _counters(d, counter, rows):
    os.makedirs(d, exist_ok=True)
    with open(os.path.join(d, "run_counter_collection.csv"), "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=["Kernel_Name", "Counter_Name", "Counter_Value"])
        w.writeheader()
        for name, value in rows:
            w.writerow({"Kernel_Name": name, "Counter_Name": counter, "Counter_Value": value})


def test_traffic_summary_calibration_and_hash_gate(tmp_path, monkeypatch):
    copy_kib = 256 * 2 * 1024  # 256 pages of 2 MiB, in KiB, each way
    # the fetch counter reads half the copy's bytes (factor 2), the write counter all of them
    _counters(tmp_path / "f", "FETCH_SIZE", [(COPY, copy_kib / 2), (SCAN, 1000.0), (SCAN, 3000.0),
                                             (PREP, 400.0)])
    _counters(tmp_path / "w", "WRITE_SIZE", [(COPY, copy_kib), (SCAN, 500.0), (SCAN, 500.0),
                                             (PREP, 100.0)])
    md = bench.summarize_pmc(str(tmp_path / "f"), str(tmp_path / "w"), ["rocprofv3 ..."])
    assert "FETCH_SIZE x 2.000, WRITE_SIZE x 1.000" in md
    summary = tmp_path / "traffic.md"
    summary.write_text(md)
    monkeypatch.setattr(bench, "TRAFFIC_SUMMARY", str(summary))
    # scan: mean fetch 2000 KiB x 2 + mean write 500 KiB, per launch
    assert bench.recorded_traffic("kda_prefill_scan") == pytest.approx((2000 * 2 + 500) * 1024, rel=1e-6)
    assert bench.recorded_traffic("kda_prefill_prep") == pytest.approx((400 * 2 + 100) * 1024, rel=1e-6)
    assert bench.recorded_traffic("kda_decode_step") is None  # not in the counter files
    # once the kernel's source no longer hashes to the recorded value, no traffic is reported
    real = bench.source_hash
    monkeypatch.setattr(bench, "source_hash",
                        lambda name: "0" * 16 if name == "kda_prefill.hip" else real(name))
    assert bench.recorded_traffic("kda_prefill_scan") is None


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, bench.__file__, "--gpus", "2"], capture_output=True, text=True,
                       timeout=120)
    assert r.returncode == 2 and "one GPU" in r.stderr
