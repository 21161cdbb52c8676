"""Host-side parts of the benchmark, without a GPU.

- A request for more than one GPU is refused before anything touches a device.
- Two rocprofv3 counter runs (FETCH_SIZE, then WRITE_SIZE, KiB per dispatch)
  become HBM bytes per launch, each scaled by what the same counter reads for
  the 1 GiB device copy of the same run.
- A counter summary applies only to the library sources and the kernel it was
  taken with; otherwise the benchmark reports no traffic figure.

The counter files here are synthetic CSVs in the layout rocprofv3 writes
(one row per counter instance; the digest sums them per dispatch).
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
from dense_gemm_16_amd import inputs  # noqa: E402

GEMM = "void migemm::mfma16_direct_kernel<migemm::DirectCfg<migemm::bf16_t, 256, 256>>(long)"


def _write_pass(d, counter, copy_kib, gemm_kib, reps=3, copies=3):
    """A profile pass: a fill, `copies` 1 GiB copies, then `reps` GEMM launches.
    Each dispatch's value is split over two instances (two rows)."""
    d.mkdir(parents=True)
    rows = [(1, "void at::native::vectorized_elementwise_kernel<FillFunctor>", 20.0)]
    rows += [(2 + i, "__amd_rocclr_copyBuffer", copy_kib) for i in range(copies)]
    rows += [(2 + copies + i, GEMM, gemm_kib) for i in range(reps)]
    with open(d / "run_counter_collection.csv", "w", newline="") as f:
        w = csv.writer(f)
        w.writerow(["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"])
        for did, name, v in rows:
            w.writerow([did, name, counter, v * 0.25])
            w.writerow([did, name, counter, v * 0.75])


def test_more_than_one_gpu_is_refused():
    p = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=300)
    assert p.returncode == 2
    assert "one GPU" in p.stderr
    assert p.stdout == ""  # no JSON line


def test_digest_scales_each_counter_by_the_copy(tmp_path, monkeypatch):
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(tmp_path / "traffic.json"))
    w = inputs.WORKLOADS["c4-bf16-8192"]
    # FETCH_SIZE reads half of the copy's 1 GiB (factor 2), WRITE_SIZE all of it
    _write_pass(tmp_path / "fetch", "FETCH_SIZE", 524288.0, 786432.0)
    _write_pass(tmp_path / "write", "WRITE_SIZE", 1048576.0, 262144.0)
    bench.digest_counters(w, str(tmp_path / "fetch"), str(tmp_path / "write"), 3)
    e = json.load(open(tmp_path / "traffic.json"))["entries"][w.name]
    assert e["fetch_factor"] == 2.0 and e["write_factor"] == 1.0
    assert e["fetch_bytes_per_launch"] == 786432 * 2 * 1024
    assert e["write_bytes_per_launch"] == 262144 * 1024
    assert e["hbm_bytes_per_launch"] == 786432 * 2 * 1024 + 262144 * 1024
    assert e["source_hash"] == bench.source_hash()
    assert e["fetch_kernel_in_csv"].startswith("void migemm::mfma16_direct_kernel")

    # the summary applies to this kernel at these sources only
    got, _ = bench.traffic_for(e["kernel"], w.name)
    assert got == e["hbm_bytes_per_launch"]
    assert bench.traffic_for("other[kernel]", w.name)[0] is None
    assert bench.traffic_for(e["kernel"], "c1-f32-1024") == (None, "workload not profiled")
    monkeypatch.setattr(bench, "source_hash", lambda: "0" * 16)
    assert bench.traffic_for(e["kernel"], w.name) == (
        None, "kernel changed since the counters were taken")


def test_digest_takes_the_median_of_the_gemm_launches(tmp_path, monkeypatch):
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(tmp_path / "traffic.json"))
    w = inputs.WORKLOADS["c4-bf16-8192"]
    _write_pass(tmp_path / "fetch", "FETCH_SIZE", 524288.0, 0.0)
    _write_pass(tmp_path / "write", "WRITE_SIZE", 1048576.0, 262144.0)
    # make the three GEMM fetches 100, 300 and 200 KiB: the median is 200
    path = tmp_path / "fetch" / "run_counter_collection.csv"
    rows = list(csv.reader(open(path)))
    for r in rows[1:]:
        if r[0] in ("5", "6", "7"):
            r[3] = str({"5": 50.0, "6": 150.0, "7": 100.0}[r[0]])
    with open(path, "w", newline="") as f:
        csv.writer(f).writerows(rows)
    bench.digest_counters(w, str(tmp_path / "fetch"), str(tmp_path / "write"), 3)
    e = json.load(open(tmp_path / "traffic.json"))["entries"][w.name]
    assert e["fetch_kib_raw"] == 200.0
    assert e["fetch_bytes_per_launch"] == 200 * 2 * 1024


def test_digest_refuses_a_run_without_the_calibration_copies(tmp_path, monkeypatch):
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(tmp_path / "traffic.json"))
    w = inputs.WORKLOADS["c4-bf16-8192"]
    _write_pass(tmp_path / "fetch", "FETCH_SIZE", 524288.0, 786432.0, copies=0)
    _write_pass(tmp_path / "write", "WRITE_SIZE", 1048576.0, 262144.0)
    with pytest.raises(SystemExit):
        bench.digest_counters(w, str(tmp_path / "fetch"), str(tmp_path / "write"), 3)
    assert not (tmp_path / "traffic.json").exists()
