"""Host-only logic of bench.py (no GPU): the one-GPU refusal, the HBM traffic summary built from
rocprofv3 counter files, and the source-hash check that keeps a stale summary out of the bench
line. The counter files here are small synthetic CSVs in rocprofv3's column layout."""
import csv
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402

HEAD = "void nr::(anonymous namespace)::" + bench.HEADLINE_KERNEL + "(nr::ResidentArgs)"
COPY = "nr::(anonymous namespace)::" + bench.COPY_KERNEL + "(float __vector(4) const*, ...)"
OTHER = "nr::(anonymous namespace)::fill_zero_kernel(unsigned int*, long)"


def _write_counters(path, counter, dispatches):
    """dispatches: (kernel name, value in KiB) in dispatch order."""
    with open(path, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"])
        w.writeheader()
        for i, (name, value) in enumerate(dispatches, start=1):
            w.writerow({"Dispatch_Id": i, "Kernel_Name": name, "Counter_Name": counter,
                        "Counter_Value": value})


def _run_bench(*args):
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py")] + list(args),
                          capture_output=True, text=True, timeout=120)


def test_bench_refuses_more_than_one_gpu():
    r = _run_bench("--gpus", "2")
    assert r.returncode == 2
    assert "one GPU" in r.stderr and r.stdout == ""


def test_bench_refuses_zero_steps():
    r = _run_bench("--steps", "0")
    assert r.returncode == 2 and "--steps" in r.stderr


def test_counter_rows_stop_at_the_first_dispatch_of_another_kernel(tmp_path):
    p = tmp_path / "c.csv"
    _write_counters(p, "FETCH_SIZE", [(OTHER, 1.0), (HEAD, 10.0), (HEAD, 12.0), (COPY, 50.0),
                                      (HEAD, 99.0)])
    assert bench._counter_rows(p, "FETCH_SIZE", bench.HEADLINE_KERNEL) == [10.0, 12.0, 99.0]
    assert bench._counter_rows(p, "FETCH_SIZE", bench.HEADLINE_KERNEL, before=bench.COPY_KERNEL) == [10.0, 12.0]
    assert bench._counter_rows(p, "WRITE_SIZE", bench.HEADLINE_KERNEL) == []


def test_traffic_summary_calibrates_each_counter_by_the_copy_kernel(tmp_path, monkeypatch):
    # the copy moves MIN_BYTES / 2 each way; suppose its counters read half of that (FETCH) and
    # all of it (WRITE), as on MI355X. A headline launch that reads 1 % more than its bytes and
    # writes them exactly must come out as 1.01 x and 1.00 x of MIN_BYTES / 2.
    each_kib = bench.MIN_BYTES / 2 / 1024
    fetch, write = tmp_path / "fetch.csv", tmp_path / "write.csv"
    _write_counters(fetch, "FETCH_SIZE", [(HEAD, 0.505 * each_kib), (HEAD, 0.505 * each_kib),
                                          (COPY, 0.5 * each_kib), (COPY, 0.001 * each_kib),
                                          (HEAD, 0.9 * each_kib)])
    _write_counters(write, "WRITE_SIZE", [(HEAD, each_kib), (HEAD, each_kib), (COPY, each_kib),
                                          (COPY, 0.002 * each_kib), (HEAD, 0.9 * each_kib)])
    out = tmp_path / "traffic.json"
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(out))
    assert bench.traffic_summary(str(fetch), str(write)) == 0
    t = json.loads(out.read_text())
    # the small copy dispatches (other workloads' cold copies) and the headline kernel's later
    # launches (after the copy kernel's first) are left out
    assert t["fetch_scale"] == pytest.approx(2.0, rel=1e-6)
    assert t["write_scale"] == pytest.approx(1.0, rel=1e-6)
    assert t["hbm_read_bytes_per_launch"] == pytest.approx(1.01 * bench.MIN_BYTES / 2, rel=1e-6)
    assert t["hbm_write_bytes_per_launch"] == pytest.approx(bench.MIN_BYTES / 2, rel=1e-6)
    assert t["traffic_over_algorithmic"] == pytest.approx(1.005, abs=1e-5)
    assert t["kernel_source_sha256"] == bench.kernel_source_hash()


def test_committed_traffic_is_dropped_when_the_kernel_source_changes(tmp_path, monkeypatch):
    p = tmp_path / "traffic.json"
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(p))
    assert bench.committed_traffic()[0] is None  # no file
    p.write_text(json.dumps({"kernel_source_sha256": bench.kernel_source_hash(),
                             "hbm_bytes_per_launch": 123}))
    assert bench.committed_traffic()[0] == 123
    p.write_text(json.dumps({"kernel_source_sha256": "0" * 64, "hbm_bytes_per_launch": 123}))
    value, note = bench.committed_traffic()
    assert value is None and "changed" in note


def test_committed_traffic_summary_matches_the_current_kernel_source():
    # the summary in profiles/ must describe the headline kernel as built now, or the bench line
    # reports no traffic
    with open(os.path.join(ROOT, "profiles", "inorm_pipelined_112x64x512x512_traffic.json")) as f:
        t = json.load(f)
    assert t["kernel_source_sha256"] == bench.kernel_source_hash()
    assert 1.0 <= t["traffic_over_algorithmic"] < 1.01
