"""bench.py's output contract on an MI355X (run with -m gpu): a short run prints one JSON line
whose fields are consistent with one another -- value from ms_per_step and the minimum bytes,
roofline.frac from roofline.achieved and the 8 TB/s peak, the CPU baseline from the oracle with
its sample's parity within the 1e-4 gate."""
import json
import os
import subprocess
import sys

import pytest

pytestmark = pytest.mark.gpu
ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
MIN_BYTES = 2 * 4 * 112 * 64 * 512 * 512


def test_bench_prints_one_consistent_json_line():
    print("case bench.py --steps 3 --warmup 1 --no-extra --cpu-seconds 2", flush=True)
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--steps", "3", "--warmup", "1",
                        "--no-extra", "--cpu-seconds", "2"],
                       capture_output=True, text=True, timeout=600, cwd=ROOT)
    assert r.returncode == 0, r.stderr[-2000:]
    lines = [l for l in r.stdout.splitlines() if l.strip()]
    assert len(lines) == 1, r.stdout
    d = json.loads(lines[0])
    for key in ("metric", "value", "unit", "n_gpus", "steps", "warmup", "ms_per_step", "higher_is_better",
                "scaling", "vs_baseline", "dtype", "data", "config", "roofline", "cpu_baseline"):
        assert key in d, key
    assert d["n_gpus"] == 1 and d["steps"] == 3 and d["warmup"] == 1
    assert d["unit"] == "GB/s" and d["higher_is_better"] is True and d["dtype"] == "f32"
    assert d["vs_baseline"] is None
    assert d["config"]["min_bytes_per_step"] == MIN_BYTES and "workload" in d["config"]
    assert d["value"] == pytest.approx(MIN_BYTES / (d["ms_per_step"] / 1e3) / 1e9, rel=1e-3)
    rf = d["roofline"]
    assert rf["bound"] == "hbm" and rf["unit"] == "GB/s" and rf["peak"] == 8000.0
    assert rf["frac"] == pytest.approx(rf["achieved"] / rf["peak"], abs=1e-4)
    assert rf["traffic"] is None or rf["traffic"] >= MIN_BYTES
    assert 1000.0 < rf["achieved"] < rf["peak"]
    cb = d["cpu_baseline"]
    assert cb["kind"] == "oracle" and cb["unit"] == "GB/s" and cb["cores"] >= 1 and cb["value"] > 0
    assert d["parity_sample"]["max_abs_err"] <= 1e-4
    print("bench line: value %.1f GB/s, frac %.4f, oracle %.1f GB/s on %d cores"
          % (d["value"], rf["frac"], cb["value"], cb["cores"]), flush=True)
