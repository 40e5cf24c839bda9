"""bench.py prints one JSON line with the fields its readers rely on: the
metric and its value, the step timing, the configuration, the roofline of the
token-sparse kernel and the oracle's CPU baseline.  Run on the small tiny
workload, in a child process."""
import json
import os
import subprocess
import sys

import pytest

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_bench_prints_one_json_line_with_the_contract_fields():
    print("[bench contract] tiny workload, 2 steps", flush=True)
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--workload", "tiny", "--steps", "2",
                        "--warmup", "1", "--cpu-sample-rows", "256", "--cpu-sample-groups", "4"],
                       cwd=ROOT, capture_output=True, text=True, timeout=240)
    assert r.returncode == 0, r.stderr[-2000:]
    lines = [l for l in r.stdout.splitlines() if l.strip()]
    assert len(lines) == 1, r.stdout[-2000:]
    b = json.loads(lines[0])
    for key in ("metric", "value", "unit", "n_gpus", "steps", "warmup", "ms_per_step", "higher_is_better",
                "scaling", "vs_baseline", "dtype", "data", "config", "roofline", "cpu_baseline"):
        assert key in b, key
    assert b["n_gpus"] == 1 and b["steps"] == 2 and b["warmup"] == 1
    assert b["value"] > 0 and b["ms_per_step"] > 0 and b["higher_is_better"] is True
    assert b["dtype"] == "bf16" and b["data"] == "synthetic" and b["config"]["workload"].startswith("tiny")
    rl = b["roofline"]
    assert rl["bound"] == "mfma" and rl["unit"] == "TFLOP/s" and rl["peak"] == 2500.0
    assert rl["frac"] == pytest.approx(rl["achieved"] / rl["peak"], abs=1e-4)   # printed to 4 places
    assert "traffic" in rl
    cb = b["cpu_baseline"]
    assert cb["kind"] == "oracle" and cb["value"] > 0 and cb["cores"] >= 1
    assert cb["unit"] and cb["sample"]
