"""bench.py prints one JSON line with the fields its consumers read (run on the
tiny workload, so the check takes seconds)."""
import json
import os
import subprocess
import sys

import pytest

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_bench_json_line_fields():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--workload", "1", "--steps", "3",
                        "--warmup", "1", "--no-extra", "--no-cpu-baseline"],
                       capture_output=True, text=True, timeout=110, cwd=ROOT)
    assert r.returncode == 0, r.stderr[-2000:]
    lines = [ln for ln in r.stdout.splitlines() if ln.strip()]
    assert len(lines) == 1
    d = json.loads(lines[0])
    for key in ("metric", "value", "unit", "n_gpus", "steps", "warmup", "ms_per_step", "higher_is_better",
                "scaling", "vs_baseline", "dtype", "data", "config", "roofline"):
        assert key in d, key
    assert d["n_gpus"] == 1 and d["steps"] == 3 and d["warmup"] == 1
    assert d["unit"] == "TB/s" and d["higher_is_better"] is True and d["value"] > 0
    assert d["config"]["workload"] == "tiny decode"
    roof = d["roofline"]
    for key in ("bound", "achieved", "peak", "unit", "frac", "traffic"):
        assert key in roof, key
    assert roof["bound"] == "hbm" and roof["peak"] == 8000.0
    assert abs(roof["frac"] - roof["achieved"] / roof["peak"]) < 1e-3
    assert d["config"]["step_path"]
    pct = d["ms_per_step_percentiles"]
    assert pct["p10"] <= pct["p50"] <= pct["p90"]


def test_bench_prefill_roofline_object():
    """The mixed chunked-prefill workload carries a prefill roofline against the
    dense bf16 MFMA peak."""
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--workload", "4", "--steps", "2",
                        "--warmup", "1", "--no-extra", "--no-cpu-baseline"],
                       capture_output=True, text=True, timeout=110, cwd=ROOT)
    assert r.returncode == 0, r.stderr[-2000:]
    d = json.loads(r.stdout.strip().splitlines()[-1])
    pr = d["prefill_roofline"]
    assert pr["bound"] == "mfma" and pr["peak"] == 2500.0 and pr["unit"] == "TFLOP/s"
    assert 0 < pr["frac"] < 1 and abs(pr["frac"] - pr["achieved"] / pr["peak"]) < 1e-3
    assert pr["flops_per_launch"] == 77_342_965_760


def test_bench_refuses_more_than_one_gpu():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=60, cwd=ROOT)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
