"""The benchmark's JSON line, from a short run of bench.py in its own process
(as it is run for the record): every field the line promises, and its headline
numbers consistent with each other."""
import json
import os
import subprocess
import sys

import pytest

import workloads as W
from parity import announce

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_bench_line_contract():
    announce("bench.py --steps 3 --warmup 1 --no-cpu-baseline --no-secondary")
    r = subprocess.run([sys.executable, "-u", "bench.py", "--steps", "3", "--warmup", "1", "--no-cpu-baseline",
                        "--no-secondary"], cwd=ROOT, capture_output=True, text=True, timeout=110)
    assert r.returncode == 0, r.stderr[-2000:]
    lines = [l for l in r.stdout.splitlines() if l.startswith("{")]
    assert len(lines) == 1, r.stdout[-2000:]
    b = json.loads(lines[0])
    for key in ("metric", "value", "unit", "n_gpus", "steps", "warmup", "ms_per_step", "higher_is_better", "scaling",
                "vs_baseline", "dtype", "data", "config", "roofline", "cpu_baseline"):
        assert key in b, key
    assert b["n_gpus"] == 1 and b["steps"] == 3 and b["warmup"] == 1
    assert b["higher_is_better"] is True and b["dtype"] == "bf16" and b["unit"] == "TFLOP/s"
    assert b["cpu_baseline"] is None
    wl = W.packed_16k()
    assert b["config"]["workload"] == wl.name
    # value is the accounted forward+backward work (3.5 forward flops) over ms_per_step
    assert b["ms_per_step"] > 0
    assert b["value"] == pytest.approx(3.5 * wl.accounted_fwd_flop() / (b["ms_per_step"] * 1e-3) / 1e12, rel=1e-9)
    rf = b["roofline"]
    for key in ("bound", "achieved", "peak", "unit", "frac", "traffic"):
        assert key in rf, key
    assert rf["bound"] == "mfma" and rf["unit"] == "TFLOP/s" and rf["peak"] == 2500.0
    assert rf["frac"] == pytest.approx(rf["achieved"] / rf["peak"], rel=1e-9)
    assert 0 < rf["frac"] < 1
    # the dominant kernel's figure is its algorithmic flops over its measured launch time
    assert rf["achieved"] == pytest.approx(rf["flop_per_launch"] / (rf["avg_ms"] * 1e-3) / 1e12, rel=1e-9)
