"""bench.py's output line: one JSON object whose headline figures agree with
each other (value = layers x bytes per layer / step time, the dominant
kernel's launch time = step time / launches) and that carries the roofline
and the per-call figures.  A short run (64 layers, few steps, the other
configurations and legs off) in a child process."""
import json
import os
import subprocess
import sys

import pytest

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_bench_json_line_is_consistent():
    cmd = [sys.executable, os.path.join(ROOT, "bench.py"), "--steps", "3", "--warmup", "1",
           "--layers", "64", "--no-cpu", "--no-configs", "--no-legs"]
    out = subprocess.run(cmd, cwd=ROOT, capture_output=True, text=True, timeout=110)
    assert out.returncode == 0, out.stderr[-2000:]
    lines = [ln for ln in out.stdout.splitlines() if ln.strip()]
    assert len(lines) == 1, out.stdout[-2000:]
    d = json.loads(lines[0])
    for key in ("metric", "value", "unit", "n_gpus", "steps", "warmup", "ms_per_step",
                "higher_is_better", "scaling", "vs_baseline", "dtype", "data", "config",
                "roofline", "fused_per_call", "cpu_baseline"):
        assert key in d, key
    assert d["n_gpus"] == 1 and d["steps"] == 3 and d["warmup"] == 1
    cfg = d["config"]
    assert cfg["layers_per_step"] == 64 and cfg["launches_per_step"] == 2
    implied = d["value"] * 1e9 * d["ms_per_step"] * 1e-3 / cfg["bytes_per_layer"]
    assert abs(implied - cfg["layers_per_step"]) < 0.01 * cfg["layers_per_step"]
    roof = d["roofline"]
    for key in ("bound", "achieved", "peak", "unit", "frac", "traffic"):
        assert key in roof, key
    assert abs(roof["frac"] - roof["achieved"] / roof["peak"]) < 1e-3
    assert abs(roof["us_per_launch"] * cfg["launches_per_step"] - d["ms_per_step"] * 1e3) \
        < 0.01 * d["ms_per_step"] * 1e3
    fused = d["fused_per_call"]
    assert fused["instances"] == 64 and "rotate_in_deq_gemv_2bit" in fused["kernels"]
