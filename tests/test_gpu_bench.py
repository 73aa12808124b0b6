"""bench.py end to end on the GPU, briefly: the one JSON line it prints
keeps its contract (the fields the benchmark's consumers read, a positive
rate that agrees with its own step time, the roofline of the dominant
kernel and the oracle's CPU baseline)."""
import json
import os
import subprocess
import sys

import pytest

from gpu_util import require_gpu

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_bench_prints_one_line_with_its_contract():
    require_gpu()
    print("bench.py --steps 4 --warmup 2 --no-ceilings --no-bf16-baseline --cpu-budget-s 2", flush=True)
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--steps", "4", "--warmup", "2",
                        "--no-ceilings", "--no-bf16-baseline", "--cpu-budget-s", "2"],
                       capture_output=True, text=True, timeout=170)
    assert r.returncode == 0, r.stderr[-2000:]
    lines = [ln for ln in r.stdout.splitlines() if ln.startswith("{")]
    assert len(lines) == 1, r.stdout[-2000:]
    d = json.loads(lines[0])
    for k in ("metric", "value", "unit", "n_gpus", "steps", "warmup", "ms_per_step", "higher_is_better", "scaling",
              "vs_baseline", "dtype", "data", "config", "roofline", "cpu_baseline"):
        assert k in d, k
    assert d["n_gpus"] == 1 and d["steps"] == 4 and d["warmup"] == 2 and d["unit"] == "TFLOP/s"
    assert d["config"]["workload"] and d["config"]["tokens"] == 8192
    step_flop = d["config"]["gemm_tflop_per_step"] * 1e12
    assert d["value"] > 0 and abs(d["value"] - step_flop / (d["ms_per_step"] * 1e-3) / 1e12) <= 0.01 * d["value"]
    roof = d["roofline"]
    for k in ("bound", "achieved", "peak", "unit", "frac", "traffic"):
        assert k in roof, k
    assert roof["bound"] == "mfma" and roof["peak"] == 5000.0 and 0 < roof["frac"] < 1
    assert abs(roof["frac"] - roof["achieved"] / roof["peak"]) < 1e-3
    cb = d["cpu_baseline"]
    assert cb["kind"] == "oracle" and cb["cores"] >= 1 and cb["value"] > 0 and cb["sample"]
