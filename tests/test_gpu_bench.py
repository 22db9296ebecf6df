"""bench.py's JSON line on the GPU: one step of the dense Linear part, every
field the line promises, with consistent values."""
import json
import os
import subprocess
import sys

import pytest

pytestmark = pytest.mark.gpu
ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_bench_line_contract():
    print("bench: linear part, one step after one warmup", flush=True)
    r = subprocess.run([sys.executable, "-u", os.path.join(ROOT, "bench.py"), "--parts", "linear", "--steps", "1",
                        "--warmup", "1", "--no-cpu-baseline", "--no-study"],
                       capture_output=True, text=True, timeout=240)
    assert r.returncode == 0, r.stderr[-2000:]
    line = json.loads(r.stdout.strip().splitlines()[-1])
    for k in ("metric", "value", "unit", "n_gpus", "steps", "warmup", "ms_per_step", "higher_is_better", "scaling",
              "vs_baseline", "dtype", "data", "config", "roofline", "cpu_baseline"):
        assert k in line, k
    assert line["n_gpus"] == 1 and line["steps"] == 1 and line["warmup"] == 1
    assert 0 < line["value"] < 100 and line["ms_per_step"] > 0 and line["higher_is_better"] is True
    assert line["vs_baseline"] is None and line["cpu_baseline"] is None
    assert "workload" in line["config"]
    rf = line["roofline"]
    for k in ("bound", "achieved", "peak", "unit", "frac", "traffic"):
        assert k in rf, k
    assert rf["bound"] in ("hbm", "mfma", "alu")
    assert abs(rf["frac"] - rf["achieved"] / rf["peak"]) < 1e-3
    assert len(line["kernels"]) == 9  # the Linear forward and backward: 3 quant, 2 transposes, W^T, 3 GEMMs
