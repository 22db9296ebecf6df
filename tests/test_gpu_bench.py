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
    g = line["graph"]  # the step replayed as one HIP graph equals the eager step bit for bit
    assert g["outputs_match_eager"] is True and g["ms_per_step"] > 0 and g["outputs_compared"] == 3
    rf = line["roofline"]
    for k in ("bound", "achieved", "peak", "unit", "frac", "traffic"):
        assert k in rf, k
    assert rf["bound"] in ("hbm", "mfma", "alu")
    assert abs(rf["frac"] - rf["achieved"] / rf["peak"]) < 1e-3
    if rf["bound"] == "mfma":
        assert abs(rf["frac_of_fp8_peak"] - rf["achieved"] / 5000.0) < 1e-3
    assert len(line["kernels"]) == 9  # the Linear forward and backward: 3 quant, 2 transposes, W^T, 3 GEMMs
    # every GEMM is priced at the dense FP8 peak in `value`; the mode's own instruction peak beside it
    assert line["value_at_contraction_peak"] >= line["value"] > 0
    for name, k in line["kernels"].items():
        if k["unit"] == "TFLOP/s":
            assert abs(k["frac_of_fp8_peak"] - k["achieved"] / 5000.0) < 1e-3, name
    hist = line["scale_exponent_histograms"]
    assert set(hist) >= {"lin.X 1x128", "lin.W 128x128", "lin.dY 1x128"}
    for h in hist.values():
        assert h["min_e"] <= h["max_e"] and sum(h["counts"].values()) > 0
    assert sum(hist["lin.X 1x128"]["counts"].values()) == 8192 * 7168 // 128
    und = line["transpose_underflow"]
    assert set(und) == {"lin.direct_transpose Xq", "lin.direct_transpose dYq"}
    for u in und.values():
        assert 0 <= u["became_zero"] <= u["nonzero_in"]


def test_bench_output_check_against_the_oracle():
    print("bench: linear part with the CPU-baseline leg and its output check", flush=True)
    r = subprocess.run([sys.executable, "-u", os.path.join(ROOT, "bench.py"), "--parts", "linear", "--steps", "1",
                        "--warmup", "1", "--no-study"],
                       capture_output=True, text=True, timeout=600)
    assert r.returncode == 0, r.stderr[-2000:]
    line = json.loads(r.stdout.strip().splitlines()[-1])
    chk = line["cpu_baseline"]["output_check"]
    for name in ("lin.gemm fprop", "lin.gemm dgrad", "lin.gemm wgrad"):
        c = chk[name]
        assert c["within_tolerance"] and c["beyond_one_bf16_ulp"] == 0, (name, c)
        assert 0 <= c["calc_diff"] < 1e-4, (name, c)
