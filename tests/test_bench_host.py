"""Host-side checks of bench.py: the one-GPU refusal, and that every operation
the timed step records is priced by one of the oracle's sampled rates."""
import json
import os
import re
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)


def test_bench_refuses_more_than_one_gpu():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    msg = json.loads(r.stdout.strip().splitlines()[-1])
    assert "one GPU" in msg["error"]


def test_every_step_operation_has_an_oracle_rate():
    import bench

    src = open(os.path.join(ROOT, "bench.py")).read()
    names = set(re.findall(r'rec\("((?:lin|moe|moe_bwd|wgrad|moss)\.[^"]+)"', src))
    assert len(names) >= 30
    rate_keys = {"gemm", "transpose", "quant_blockwise", "quant_rowwise", "permute", "unpermute_bwd", "unpermute",
                 "dswiglu", "swiglu", "mx2"}
    for n in names:
        assert bench.oracle_family(n) in rate_keys, n
    assert bench.oracle_family("moe.quant_blockwise+transpose W1") == "quant_blockwise"
    assert bench.oracle_family("moe_bwd.unpermute_backward_quant dO") == "unpermute_bwd"
    assert bench.oracle_family("moe_bwd.dswiglu_quant") == "dswiglu"
    assert bench.oracle_family("lin.transpose W (block)") == "transpose"


def test_graph_leg_compares_every_step_output():
    """The graph leg compares the replayed step's outputs with the eager step's:
    every tensor the step returns, in a fixed order, and none of the
    observability tensors (kept under "obs")."""
    import bench

    out = {"lin": ("y", "dx", "dw"), "moe": ("o", "offs"), "moe_bwd": ("dx", "dw1", "dw2"), "wg": "dw",
           "moss": ("xh", "y", "wh"), "obs": {"lin": {"xq": "not compared"}}}
    got = list(bench._tensors(out))
    assert got == ["y", "dx", "dw", "o", "offs", "dx", "dw1", "dw2", "xh", "y", "wh", "dw"]
    assert "not compared" not in got
    assert list(bench._tensors({"lin": ("a", None, "b")})) == ["a", "b"]
