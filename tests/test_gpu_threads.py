"""Host threads calling the library at once, each on its own stream.

A fresh process (so the per-device launch settings start unset) starts four
threads that wait on a barrier and then run the Linear forward and backward
and the MoE expert forward through the library, each on its own stream with
its own inputs; every output must equal, bit for bit, the same work run
afterwards on one thread.  Errors are per thread: a fifth thread makes calls
that the C library rejects, and sees its own message each time, while the
others' calls succeed."""
import os
import subprocess
import sys

import pytest

pytestmark = pytest.mark.gpu
ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

SCRIPT = r"""
import sys, threading
sys.path.insert(0, sys.argv[1])
import numpy as np, torch
import fine_grained_blockwise_amd as fgb
dev = "cuda:0"
NT, T, CIN, COUT, G, TOPK, F = 4, 512, 512, 256, 6, 2, 128

def inputs(i):
    g = torch.Generator().manual_seed(100 + i)
    r = lambda *s, sc=1.0: (torch.randn(*s, generator=g) * sc).to(torch.bfloat16).to(dev)
    idx = torch.stack([torch.randperm(G, generator=g)[:TOPK] for _ in range(T)]).to(torch.int32).to(dev)
    return dict(x=r(T, CIN), w=r(COUT, CIN, sc=0.05), dy=r(T, COUT, sc=1e-3), w1=r(G * 2 * F, CIN, sc=0.05),
                w2=r(G * CIN, F, sc=0.05), idx=idx, probs=torch.rand(T, TOPK, generator=g).to(dev))

def step(I):
    xq, xs = fgb.fp8_quant_rowwise(I["x"])
    wq, ws = fgb.fp8_quant_blockwise(I["w"])
    gq, gs = fgb.fp8_quant_rowwise(I["dy"])
    y = fgb.fp8_block_gemm(xq, xs, fgb.ROW1x128, wq, ws, fgb.BLOCK128)
    wqt, wst = fgb.fp8_direct_transpose(wq, ws, fgb.BLOCK128)
    dx = fgb.fp8_block_gemm(gq, gs, fgb.ROW1x128, wqt, wst, fgb.BLOCK128)
    xqt, xst = fgb.fp8_direct_transpose(xq, xs)
    gqt, gst = fgb.fp8_direct_transpose(gq, gs)
    dw = fgb.fp8_block_gemm(gqt, gst, fgb.ROW1x128, xqt, xst, fgb.ROW1x128, out_dtype=torch.float32)
    w1q, w1s = fgb.fp8_quant_blockwise(I["w1"])
    w2q, w2s = fgb.fp8_quant_blockwise(I["w2"])
    pq, ps, rmap, offs = fgb.permute_pad(xq, xs, I["idx"], G, 16)
    h = fgb.fp8_grouped_gemm(pq, ps, w1q.view(G, 2 * F, CIN), w1s.view(G, 2 * F // 128, CIN // 128), offs)
    aq, as_ = fgb.swiglu_quant(h, offs)
    o = fgb.fp8_grouped_gemm(aq, as_, w2q.view(G, CIN, F), w2s.view(G, CIN // 128, F // 128), offs)
    out = fgb.unpermute_unpad(o, rmap, I["probs"])
    return [y, dx, dw, offs, rmap, out]

def host(ts):
    return [t.cpu().view(torch.int16) if t.dtype == torch.bfloat16 else t.cpu() for t in ts]

ins = [inputs(i) for i in range(NT)]
torch.cuda.synchronize()
barrier = threading.Barrier(NT + 1)
got, errs, fails = [None] * NT, [None] * (NT + 1), []

def work(i):
    try:
        s = torch.cuda.Stream()
        with torch.cuda.stream(s):
            barrier.wait()
            r = step(ins[i])
        s.synchronize()
        got[i] = host(r)
    except BaseException as e:
        fails.append((i, repr(e)))

a0 = torch.zeros((128, 128), dtype=torch.uint8, device=dev)
s0 = torch.full((128, 1), 127, dtype=torch.uint8, device=dev)
sb0 = torch.full((1, 1), 127, dtype=torch.uint8, device=dev)

def bad():  # calls the C library rejects, on their own thread: each error message is this thread's
    barrier.wait()
    for _ in range(50):
        try:
            fgb.fp8_block_gemm_fmt(a0, s0, fgb.ROW1x128, 7, a0, sb0, fgb.BLOCK128)  # no element format 7
        except fgb.FgbError as e:
            if "a_fmt must be" not in str(e):
                fails.append(("bad", str(e)))
            errs[NT] = str(e)
        else:
            fails.append(("bad", "the call with a_fmt = 7 was accepted"))

threads = [threading.Thread(target=work, args=(i,)) for i in range(NT)] + [threading.Thread(target=bad)]
for t in threads:
    t.start()
for t in threads:
    t.join()
assert not fails, fails
assert errs[NT] is not None, "the rejected call did not raise"
for i in range(NT):
    want = host(step(ins[i]))
    torch.cuda.synchronize()
    assert len(want) == len(got[i])
    for k, (a, b) in enumerate(zip(got[i], want)):
        assert a.shape == b.shape and torch.equal(a, b), (i, k)
print("threads ok:", NT, "concurrent streams matched the sequential run; rejected call:", errs[NT][:60], flush=True)
"""


def test_concurrent_threads_and_streams():
    print("library called from four threads at once, first use in a fresh process", flush=True)
    r = subprocess.run([sys.executable, "-u", "-c", SCRIPT, ROOT], capture_output=True, text=True, timeout=240)
    assert r.returncode == 0, (r.stdout[-2000:], r.stderr[-3000:])
    assert "threads ok: 4" in r.stdout, r.stdout[-2000:]
