#!/usr/bin/env python3
"""Benchmark of the fine-grained blockwise FP8 hot path on one MI355X.

One step is one pass of every hot-path operation over one batch of seeded
synthetic input, already resident in HBM:
  linear  DeepSeek-V3-shaped Linear, T=8192, Cin=7168, Cout=2048 (bf16 in):
          1x128 quant of X and dY, 128x128 quant of W, block transpose of W,
          direct transposes of Xq and dYq, Fprop / Dgrad / Wgrad (bf16 out)
  moe     one GPU's 32 local experts, 16384 tokens x 7168, top-8: quant of X,
          128x128 quant of W1 [32x4096x7168] and W2 [32x7168x2048],
          permute+pad-16, grouped fc1, SwiGLU+quant, grouped fc2,
          unpermute+unpad
  wgrad   direct transposes of row-wise codes [32768, 7168] and [32768, 2048]
          (scales 2^-20..2^4) and the Wgrad GEMM over K=32768 (fp32 out)
  moss    two-level microscaling of W^T [28672, 8192] (quant + dequant),
          1x32 quant of A [4096, 8192], MX-scaled GEMM (fp32 out)

Reported value: the step's roofline efficiency in percent -- the sum over the
step's kernels of their roofline floor time (algorithmic bytes at 8 TB/s HBM
for the data-movement kernels, flops at the dense FP8 matrix peak of 5.0
PFLOP/s for every GEMM, whichever arithmetic mode computes it) divided by the
measured step time.  Beside it, value_at_contraction_peak prices each GEMM at
the peak of the matrix instruction the mode actually issues (bf16 2.5 PFLOP/s
in the exact mode, whose bf16 contraction caps it at half the FP8 peak).
Per-kernel figures come from HIP events recorded on the launch stream around
every kernel of the timed steps.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--gemm-mode exact|fast]
"""
import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
FP8_PEAK_TFLOPS = 5000.0  # dense FP8 matrix peak: the price of every GEMM in `value`
MFMA_PEAK_TFLOPS = {"exact": 2500.0, "fast": 5000.0}  # peak of the instruction each mode issues: bf16 / fp8


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--gemm-mode", choices=["exact", "fast"], default="exact")
    ap.add_argument("--parts", default="linear,moe,moe_bwd,wgrad,moss")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-study", action="store_true", help="skip the untimed transpose comparison")
    ap.add_argument("--no-graph", action="store_true",
                    help="skip the HIP-graph leg (the step captured once and replayed --steps times)")
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a plain 1 GiB read + 1 GiB write elementwise kernel 3 times (the reference "
                         "point for scaling HBM byte counters), then exit")
    ap.add_argument("--vendor-gemm", action="store_true",
                    help="only time this library's blockwise GEMM (both modes) beside the vendor library's plain "
                         "bf16 GEMM and row-wise-scaled FP8 GEMM (torch.matmul, torch._scaled_mm) at three shapes "
                         "of the step, then exit: context for the GEMM rates, not part of the path")
    return ap.parse_args()


class Recorder:
    """HIP events around each kernel on torch's current stream (the launch stream)."""

    def __init__(self, torch):
        self.torch = torch
        self.on = False
        self.ev = {}
        self.meta = {}

    def __call__(self, name, kind, work, fn, *a, **kw):
        if not self.on:
            return fn(*a, **kw)
        t = self.torch
        e0 = t.cuda.Event(enable_timing=True)
        e1 = t.cuda.Event(enable_timing=True)
        e0.record()
        out = fn(*a, **kw)
        e1.record()
        self.ev.setdefault(name, []).append((e0, e1))
        self.meta[name] = (kind, work)
        return out

    def results(self):
        res = {}
        for name, lst in self.ev.items():
            ms = sum(a.elapsed_time(b) for a, b in lst) / len(lst)
            res[name] = (ms,) + self.meta[name]
        return res


def build(fgb, torch, synth, dev, seed, parts):
    """All inputs and weights, resident on the GPU (untimed)."""
    W = {}
    if "linear" in parts:
        X, Wl, dY = synth.linear_dsv3(seed, device=dev)
        W["lin"] = dict(X=X, W=Wl, dY=dY)
    if "moe" in parts:
        X, idx, probs, W1, W2 = synth.moe(seed, device=dev)
        T, topk, G, H = X.shape[0], idx.shape[1], 32, X.shape[1]
        M_cap = T * topk + 15 * G
        W["moe"] = dict(X=X, idx=torch.from_numpy(idx).to(dev), probs=torch.from_numpy(probs).to(dev),
                        W1=W1.reshape(-1, H), W2=W2.reshape(-1, W2.shape[2]), G=G, M_cap=M_cap,
                        F=W1.shape[1] // 2, N1=W1.shape[1], N2=W2.shape[1],
                        ws=torch.empty(fgb.permute_pad_workspace_size(T, topk, G), dtype=torch.uint8,
                                       device=dev),
                        counts=torch.from_numpy(__import__("numpy").bincount(idx.ravel(), minlength=G)))
    if "moe_bwd" in parts:
        if "moe" not in W:
            raise SystemExit("--parts: moe_bwd needs moe (the backward reads the forward's tensors)")
        E = W["moe"]
        E["dO"] = synth.moe_grad(seed, device=dev)
        E["ws_bwd"] = torch.empty(fgb.unpermute_backward_workspace_size(E["M_cap"]), dtype=torch.uint8, device=dev)
    if "wgrad" in parts:
        xq, xs = synth.wgrad_codes(32768, 7168, seed, 41, device=dev)
        gq, gs = synth.wgrad_codes(32768, 2048, seed, 42, device=dev)
        W["wg"] = dict(xq=xq, xs=xs, gq=gq, gs=gs)
    if "moss" in parts:
        Wm, A = synth.moss(seed, device=dev)
        W["moss"] = dict(W=Wm, Wt=Wm.t().contiguous(), A=A)
    torch.cuda.synchronize()
    return W


def step(fgb, torch, W, rec, mode):
    gm = fgb.GEMM_EXACT if mode == "exact" else fgb.GEMM_FAST
    out = {}
    if "lin" in W:
        L = W["lin"]
        T, Cin = L["X"].shape
        Cout = L["W"].shape[0]
        xq, xs = rec("lin.quant_rowwise X", "hbm", T * Cin * 3 + T * Cin // 128, fgb.fp8_quant_rowwise, L["X"])
        wq, ws = rec("lin.quant_blockwise W", "hbm", Cout * Cin * 3 + (Cout * Cin) // 16384,
                     fgb.fp8_quant_blockwise, L["W"])
        gq, gs = rec("lin.quant_rowwise dY", "hbm", T * Cout * 3 + T * Cout // 128, fgb.fp8_quant_rowwise, L["dY"])
        y = rec("lin.gemm fprop", "mfma", 2 * T * Cout * Cin, fgb.fp8_block_gemm, xq, xs, fgb.ROW1x128, wq, ws,
                fgb.BLOCK128, mode=gm)
        wqt, wst = rec("lin.transpose W (block)", "hbm", 2 * Cout * Cin + 2 * (Cout * Cin) // 16384,
                       fgb.fp8_direct_transpose, wq, ws, fgb.BLOCK128)
        dx = rec("lin.gemm dgrad", "mfma", 2 * T * Cin * Cout, fgb.fp8_block_gemm, gq, gs, fgb.ROW1x128, wqt, wst,
                 fgb.BLOCK128, mode=gm)
        xqt, xst = rec("lin.direct_transpose Xq", "hbm", 2 * (T * Cin + T * Cin // 128), fgb.fp8_direct_transpose,
                       xq, xs)
        gqt, gst = rec("lin.direct_transpose dYq", "hbm", 2 * (T * Cout + T * Cout // 128),
                       fgb.fp8_direct_transpose, gq, gs)
        dw = rec("lin.gemm wgrad", "mfma", 2 * Cout * Cin * T, fgb.fp8_block_gemm, gqt, gst, fgb.ROW1x128, xqt, xst,
                 fgb.ROW1x128, mode=gm)
        out["lin"] = (y, dx, dw)
        out["obs"] = {"lin": dict(xq=xq, xs=xs, wq=wq, ws=ws, gq=gq, gs=gs, xqt=xqt, xst=xst, gqt=gqt, gst=gst)}
    if "moe" in W:
        E = W["moe"]
        T, H = E["X"].shape
        topk = E["idx"].shape[1]
        G, M_cap, F, N1, N2 = E["G"], E["M_cap"], E["F"], E["N1"], E["N2"]
        rows = int(E["counts"].sum())
        pad_rows = int(((E["counts"] + 15) // 16 * 16).sum())
        xq, xs = rec("moe.quant_rowwise X", "hbm", T * H * 3 + T * H // 128, fgb.fp8_quant_rowwise, E["X"])
        bwd = "dO" in E
        if bwd:  # the expert backward's Dgrad reads W^T: the quantizer writes both copies in one pass
            w1q, w1s, w1t, w1ts = rec("moe.quant_blockwise+transpose W1", "hbm",
                                      E["W1"].numel() * 4 + 2 * (E["W1"].numel() // 16384),
                                      fgb.fp8_quant_blockwise_t, E["W1"].view(G, N1, H))
            w2q, w2s, w2t, w2ts = rec("moe.quant_blockwise+transpose W2", "hbm",
                                      E["W2"].numel() * 4 + 2 * (E["W2"].numel() // 16384),
                                      fgb.fp8_quant_blockwise_t, E["W2"].view(G, N2, F))
        else:
            w1q, w1s = rec("moe.quant_blockwise W1", "hbm", E["W1"].numel() * 3 + E["W1"].numel() // 16384,
                           fgb.fp8_quant_blockwise, E["W1"])
            w2q, w2s = rec("moe.quant_blockwise W2", "hbm", E["W2"].numel() * 3 + E["W2"].numel() // 16384,
                           fgb.fp8_quant_blockwise, E["W2"])
        pq, ps, rmap, offs = rec("moe.permute_pad", "hbm",
                                 T * H * (1 + 1 / 128) + pad_rows * H * (1 + 1 / 128) + 8 * T * topk,
                                 fgb.permute_pad, xq, xs, E["idx"], G, 16, M_cap, E["ws"])
        h = rec("moe.grouped_gemm fc1", "mfma", 2 * rows * N1 * H, fgb.fp8_grouped_gemm, pq, ps,
                w1q.view(G, N1, H), w1s.view(G, N1 // 128, H // 128), offs, mode=gm)
        if bwd:  # the backward recomputes SwiGLU from an FP8 copy of h written by the same pass
            aq, as_, hq, hs = rec("moe.swiglu_quant+cache", "hbm",
                                  pad_rows * (2 * F * 2 + F * (1 + 1 / 128) + 2 * F * (1 + 1 / 128)),
                                  fgb.swiglu_quant_cache, h, offs)
        else:
            aq, as_ = rec("moe.swiglu_quant", "hbm", pad_rows * (2 * F * 2 + F * (1 + 1 / 128)),
                          fgb.swiglu_quant, h, offs)
        y = rec("moe.grouped_gemm fc2", "mfma", 2 * rows * N2 * F, fgb.fp8_grouped_gemm, aq, as_,
                w2q.view(G, N2, F), w2s.view(G, N2 // 128, F // 128), offs, mode=gm)
        o = rec("moe.unpermute_unpad", "hbm", T * topk * H * 2 + T * H * 2 + 8 * T * topk, fgb.unpermute_unpad,
                y, rmap, E["probs"])
        out["moe"] = (o, offs)
        out.setdefault("obs", {})["moe"] = dict(xq=xq, xs=xs, w1s=w1s, w2s=w2s, pq=pq, ps=ps, as_=as_, offs=offs,
                                                h=h, y=y, rmap=rmap)
        if bwd:
            # expert backward: Dgrad and K-grouped Wgrad of both expert linears, all operands FP8
            dyq, dys = rec("moe_bwd.unpermute_backward_quant dO", "hbm",
                           T * H * 2 + M_cap * H * (1 + 1 / 128) + 8 * T * topk,
                           fgb.unpermute_backward_quant, E["dO"], rmap, E["probs"], M_cap, workspace=E["ws_bwd"])
            da = rec("moe_bwd.grouped_gemm fc2 dgrad", "mfma", 2 * rows * F * N2, fgb.fp8_grouped_gemm, dyq, dys,
                     w2t, w2ts, offs, mode=gm)
            dyt, dyts, koff = rec("moe_bwd.grouped_direct_transpose dY", "hbm", 2 * pad_rows * H * (1 + 1 / 128),
                                  fgb.fp8_grouped_direct_transpose, dyq, dys, offs)
            at, ats, _ = rec("moe_bwd.grouped_direct_transpose A", "hbm", 2 * pad_rows * F * (1 + 1 / 128),
                             fgb.fp8_grouped_direct_transpose, aq, as_, offs)
            dw2 = rec("moe_bwd.kgrouped_gemm fc2 wgrad", "mfma", 2 * rows * N2 * F, fgb.fp8_kgrouped_gemm, dyt, dyts,
                      at, ats, koff, mode=gm)
            dhq, dhs = rec("moe_bwd.dswiglu_quant", "hbm", pad_rows * (6 * F + 4 * F / 128), fgb.dswiglu_quant,
                           hq, hs, da, offs)
            dxp = rec("moe_bwd.grouped_gemm fc1 dgrad", "mfma", 2 * rows * H * N1, fgb.fp8_grouped_gemm, dhq, dhs,
                      w1t, w1ts, offs, mode=gm)
            dht, dhts, _ = rec("moe_bwd.grouped_direct_transpose dH", "hbm", 2 * pad_rows * N1 * (1 + 1 / 128),
                               fgb.fp8_grouped_direct_transpose, dhq, dhs, offs)
            xt, xts, _ = rec("moe_bwd.grouped_direct_transpose X", "hbm", 2 * pad_rows * H * (1 + 1 / 128),
                             fgb.fp8_grouped_direct_transpose, pq, ps, offs)
            dw1 = rec("moe_bwd.kgrouped_gemm fc1 wgrad", "mfma", 2 * rows * N1 * H, fgb.fp8_kgrouped_gemm, dht, dhts,
                      xt, xts, koff, mode=gm)
            dx = rec("moe_bwd.unpermute_unpad dX (permute backward)", "hbm",
                     T * topk * H * 2 + T * H * 2 + 4 * T * topk, fgb.unpermute_unpad, dxp, rmap, None)
            out["moe_bwd"] = (dx, dw1, dw2)
            out["obs"]["moe"].update(dys=dys, dhs=dhs, dyq=dyq, dyt=dyt, koff=koff)
    if "wg" in W:
        Wg = W["wg"]
        T, Cin = Wg["xq"].shape
        Cout = Wg["gq"].shape[1]
        xqt, xst = rec("wgrad.direct_transpose X", "hbm", 2 * (T * Cin + T * Cin // 128), fgb.fp8_direct_transpose,
                       Wg["xq"], Wg["xs"])
        gqt, gst = rec("wgrad.direct_transpose dY", "hbm", 2 * (T * Cout + T * Cout // 128),
                       fgb.fp8_direct_transpose, Wg["gq"], Wg["gs"])
        dw = rec("wgrad.gemm K=32768", "mfma", 2 * Cout * Cin * T, fgb.fp8_block_gemm, gqt, gst, fgb.ROW1x128, xqt,
                 xst, fgb.ROW1x128, out_dtype=torch.float32, mode=gm)
        out["wg"] = dw
        out.setdefault("obs", {})["wg"] = dict(xqt=xqt, xst=xst, gqt=gqt, gst=gst)
    if "moss" in W:
        Mo = W["moss"]
        R, Cc = Mo["Wt"].shape
        M = Mo["A"].shape[0]
        g1 = 10240
        # the weight in its own layout [8192, 28672] (three level-1 groups per row: 10240, 10240, 8192)
        Rw, Cw = Mo["W"].shape
        wq2, ws2, ws1 = rec("moss.mx2_quant W", "hbm", Rw * Cw * (3 + 1 / 32) + 4 * Rw * ((Cw + g1 - 1) // g1),
                            fgb.mx2_quant, Mo["W"], g1)
        wh = rec("moss.mx2_dequant W", "hbm", Rw * Cw * (1 + 4 + 1 / 32) + 4 * Rw * ((Cw + g1 - 1) // g1),
                 fgb.mx2_dequant, wq2, ws2, ws1, g1)
        # the GEMM's operand: W^T [28672, 8192], one level-1 group per row (K = 8192 <= 10240)
        q, s2, s1 = rec("moss.mx2_quant W^T", "hbm", R * Cc * (3 + 1 / 32) + 4 * R * ((Cc + g1 - 1) // g1),
                        fgb.mx2_quant, Mo["Wt"], g1)
        xh = rec("moss.mx2_dequant", "hbm", R * Cc * (1 + 4 + 1 / 32) + 4 * R * ((Cc + g1 - 1) // g1),
                 fgb.mx2_dequant, q, s2, s1, g1)
        aq, as_ = rec("moss.quant_rowwise A 1x32", "hbm", M * Cc * 3 + M * Cc // 32, fgb.fp8_quant_rowwise,
                      Mo["A"], 32)
        y = rec("moss.gemm MX", "mfma", 2 * M * R * Cc, fgb.fp8_block_gemm, aq, as_, fgb.ROW1x32, q, s2,
                fgb.ROW1x32, b_l1=s1.view(-1), g1=g1, out_dtype=torch.float32, mode=gm)
        out["moss"] = (xh, y, wh)
        out.setdefault("obs", {})["moss"] = dict(s2=s2, ws2=ws2, aq=aq, as_=as_, q=q, s1=s1)
    return out


def _tensors(x):
    if isinstance(x, dict):
        for k in sorted(x):
            if k != "obs":
                yield from _tensors(x[k])
    elif isinstance(x, (tuple, list)):
        for v in x:
            yield from _tensors(v)
    elif x is not None:
        yield x


def graph_leg(fgb, torch, W, args, eager_out):
    """The same step captured once in a HIP graph and replayed: the step time
    without per-launch host overhead, and whether every output of the replays
    equals the eager step's bit for bit (the inputs do not change)."""
    rec = Recorder(torch)  # off: plain calls
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        gout = step(fgb, torch, W, rec, args.gemm_mode)
    for _ in range(2):
        g.replay()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        g.replay()
    torch.cuda.synchronize()
    ms = (time.perf_counter() - t0) * 1e3 / args.steps
    a, b = list(_tensors(eager_out)), list(_tensors(gout))
    match = len(a) == len(b) and all(x.shape == y.shape and x.dtype == y.dtype and torch.equal(x, y)
                                     for x, y in zip(a, b))
    del g, gout
    torch.cuda.synchronize()
    log(f"graph leg: {ms:.3f} ms/step over {args.steps} replays; outputs match eager: {match}")
    return {"ms_per_step": round(ms, 3), "replays": args.steps, "outputs_compared": len(a),
            "outputs_match_eager": match}


def source_sha(paths):
    h = hashlib.sha256()
    for p in paths:
        h.update(open(os.path.join(ROOT, p), "rb").read())
    return h.hexdigest()[:16]


def traffic_for(kernel_name, mode):
    """HBM bytes per launch (FETCH_SIZE + WRITE_SIZE, copy-calibrated) from
    committed rocprofv3 counter runs, when the kernel's sources and GEMM mode
    are unchanged since; else None."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(path):
        return None
    try:
        rec = json.load(open(path)).get(kernel_name)
        if not rec or rec.get("source_sha") != source_sha(rec["sources"]):
            return None
        if rec.get("gemm_mode", mode) != mode:
            return None
        return rec["traffic_bytes_per_launch"]
    except Exception:
        return None


# Which sampled oracle rate prices each recorded operation of the step (first
# match wins: the fused weight quantizer is a quantizer, not a transpose).
ORACLE_FAMILIES = [("gemm", "gemm"), ("quant_blockwise", "quant_blockwise"), ("quant_rowwise", "quant_rowwise"),
                   ("transpose", "transpose"), ("permute_pad", "permute"), ("unpermute_backward", "unpermute_bwd"),
                   ("unpermute", "unpermute"), ("dswiglu", "dswiglu"), ("swiglu", "swiglu"), ("mx2", "mx2")]


def oracle_family(name):
    for key, fam in ORACLE_FAMILIES:
        if key in name:
            return fam
    return None


INPUT_KEYS = {"lin": ["X", "W", "dY"], "moe": ["X", "idx", "probs", "W1", "W2", "dO"],
              "wg": ["xq", "xs", "gq", "gs"], "moss": ["W", "Wt", "A"]}


def input_digest(torch, W):
    """SHA-256 (first 16 hex digits) of every 64th row of each synthetic input,
    so that two runs can be checked to have timed the same data."""
    out = {}
    for part, keys in INPUT_KEYS.items():
        for k in keys:
            t = W.get(part, {}).get(k)
            if t is None:
                continue
            rows = t.reshape(t.shape[0], -1)[::64].contiguous()
            out[f"{part}.{k}"] = hashlib.sha256(rows.view(torch.uint8).cpu().numpy().tobytes()).hexdigest()[:16]
    return out


def cpu_baseline(torch, synth, seed, kernel_results, step_floor_s, W=None, out=None, mode="exact"):
    """The oracle, as it stands, on a bounded sample of each op; the whole step's
    CPU time is extrapolated from the per-op rates (single thread).  The same
    leg checks sampled GEMM outputs of the timed step against the oracle
    (oracle_output_check)."""
    import numpy as np

    import oracle as O

    import oracle.parallel as OP

    rates = {}  # units of work per second, per op family (one thread)
    rates_all = {}  # the same with the row-parallel oracle on every host core (bit-identical results)
    budget_s = 1.5  # per op family: the sample is repeated until this much CPU time is spent
    n_thr = max(1, min(len(os.sched_getaffinity(0)), 16))

    def timed_rate(work, fn, budget):
        n, t0 = 0, time.perf_counter()
        while True:
            fn()
            n += 1
            dt = time.perf_counter() - t0
            if dt >= budget:
                return n * work / dt

    def rate(key, work, fn, fn_par=None):
        rates[key] = timed_rate(work, fn, budget_s)
        rates_all[key] = timed_rate(work, fn_par or fn, budget_s / 2)

    t_all = time.perf_counter()
    X, Wl, dY = synth.linear_dsv3(seed, T=1024)
    xb = synth.bf16_bits(X)
    rate("quant_rowwise", xb.size * 3, lambda: O.quant_rowwise(xb), lambda: OP.quant_rowwise_par(xb, 128, n_thr))
    xq, xs = O.quant_rowwise(xb)
    wb = synth.bf16_bits(Wl[:1024])
    rate("quant_blockwise", wb.size * 3, lambda: O.quant_blockwise(wb), lambda: OP.quant_blockwise_par(wb, n_thr))
    rate("transpose", 2 * xq.size, lambda: O.direct_transpose(xq, xs), lambda: OP.direct_transpose_par(xq, xs, n_thr))
    wq, ws = O.quant_blockwise(synth.bf16_bits(Wl))
    mi = np.arange(20000) % 1024
    ni = (np.arange(20000) * 7) % 2048
    rate("gemm", 2 * 20000 * 7168, lambda: O.block_gemm_sampled(xq, xs, O.ROW1x128, wq, ws, O.BLOCK128, mi, ni),
         lambda: OP.block_gemm_sampled_par(xq, xs, O.ROW1x128, wq, ws, O.BLOCK128, mi, ni, threads=n_thr))
    Xm, idx, probs, _, _ = synth.moe(seed, T=2048, weights=False)
    xmq, xms = O.quant_rowwise(synth.bf16_bits(Xm))
    pq, ps, rm, off, used = O.permute_pad(xmq, xms, idx, 32, 16)
    rate("permute", xmq.size + used * 7168, lambda: O.permute_pad(xmq, xms, idx, 32, 16))  # not row-parallel
    y = synth.bf16_bits(torch.randn(used, 7168).to(torch.bfloat16))
    rate("unpermute", 2048 * 8 * 7168 * 2, lambda: O.unpermute_unpad(y, rm, probs),
         lambda: OP.unpermute_unpad_par(y, rm, probs, n_thr))
    h = synth.bf16_bits(torch.randn(1024, 4096).to(torch.bfloat16))
    rate("swiglu", h.size * 2 * 1.25, lambda: O.swiglu_quant(h), lambda: OP.swiglu_quant_par(h, n_thr))
    hq, hs = O.quant_rowwise(h, 128)
    da = synth.bf16_bits(torch.randn(1024, 2048).to(torch.bfloat16))
    rate("dswiglu", 1024 * (6 * 2048 + 4 * 2048 / 128), lambda: O.dswiglu_quant(hq, hs, da, None),
         lambda: OP.dswiglu_quant_par(hq, hs, da, n_thr))
    M_cap = 2048 * 8 + 15 * 32
    rate("unpermute_bwd", 2048 * 7168 * 2 + M_cap * 7168 * (1 + 1 / 128),
         lambda: O.quant_rowwise(O.unpermute_backward(y[:2048], rm, probs, M_cap), 128),
         lambda: OP.quant_rowwise_par(O.unpermute_backward(y[:2048], rm, probs, M_cap), 128, n_thr))
    Wm, _ = synth.moss(seed, R=256, C=8192, M=1)
    wmb = synth.bf16_bits(Wm)
    rate("mx2", wmb.size * 3, lambda: O.mx2_quant(wmb, 10240), lambda: OP.mx2_quant_par(wmb, 10240, n_thr))
    sample_s = time.perf_counter() - t_all

    cpu_step_s = cpu_step_all_s = 0.0
    for name, (ms, kind, work) in kernel_results.items():
        f = oracle_family(name)
        cpu_step_s += work / rates[f]
        cpu_step_all_s += work / rates_all[f]
    value = 100.0 * step_floor_s / cpu_step_s
    check = None
    if W is not None and out is not None:
        t_chk = time.perf_counter()
        check = oracle_output_check(torch, synth, W, out, mode, seed)
        check["seconds"] = round(time.perf_counter() - t_chk, 1)
    cpu_model = ""
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                cpu_model = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    return {"value": value, "unit": "% of MI355X roofline (step, extrapolated)", "cores": 1, "kind": "oracle",
            "host_cpu": cpu_model, "host_nproc": os.cpu_count(),
            "step_seconds_extrapolated": cpu_step_s,
            "all_cores": {"value": 100.0 * step_floor_s / cpu_step_all_s, "cores": n_thr,
                          "step_seconds_extrapolated": cpu_step_all_s,
                          "speedup_over_one_core": cpu_step_s / cpu_step_all_s},
            "rates": {"quant_rowwise_GBps": rates["quant_rowwise"] / 1e9, "transpose_GBps": rates["transpose"] / 1e9,
                      "gemm_GFLOPs": rates["gemm"] / 1e9, "permute_GBps": rates["permute"] / 1e9,
                      "unpermute_GBps": rates["unpermute"] / 1e9, "swiglu_GBps": rates["swiglu"] / 1e9,
                      "mx2_GBps": rates["mx2"] / 1e9, "quant_blockwise_GBps": rates["quant_blockwise"] / 1e9,
                      "dswiglu_GBps": rates["dswiglu"] / 1e9, "unpermute_backward_quant_GBps": rates["unpermute_bwd"] / 1e9},
            "output_check": check,
            "sample": ("single-threaded oracle on: 1024x7168 bf16 quant (row and block) and direct transpose, "
                       "20000 sampled outputs of the 7168-deep Fprop, permute_pad of 2048 tokens top-8, "
                       "unpermute of 2048 tokens, SwiGLU+quant of 1024x4096, SwiGLU backward of 1024x4096, "
                       "unpermute backward + quant of 2048 tokens, MOSS quant of 256x8192; each repeated "
                       f"until {budget_s} s of CPU time (all_cores: the row-parallel oracle on {n_thr} threads, "
                       f"bit-identical results, {budget_s / 2} s per op; permute_pad and the unpermute backward "
                       f"stay on one thread); {sample_s:.1f} s in all; step time extrapolated from the per-op "
                       "rates")}


def observability(torch, W, out):
    """Scale-exponent histograms of the step's quantized tensors (e = byte - 127,
    rows past an expert layout's last segment left out) and, for every direct
    transpose of the step, how many non-zero codes the exponent shift turned
    into +-0 (a shift only ever clears codes, and the transpose is otherwise a
    permutation, so that is the difference of the non-zero counts)."""
    obs = out.get("obs", {})
    hist, under = {}, {}

    def h(name, s):
        e = s.reshape(-1).to(torch.int32) - 127
        vals, cnt = torch.unique(e, return_counts=True)
        hist[name] = {"min_e": int(vals.min()), "max_e": int(vals.max()),
                      "counts": {int(v): int(c) for v, c in zip(vals.tolist(), cnt.tolist())}}

    def nz(q):
        return int(torch.count_nonzero(q & 0x7F))

    def u(name, q, qt):
        a, b = nz(q), nz(qt)
        under[name] = {"nonzero_in": a, "became_zero": a - b, "fraction": round((a - b) / max(a, 1), 8)}

    if "lin" in obs:
        o = obs["lin"]
        h("lin.X 1x128", o["xs"]), h("lin.W 128x128", o["ws"]), h("lin.dY 1x128", o["gs"])
        u("lin.direct_transpose Xq", o["xq"], o["xqt"]), u("lin.direct_transpose dYq", o["gq"], o["gqt"])
    if "moe" in obs:
        o = obs["moe"]
        used = int(o["offs"][-1])
        h("moe.X 1x128", o["xs"]), h("moe.W1 128x128", o["w1s"]), h("moe.W2 128x128", o["w2s"])
        h("moe.SwiGLU out 1x128", o["as_"][:used])
        if "dys" in o:
            h("moe_bwd.dY 1x128", o["dys"][:used]), h("moe_bwd.dH 1x128", o["dhs"][:used])
            kused = int(o["koff"][-1])
            u("moe_bwd.grouped_direct_transpose dY", o["dyq"][:used], o["dyt"][:, :kused])
    if "wg" in obs:
        o = obs["wg"]
        h("wgrad.X 1x128 (drawn 2^-20..2^4)", W["wg"]["xs"])
        u("wgrad.direct_transpose X", W["wg"]["xq"], o["xqt"]), u("wgrad.direct_transpose dY", W["wg"]["gq"], o["gqt"])
        h("wgrad.X^T block-max scales", o["xst"])
    if "moss" in obs:
        o = obs["moss"]
        h("moss.W level-2 1x32", o["ws2"]), h("moss.W^T level-2 1x32", o["s2"]), h("moss.A 1x32", o["as_"])
    return {"scale_exponent_histograms": hist, "transpose_underflow": under}


def _calc_diff(x, y):
    """DeepSeek-V3's GEMM similarity measure: 1 - 2 sum(xy) / sum(x^2 + y^2)."""
    x = x.astype("float64")
    y = y.astype("float64")
    return float(1.0 - 2.0 * (x * y).sum() / (x * x + y * y).sum())


def oracle_output_check(torch, synth, W, out, mode, seed):
    """Part of the CPU-baseline leg: the oracle recomputes sampled outputs of the
    step's GEMMs whose operands it can quantize from the synthetic inputs itself
    (the Linear's three, the K = 32768 Wgrad, the MoE fc1, the MOSS GEMM) and
    the GPU's values from the last timed step are compared with them: maximum
    |d| / max|ref|, elementwise one-bf16-ulp count for BF16 outputs, and
    DeepSeek-V3's calc_diff."""
    import numpy as np

    import oracle as O

    rng = np.random.default_rng(seed + 99)
    res = {}

    def bf16_vals(t):
        return t.float().cpu().numpy().astype(np.float64)

    def judge(name, got, ref, bf16):
        d = np.abs(got - ref)
        scale = float(np.max(np.abs(ref)))
        r = {"samples": int(ref.size), "max_abs_err_over_max_ref": float(d.max() / scale),
             "calc_diff": _calc_diff(got, ref)}
        if bf16:
            ulp = np.exp2(np.floor(np.log2(np.maximum(np.abs(ref), 2.0 ** -133))) - 7)
            ok = (d <= ulp) | (d <= 1e-5 * scale)
            r["beyond_one_bf16_ulp"] = int((~ok).sum())
            r["within_tolerance"] = bool(ok.all())
        else:
            r["within_tolerance"] = bool(d.max() / scale <= 1e-5)
        res[name] = r

    def samples(M, N, n):
        mi = np.concatenate([rng.integers(0, M, n), [0, M - 1, 255, 256 % M]])
        ni = np.concatenate([rng.integers(0, N, n), [N - 1, 0, 256 % N, 255]])
        return mi.astype(np.int64), ni.astype(np.int64)

    if "lin" in out:
        L = W["lin"]
        y, dx, dw = out["lin"]
        xq, xs = O.quant_rowwise(synth.bf16_bits(L["X"]))
        wq, ws = O.quant_blockwise(synth.bf16_bits(L["W"]))
        gq, gs = O.quant_rowwise(synth.bf16_bits(L["dY"]))
        for name, a, sa, ag, b, sb, bg, d in [
                ("lin.gemm fprop", xq, xs, O.ROW1x128, wq, ws, O.BLOCK128, y),
                ("lin.gemm dgrad", gq, gs, O.ROW1x128, wq.T.copy(), ws.T.copy(), O.BLOCK128, dx)]:
            mi, ni = samples(a.shape[0], b.shape[0], 1000)
            judge(name, bf16_vals(d[mi, ni]), O.block_gemm_sampled(a, sa, ag, b, sb, bg, mi, ni), True)
        xqt, xst = O.direct_transpose(xq, xs)
        gqt, gst = O.direct_transpose(gq, gs)
        mi, ni = samples(gqt.shape[0], xqt.shape[0], 600)
        judge("lin.gemm wgrad", bf16_vals(dw[mi, ni]),
              O.block_gemm_sampled(gqt, gst, O.ROW1x128, xqt, xst, O.ROW1x128, mi, ni), True)
    if "wg" in out:
        Wg = W["wg"]
        xqt, xst = O.direct_transpose(Wg["xq"].cpu().numpy(), Wg["xs"].cpu().numpy())
        gqt, gst = O.direct_transpose(Wg["gq"].cpu().numpy(), Wg["gs"].cpu().numpy())
        mi, ni = samples(gqt.shape[0], xqt.shape[0], 250)
        judge("wgrad.gemm K=32768", out["wg"][mi, ni].cpu().numpy().astype(np.float64),
              O.block_gemm_sampled(gqt, gst, O.ROW1x128, xqt, xst, O.ROW1x128, mi, ni), False)
    if "moe" in out and "obs" in out and "moe" in out["obs"]:
        E = W["moe"]
        xq, xs = O.quant_rowwise(synth.bf16_bits(E["X"]))
        pq, ps, _, off, used = O.permute_pad(xq, xs, E["idx"].cpu().numpy(), E["G"], 16, E["M_cap"])
        h = out["obs"]["moe"]["h"]
        H, N1 = E["X"].shape[1], E["N1"]
        W1 = E["W1"].view(E["G"], N1, H)
        mis, nis, refs = [], [], []
        for e in rng.choice([g for g in range(E["G"]) if off[g + 1] > off[g]], 4, replace=False):
            rb = int(rng.integers(0, N1 // 128))
            bq, bs = O.quant_blockwise(synth.bf16_bits(W1[e, rb * 128:(rb + 1) * 128]))
            mi = rng.integers(off[e], off[e + 1], 150).astype(np.int64)
            nl = rng.integers(0, 128, 150).astype(np.int64)
            refs.append(O.block_gemm_sampled(pq, ps, O.ROW1x128, bq, bs, O.BLOCK128, mi, nl))
            mis.append(mi)
            nis.append(nl + rb * 128)
        mi, ni = np.concatenate(mis), np.concatenate(nis)
        judge("moe.grouped_gemm fc1", bf16_vals(h[mi, ni]), np.concatenate(refs), True)
    if "moss" in out:
        Mo = W["moss"]
        y = out["moss"][1]
        mi, ni = samples(Mo["A"].shape[0], Mo["Wt"].shape[0], 500)
        um, im = np.unique(mi, return_inverse=True)
        un, in_ = np.unique(ni, return_inverse=True)
        aq, as_ = O.quant_rowwise(synth.bf16_bits(Mo["A"][torch.from_numpy(um).to(Mo["A"].device)]), 32)
        bq, bs2, bs1 = O.mx2_quant(synth.bf16_bits(Mo["Wt"][torch.from_numpy(un).to(Mo["Wt"].device)]), 10240)
        ref = O.block_gemm_sampled(aq, as_, O.ROW1x32, bq, bs2, O.ROW1x32, im.astype(np.int64), in_.astype(np.int64),
                                   b_l1=bs1, g1=10240)
        judge("moss.gemm MX", y[mi, ni].cpu().numpy().astype(np.float64), ref, False)
        # the SNR of both weight layouts, the oracle's own quantization of 256 rows beside the GPU's
        snr = {}
        for key, x, xh in (("W [8192, 28672]", Mo["W"], out["moss"][2]), ("W^T [28672, 8192]", Mo["Wt"], out["moss"][0])):
            xb = synth.bf16_bits(x[:256])
            oq, o2, o1 = O.mx2_quant(xb, 10240)
            oxh = O.mx2_dequant(oq, o2, o1, 10240)
            xf = (xb.astype(np.uint32) << 16).view(np.float32)
            gxh = xh[:256].cpu().numpy()
            snr[key] = {"oracle_snr_db_rows_0_255": round(O.snr_db(xf, oxh), 4),
                        "gpu_snr_db_rows_0_255": round(O.snr_db(xf, np.ascontiguousarray(gxh)), 4),
                        "gpu_dequant_bit_identical_to_oracle": bool(np.array_equal(gxh.view(np.uint32),
                                                                                   oxh.view(np.uint32)))}
        res["moss_snr"] = snr
    res["gemm_mode"] = mode
    return res


def _time_us(torch, fn, reps=10):
    for _ in range(2):
        fn()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        fn()
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / reps * 1e3


def median_flushed_us(torch, scratch, fn):
    """Median duration of fn in us over the last 20 of 21 repetitions, each
    preceded by a write of the 512 MB scratch buffer (twice the 256 MB
    Infinity Cache), so fn's operands come from HBM."""
    ts = []
    for r in range(21):
        scratch.fill_(float(r))
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        fn()
        e1.record()
        torch.cuda.synchronize()
        ts.append(e0.elapsed_time(e1) * 1e3)
    ts = sorted(ts[1:])
    return (ts[9] + ts[10]) / 2


def hbm_reference(fgb, torch, dev):
    """What plain byte movement sustains in each access pattern of the
    data-movement kernels (fgb_hbm_probe: the same 16-byte nontemporal loads
    and stores, nothing else), on a [32768, 7168] byte matrix, cache flushed
    as in isolated_flushed; beside them the library's k = 0 block transpose of
    the same matrix (a pure byte transpose with its LDS staging)."""
    scratch = torch.empty(512 * 2 ** 20 // 4, dtype=torch.float32, device=dev)
    rows, cols = 32768, 7168
    n = rows * cols
    g = torch.Generator(device="cpu").manual_seed(5)
    src = torch.randint(0, 256, (rows, cols), dtype=torch.uint8, generator=g).to(dev)
    dst = torch.empty_like(src)
    red = torch.empty(n // 256, dtype=torch.uint8, device=dev)
    sb = torch.full((rows // 128, cols // 128), 127, dtype=torch.uint8, device=dev)
    out = {}

    def rec(name, nbytes, fn):
        us = median_flushed_us(torch, scratch, fn)
        out[name] = {"us": round(us, 1), "GB/s": round(nbytes / us / 1e3, 1),
                     "frac": round(nbytes / us / 1e3 / HBM_PEAK_GBS, 4)}

    rec("copy", 2 * n, lambda: fgb.fgb_hbm_probe(src, dst, fgb.PROBE_COPY))
    rec("read", n + n // 256, lambda: fgb.fgb_hbm_probe(src, red, fgb.PROBE_READ))
    rec("fill (write only)", n, lambda: fgb.fgb_hbm_probe(None, dst, fgb.PROBE_FILL))
    rec("strided read (128-byte row pieces), contiguous write", 2 * n,
        lambda: fgb.fgb_hbm_probe(src, dst, fgb.PROBE_STRIDED_READ))
    rec("contiguous read, strided write (128-byte row pieces)", 2 * n,
        lambda: fgb.fgb_hbm_probe(src, dst, fgb.PROBE_STRIDED_WRITE))
    rec("block transpose k = 0 [32768, 7168]", 2 * (n + n // 16384),
        lambda: fgb.fp8_direct_transpose(src, sb, fgb.BLOCK128))
    del scratch, src, dst, red
    return {"matrix": [rows, cols], "patterns": out}


def isolated_flushed(fgb, torch, W, dev):
    """The bandwidth kernels of the step, each timed alone: before every one of
    21 repetitions a 512 MB scratch buffer is written (twice the 256 MB
    Infinity Cache), so the kernel's operands come from HBM; median of the
    last 20 (the first warms up)."""
    scratch = torch.empty(512 * 2 ** 20 // 4, dtype=torch.float32, device=dev)

    def med_us(fn):
        return median_flushed_us(torch, scratch, fn)

    out = {}

    def rec(name, nbytes, fn):
        us = med_us(fn)
        out[name] = {"us": round(us, 1), "GB/s": round(nbytes / us / 1e3, 1),
                     "frac": round(nbytes / us / 1e3 / HBM_PEAK_GBS, 4)}

    E = W["moe"]
    T, H = E["X"].shape
    G, M_cap, F = E["G"], E["M_cap"], E["F"]
    topk = E["idx"].shape[1]
    pad_rows = int(((E["counts"] + 15) // 16 * 16).sum())
    xq, xs = fgb.fp8_quant_rowwise(E["X"])
    rec("quant_rowwise X [16384, 7168]", T * H * 3 + T * H // 128, lambda: fgb.fp8_quant_rowwise(E["X"], 128, xq, xs))
    L = W["lin"]
    Tl, Cin = L["X"].shape
    lq, ls = fgb.fp8_quant_rowwise(L["X"])
    rec("quant_rowwise X [8192, 7168]", Tl * Cin * 3 + Tl * Cin // 128,
        lambda: fgb.fp8_quant_rowwise(L["X"], 128, lq, ls))
    rec("quant_blockwise W1 [131072, 7168]", E["W1"].numel() * 3 + E["W1"].numel() // 16384,
        lambda: fgb.fp8_quant_blockwise(E["W1"]))
    pq, ps, rmap, offs = fgb.permute_pad(xq, xs, E["idx"], G, 16, M_cap, E["ws"])
    rec("permute_pad", T * H * (1 + 1 / 128) + pad_rows * H * (1 + 1 / 128) + 8 * T * topk,
        lambda: fgb.permute_pad(xq, xs, E["idx"], G, 16, M_cap, E["ws"]))
    h = torch.randn((M_cap, 2 * F), device=dev).to(torch.bfloat16)
    rec("swiglu_quant", pad_rows * (2 * F * 2 + F * (1 + 1 / 128)), lambda: fgb.swiglu_quant(h, offs))
    del h
    y = torch.randn((M_cap, H), device=dev).to(torch.bfloat16)
    rec("unpermute_unpad", T * topk * H * 2 + T * H * 2 + 8 * T * topk, lambda: fgb.unpermute_unpad(y, rmap, E["probs"]))
    del y, pq, ps
    Wg = W["wg"]
    for key, qk, sk in (("direct_transpose X [32768, 7168]", "xq", "xs"), ("direct_transpose dY [32768, 2048]", "gq", "gs")):
        q, sc = Wg[qk], Wg[sk]
        rec(key, 2 * (q.numel() + q.numel() // 128), lambda: fgb.fp8_direct_transpose(q, sc))
    if "moss" in W:
        Wt = W["moss"]["Wt"]
        R, Cc = Wt.shape
        rec("mx2_quant W^T [28672, 8192]", R * Cc * (3 + 1 / 32) + 4 * R * ((Cc + 10239) // 10240),
            lambda: fgb.mx2_quant(Wt, 10240))
    del scratch
    return out


def format_variants(fgb, torch, W, dev, args):
    """Outside the step: the format variants on the step's tensors -- E5M2
    gradient quantization and transpose of the MoE dO, the Dgrad GEMM with an
    E5M2 gradient, the MX floor rule in the MOSS quantizer, and the masked
    grouped GEMM at a decode shape."""
    gm = fgb.GEMM_EXACT if args.gemm_mode == "exact" else fgb.GEMM_FAST
    peak = MFMA_PEAK_TFLOPS[args.gemm_mode]
    out = {}
    dO = W["moe"]["dO"]
    T, H = dO.shape
    gq, gs = fgb.fp8_quant_rowwise_fmt(dO, 128, fgb.E5M2, fgb.SCALE_CEIL)
    us = _time_us(torch, lambda: fgb.fp8_quant_rowwise_fmt(dO, 128, fgb.E5M2, fgb.SCALE_CEIL, gq, gs))
    nb = T * H * 3 + T * H // 128
    out["quant_rowwise E5M2 dO [16384, 7168]"] = {"us": round(us, 1), "GB/s": round(nb / us / 1e3, 1),
                                                   "frac": round(nb / us / 1e3 / HBM_PEAK_GBS, 4)}
    us = _time_us(torch, lambda: fgb.fp8_direct_transpose_fmt(gq, gs, fgb.E5M2))
    nb = 2 * (T * H + T * H // 128)
    out["direct_transpose E5M2 dO"] = {"us": round(us, 1), "GB/s": round(nb / us / 1e3, 1),
                                       "frac": round(nb / us / 1e3 / HBM_PEAK_GBS, 4)}
    del gq, gs
    L = W["lin"]
    Tl, Cin = L["X"].shape
    Cout = L["W"].shape[0]
    wq, ws = fgb.fp8_quant_blockwise(L["W"])
    wqt, wst = fgb.fp8_direct_transpose(wq, ws, fgb.BLOCK128)
    lq, ls = fgb.fp8_quant_rowwise_fmt(L["dY"], 128, fgb.E5M2, fgb.SCALE_CEIL)
    d = torch.empty((Tl, Cin), dtype=torch.bfloat16, device=dev)
    us = _time_us(torch, lambda: fgb.fp8_block_gemm_fmt(lq, ls, fgb.ROW1x128, fgb.E5M2, wqt, wst, fgb.BLOCK128,
                                                        fgb.E4M3, d=d, mode=gm))
    fl = 2 * Tl * Cin * Cout
    out["gemm dgrad, dY E5M2 (8192x7168x2048)"] = {"us": round(us, 1), "TFLOP/s": round(fl / us / 1e6, 1),
                                                   "frac": round(fl / us / 1e6 / peak, 4)}
    del wq, ws, wqt, wst, lq, ls, d
    if "moss" in W:
        Wt = W["moss"]["Wt"]
        R, Cc = Wt.shape
        g1 = 10240
        us = _time_us(torch, lambda: fgb.mx2_quant_rule(Wt, g1, fgb.SCALE_OCP_FLOOR))
        nb = R * Cc * (3 + 1 / 32) + 4 * R * ((Cc + g1 - 1) // g1)
        out["mx2_quant floor rule W^T [28672, 8192]"] = {"us": round(us, 1), "GB/s": round(nb / us / 1e3, 1),
                                                         "frac": round(nb / us / 1e3 / HBM_PEAK_GBS, 4)}
    # masked grouped GEMM, decode: 512 tokens top-8 over the 32 experts' fc1 (N 4096, K 7168)
    import numpy as np

    import synth

    E = W["moe"]
    G, N1 = E["G"], E["N1"]
    w1q, w1s = fgb.fp8_quant_blockwise(E["W1"])
    idx, _ = synth.routing(512, G, 8, 1.1, args.seed)
    counts = np.bincount(idx.ravel(), minlength=G)
    M_max = 512
    xa = torch.randn((G * M_max, H), device=dev).to(torch.bfloat16)
    aq, as_ = fgb.fp8_quant_rowwise(xa)
    del xa
    mm = torch.from_numpy(counts.astype(np.int32)).to(dev)
    d = torch.empty((G, M_max, N1), dtype=torch.bfloat16, device=dev)
    us = _time_us(torch, lambda: fgb.fp8_grouped_gemm_masked(aq.view(G, M_max, H), as_.view(G, M_max, H // 128),
                                                             w1q.view(G, N1, H), w1s.view(G, N1 // 128, H // 128), mm,
                                                             d=d, mode=gm))
    fl = 2 * int(counts.sum()) * N1 * H
    wb = G * N1 * H  # the expert weights are read at least once: decode is weight-bandwidth bound
    out["masked grouped gemm, decode 512 tok top-8 (fc1)"] = {
        "us": round(us, 1), "TFLOP/s": round(fl / us / 1e6, 1), "weight GB/s": round(wb / us / 1e3, 1),
        "frac_of_hbm": round(wb / us / 1e3 / HBM_PEAK_GBS, 4)}
    del w1q, w1s, aq, as_, d
    return out


def vendor_gemm(fgb, torch, synth, dev, seed):
    """Rates of the blockwise GEMM (A 1x128, B 128x128 scales; exact and fast
    modes) and, on the same N(0,1) data, of the vendor library's bf16 GEMM
    (no scaling) and FP8 GEMM with one scale per row of A and per row of B:
    simpler computations than the blockwise one, timed as a point of
    comparison for what the chip sustains at these shapes."""
    out = {}
    for (M, N, K) in [(16384, 4096, 7168), (8192, 2048, 7168), (8192, 7168, 2048)]:
        fl = 2.0 * M * N * K
        a = synth.normal((M, K), 1.0, seed, 61, dev, torch.bfloat16)
        b = synth.normal((N, K), 1.0, seed, 62, dev, torch.bfloat16)
        aq, as_ = fgb.fp8_quant_rowwise(a)
        bq, bs = fgb.fp8_quant_blockwise(b)
        a8, b8 = a.to(torch.float8_e4m3fn), b.to(torch.float8_e4m3fn)
        sa = torch.ones(M, 1, device=dev)
        sb = torch.ones(1, N, device=dev)
        r = {}
        for name, fn in [
            ("blockwise exact", lambda: fgb.fp8_block_gemm(aq, as_, fgb.ROW1x128, bq, bs, fgb.BLOCK128,
                                                            mode=fgb.GEMM_EXACT)),
            ("blockwise fast", lambda: fgb.fp8_block_gemm(aq, as_, fgb.ROW1x128, bq, bs, fgb.BLOCK128,
                                                           mode=fgb.GEMM_FAST)),
            ("vendor bf16", lambda: torch.matmul(a, b.t())),
            ("vendor fp8 row-wise scaled", lambda: torch._scaled_mm(a8, b8.t(), scale_a=sa, scale_b=sb,
                                                                    out_dtype=torch.bfloat16)),
        ]:
            us = _time_us(torch, fn, reps=20)
            r[name] = {"us": round(us, 1), "TFLOP/s": round(fl / us / 1e6, 1)}
        out[f"{M}x{N}x{K}"] = r
        log(f"vendor gemm {M}x{N}x{K}: {r}")
        del a, b, aq, as_, bq, bs, a8, b8
    return out


def main():
    args = parse()
    if args.gpus != 1:
        print(json.dumps({"error": "this library runs on one GPU; --gpus must be 1 (multi-GPU sharding is described, not implemented)"}))
        sys.exit(2)
    import torch

    import fine_grained_blockwise_amd as fgb
    import synth

    dev = torch.device("cuda:0")
    if args.copy_calibration:
        n = 1 << 28  # float32 elements: 1 GiB in, 1 GiB out per launch
        src = torch.ones(n, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            torch.neg(src, out=dst)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration": {"launches": 3, "read_bytes_per_launch": 4 * n,
                                               "write_bytes_per_launch": 4 * n}}))
        return
    if args.vendor_gemm:
        print(json.dumps({"vendor_gemm": vendor_gemm(fgb, torch, synth, dev, args.seed)}))
        return
    parts = set(args.parts.split(","))
    W = build(fgb, torch, synth, dev, args.seed, parts)
    log(f"inputs resident: parts={sorted(parts)} gemm_mode={args.gemm_mode}")
    rec = Recorder(torch)
    for _ in range(args.warmup):
        step(fgb, torch, W, rec, args.gemm_mode)
    torch.cuda.synchronize()
    log(f"warmup done ({args.warmup} steps); timing {args.steps} steps")
    rec.on = True
    t0 = time.perf_counter()
    for _ in range(args.steps):
        out = step(fgb, torch, W, rec, args.gemm_mode)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    rec.on = False
    ms_step = (t1 - t0) * 1e3 / args.steps
    res = rec.results()
    graph = None if args.no_graph else graph_leg(fgb, torch, W, args, out)

    kernels = {}
    floor_s = 0.0  # GEMMs at the dense FP8 peak (the value)
    floor_contraction_s = 0.0  # GEMMs at the peak of the instruction the mode issues
    for name, (ms, kind, work) in res.items():
        if kind == "hbm":
            ach = work / (ms * 1e-3) / 1e9
            peak = HBM_PEAK_GBS
            unit = "GB/s"
            floor_s += work / (HBM_PEAK_GBS * 1e9)
            floor_contraction_s += work / (HBM_PEAK_GBS * 1e9)
        else:
            ach = work / (ms * 1e-3) / 1e12
            peak = MFMA_PEAK_TFLOPS[args.gemm_mode]
            unit = "TFLOP/s"
            floor_s += work / (FP8_PEAK_TFLOPS * 1e12)
            floor_contraction_s += work / (peak * 1e12)
        kernels[name] = {"ms": round(ms, 4), "achieved": round(ach, 1), "unit": unit, "frac": round(ach / peak, 4),
                         "work": work}
        if kind == "mfma":
            kernels[name]["frac_of_fp8_peak"] = round(ach / FP8_PEAK_TFLOPS, 4)
    value = 100.0 * floor_s / (ms_step * 1e-3)
    value_contraction = 100.0 * floor_contraction_s / (ms_step * 1e-3)
    dom = max(res.items(), key=lambda kv: kv[1][0])
    dname, (dms, dkind, dwork) = dom
    dpeak = HBM_PEAK_GBS if dkind == "hbm" else MFMA_PEAK_TFLOPS[args.gemm_mode]
    dach = dwork / (dms * 1e-3) / (1e9 if dkind == "hbm" else 1e12)
    roofline = {"bound": dkind, "achieved": round(dach, 1), "peak": dpeak,
                "unit": "GB/s" if dkind == "hbm" else "TFLOP/s", "frac": round(dach / dpeak, 4),
                "traffic": traffic_for(dname, args.gemm_mode), "kernel": dname}
    if dkind == "mfma":  # the FP8 GEMM's rate against the dense FP8 peak, beside its contraction's own
        roofline["frac_of_fp8_peak"] = round(dach / FP8_PEAK_TFLOPS, 4)

    extra = {}
    if "moss" in out:
        xh, _, wh = out["moss"]
        snr = {}
        for key, x, xr in (("W [8192, 28672]", W["moss"]["W"], wh), ("W^T [28672, 8192]", W["moss"]["Wt"], xh)):
            num = (x.double() ** 2).sum()
            den = ((x.double() - xr.double()) ** 2).sum()
            snr[key] = round(float(10 * torch.log10(num / den)), 3)
        extra["moss_snr_db"] = snr
    extra.update(observability(torch, W, out))

    if "wg" in W and not args.no_study:
        # Outside the step: the direct transpose against the three-pass conversion it replaces
        # (dequantize, transpose, requantize) on the Wgrad-path tensors.
        study = {}
        for key, qk, sk in (("X [32768, 7168]", "xq", "xs"), ("dY [32768, 2048]", "gq", "gs")):
            q, sc = W["wg"][qk], W["wg"][sk]
            wsb = torch.empty(fgb.fp8_naive_transpose_workspace_size(*q.shape), dtype=torch.uint8, device=dev)
            times = {}
            for name, fn in (("direct", lambda: fgb.fp8_direct_transpose(q, sc)),
                             ("three_pass", lambda: fgb.fp8_naive_transpose(q, sc, wsb))):
                for _ in range(3):
                    fn()
                e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                e0.record()
                for _ in range(10):
                    fn()
                e1.record()
                torch.cuda.synchronize()
                times[name] = e0.elapsed_time(e1) / 10 * 1e3
            study[key] = {"direct_us": round(times["direct"], 1), "three_pass_us": round(times["three_pass"], 1),
                          "speedup": round(times["three_pass"] / times["direct"], 2)}
            del wsb
        extra["direct_vs_three_pass_transpose"] = study
        log(f"transpose study: {study}")

    if "moe" in W and "moe" in out and not args.no_study:
        # Outside the step: SwiGLU backward from the FP8-cached fc1 output, at the expert-MLP size.
        E = W["moe"]
        offs = out["moe"][1]
        F = E["F"]
        g = torch.Generator(device=dev)
        g.manual_seed(args.seed + 5)
        h = (torch.randn((E["M_cap"], 2 * F), generator=g, device=dev) * 3).to(torch.bfloat16)
        hq, hs = fgb.fp8_quant_rowwise(h)
        del h
        da = torch.randn((E["M_cap"], F), generator=g, device=dev).to(torch.bfloat16)
        dq = torch.empty_like(hq)
        ds = torch.empty_like(hs)
        for _ in range(3):
            fgb.dswiglu_quant(hq, hs, da, offs, dq, ds)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(10):
            fgb.dswiglu_quant(hq, hs, da, offs, dq, ds)
        e1.record()
        torch.cuda.synchronize()
        us = e0.elapsed_time(e1) / 10 * 1e3
        rows = int(((E["counts"] + 15) // 16 * 16).sum())
        nbytes = rows * (6 * F + 4 * F // 128)
        extra["dswiglu_quant"] = {"us": round(us, 1), "GB/s": round(nbytes / (us * 1e-6) / 1e9, 1),
                                  "frac_of_hbm": round(nbytes / (us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4),
                                  "rows": rows, "F": F}
        del hq, hs, da, dq, ds
        log(f"dswiglu study: {extra['dswiglu_quant']}")

    if "moe" in W and "lin" in W and "wg" in W and not args.no_study:
        extra["isolated_flushed"] = isolated_flushed(fgb, torch, W, dev)
        log(f"isolated, Infinity Cache flushed: {extra['isolated_flushed']}")
        extra["hbm_reference"] = hbm_reference(fgb, torch, dev)
        log(f"HBM reference patterns: {extra['hbm_reference']}")
    if "moe" in W and "dO" in W["moe"] and "lin" in W and not args.no_study:
        extra["format_variants"] = format_variants(fgb, torch, W, dev, args)
        log(f"format variants: {extra['format_variants']}")

    log(f"timed: {ms_step:.3f} ms/step")
    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(torch, synth, args.seed, res, floor_s, W, out, args.gemm_mode)
        log("cpu baseline done")

    line = {
        "metric": "blockwise-FP8 GEMM TFLOP/s & quant/transpose GB/s, % of MI355X roofline",
        "value": round(value, 2),
        "unit": "% of MI355X roofline (step; every GEMM priced at the dense FP8 peak)",
        "value_at_contraction_peak": round(value_contraction, 2),
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 3),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "e4m3",
        "data": "synthetic (seeded; shapes and distributions of the DeepSeek-V3 / MoE / MOSS layers)",
        "config": {"workload": ("dsv3-linear T8192 Cin7168 Cout2048 (fwd+bwd) + moe 16384 tok top-8 of 32 "
                                "experts H7168 F2048 (fwd" + ("+bwd" if "moe_bwd" in parts else "") + ") + wgrad T32768 Cin7168 Cout2048 + moss W^T 28672x8192 "
                                "A 4096x8192"),
                   "parts": sorted(parts), "gemm_mode": args.gemm_mode,
                   "gemm_contraction": "bf16 MFMA on exact scaled fp8->bf16 operands" if args.gemm_mode == "exact"
                   else "fp8 scaled MFMA"},
        "roofline": roofline,
        "graph": graph,
        "cpu_baseline": cpu,
        "inputs_sha256_every_64th_row": input_digest(torch, W),
        "kernels": kernels,
        **extra,
    }
    print(json.dumps(line))


if __name__ == "__main__":
    main()
