"""The whole hot path captured in one HIP graph and replayed.

Every entry point enqueues kernels only on the caller's stream: no host
synchronisation, no allocation inside the library and no memset nodes (buffers
that must start at zero are cleared by the library's own fill kernels).  So a
step of the path (the Linear forward and backward, the MoE expert forward and
backward, MOSS) can be captured once and replayed.  Each replay runs on new
inputs written into the captured input buffers between replays, with eager
work and synchronisations in between; every output of every replay must equal,
bit for bit, the same step run eagerly on the same inputs (all kernels are
deterministic)."""
import numpy as np
import pytest
import torch

from test_gpu_parity import DEV, say

pytestmark = pytest.mark.gpu

T_LIN, CIN, COUT = 512, 512, 256
T_MOE, TOPK, G, H, F = 300, 4, 6, 512, 256
M_CAP = T_MOE * TOPK + 15 * G
MOSS_R, MOSS_C, MOSS_M = 256, 1024, 128


@pytest.fixture(scope="module")
def fgb():
    import fine_grained_blockwise_amd as m
    return m


def _inputs(seed):
    """Seeded CPU inputs of the step (bf16 activations and weights, routing, probs)."""
    g = torch.Generator().manual_seed(seed)
    r = lambda *s, sc=1.0: (torch.randn(*s, generator=g) * sc).to(torch.bfloat16)
    idx = torch.stack([torch.randperm(G, generator=g)[:TOPK] for _ in range(T_MOE)]).to(torch.int32)
    idx[idx == (seed % G)] = -1  # one expert empty, its slots dropped
    probs = torch.rand(T_MOE, TOPK, generator=g)
    return dict(lx=r(T_LIN, CIN), lw=r(COUT, CIN, sc=0.05), ldy=r(T_LIN, COUT, sc=1e-3),
                mx=r(T_MOE, H), w1=r(G * 2 * F, H, sc=0.05), w2=r(G * H, F, sc=0.05), idx=idx, probs=probs,
                do=r(T_MOE, H, sc=1e-3), mw=r(MOSS_R, MOSS_C, sc=0.02), ma=r(MOSS_M, MOSS_C))


def _step(fgb, I, ws_pp, ws_ub):
    """One pass of the hot path on the device buffers in I; returns every output."""
    out = []
    xq, xs = fgb.fp8_quant_rowwise(I["lx"])
    wq, ws = fgb.fp8_quant_blockwise(I["lw"])
    gq, gs = fgb.fp8_quant_rowwise(I["ldy"])
    out.append(fgb.fp8_block_gemm(xq, xs, fgb.ROW1x128, wq, ws, fgb.BLOCK128))
    wqt, wst = fgb.fp8_direct_transpose(wq, ws, fgb.BLOCK128)
    out.append(fgb.fp8_block_gemm(gq, gs, fgb.ROW1x128, wqt, wst, fgb.BLOCK128))
    xqt, xst = fgb.fp8_direct_transpose(xq, xs)
    gqt, gst = fgb.fp8_direct_transpose(gq, gs)
    out.append(fgb.fp8_block_gemm(gqt, gst, fgb.ROW1x128, xqt, xst, fgb.ROW1x128, out_dtype=torch.float32))
    # MoE expert forward
    mq, ms = fgb.fp8_quant_rowwise(I["mx"])
    w1q, w1s, w1t, w1ts = fgb.fp8_quant_blockwise_t(I["w1"].view(G, 2 * F, H))
    w2q, w2s, w2t, w2ts = fgb.fp8_quant_blockwise_t(I["w2"].view(G, H, F))
    pq, ps, rmap, offs = fgb.permute_pad(mq, ms, I["idx"], G, 16, M_CAP, ws_pp)
    h = fgb.fp8_grouped_gemm(pq, ps, w1q, w1s, offs)
    aq, as_, hq, hs = fgb.swiglu_quant_cache(h, offs)
    y = fgb.fp8_grouped_gemm(aq, as_, w2q, w2s, offs)
    out += [offs, rmap, fgb.unpermute_unpad(y, rmap, I["probs"])]
    # MoE expert backward
    dyq, dys = fgb.unpermute_backward_quant(I["do"], rmap, I["probs"], M_CAP, workspace=ws_ub)
    da = fgb.fp8_grouped_gemm(dyq, dys, w2t, w2ts, offs)
    dyt, dyts, koff = fgb.fp8_grouped_direct_transpose(dyq, dys, offs)
    at, ats, _ = fgb.fp8_grouped_direct_transpose(aq, as_, offs)
    out.append(fgb.fp8_kgrouped_gemm(dyt, dyts, at, ats, koff))
    dhq, dhs = fgb.dswiglu_quant(hq, hs, da, offs)
    dxp = fgb.fp8_grouped_gemm(dhq, dhs, w1t, w1ts, offs)
    dht, dhts, _ = fgb.fp8_grouped_direct_transpose(dhq, dhs, offs)
    xt, xts, _ = fgb.fp8_grouped_direct_transpose(pq, ps, offs)
    out.append(fgb.fp8_kgrouped_gemm(dht, dhts, xt, xts, koff))
    out.append(fgb.unpermute_unpad(dxp, rmap, None))
    # MOSS: two-level quant and dequant, MX GEMM with the level-1 factors
    q, s2, s1 = fgb.mx2_quant(I["mw"], 10240)
    out.append(fgb.mx2_dequant(q, s2, s1, 10240))
    maq, mas = fgb.fp8_quant_rowwise(I["ma"], 32)
    out.append(fgb.fp8_block_gemm(maq, mas, fgb.ROW1x32, q, s2, fgb.ROW1x32, b_l1=s1.view(-1), g1=10240,
                                  out_dtype=torch.float32))
    return out


def _bits(t):
    t = t.detach().cpu().contiguous()
    return t.view(torch.int16).numpy() if t.dtype == torch.bfloat16 else t.numpy()


def test_hot_path_graph_replays_match_eager(fgb):
    say("hot path captured in one graph: 3 replays on new inputs, each against the eager step")
    ws_pp = torch.empty(fgb.permute_pad_workspace_size(T_MOE, TOPK, G), dtype=torch.uint8, device=DEV)
    ws_ub = torch.empty(fgb.unpermute_backward_workspace_size(M_CAP), dtype=torch.uint8, device=DEV)
    static = {k: v.to(DEV) for k, v in _inputs(0).items()}
    # eager pass first: it also sets the per-device kernel attributes outside the capture
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        _step(fgb, static, ws_pp, ws_ub)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        captured = _step(fgb, static, ws_pp, ws_ub)
    for rep, seed in enumerate((1, 2, 3)):
        new = _inputs(seed)
        for k, v in new.items():
            static[k].copy_(v.to(DEV))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        got = [_bits(t) for t in captured]
        # the same inputs through the eager path, in separate buffers
        ws_pp2 = torch.empty_like(ws_pp)
        ws_ub2 = torch.empty_like(ws_ub)
        want = [_bits(t) for t in _step(fgb, {k: v.to(DEV) for k, v in new.items()}, ws_pp2, ws_ub2)]
        torch.cuda.synchronize()
        assert len(got) == len(want)
        for i, (a, b) in enumerate(zip(got, want)):
            assert a.shape == b.shape and np.array_equal(a, b), (rep, i)
        say(f"replay {rep}: {len(got)} outputs bit-identical to the eager step")
