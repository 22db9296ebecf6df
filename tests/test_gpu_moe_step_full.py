"""The MoE expert layer of the step at its full size (16384 tokens, top-8 of
32 experts, H 7168, F 2048; the bench's seeded inputs), forward and
backward, run as the bench times it (exact GEMM mode).  Every op's output is
checked against the oracle fed with that op's actual inputs from the GPU
chain, so each step is checked on its own at the workload's full size:
data movement bit for bit on sampled rows, tokens and blocks; GEMMs on
sampled outputs that include every segment's first and last row and the
columns on both sides of the 256-wide tile edges, to the exact mode's
tolerance."""
import numpy as np
import pytest
import torch

import oracle as O
import synth
from test_gpu_parity import DEV, bits, check_gemm, np_, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def fgb():
    import fine_grained_blockwise_amd as m
    return m


def _rows_sample(rng, off, n):
    """Every non-empty segment's first and last row, plus n random rows of the segments."""
    edges = np.concatenate([[off[g], off[g + 1] - 1] for g in range(len(off) - 1) if off[g + 1] > off[g]])
    return np.unique(np.concatenate([edges, rng.integers(0, off[-1], n)])).astype(np.int64)


def _cols_sample(rng, N, n):
    edges = [c for c in range(0, N, 256)] + [c - 1 for c in range(256, N + 1, 256)] + [N - 1]
    return np.unique(np.concatenate([edges, rng.integers(0, N, n)])).astype(np.int64)


def _grouped_check(a, sa, b, sb, off, d, rng, K):
    """Sampled outputs of an M-grouped GEMM (BF16 out) against the oracle."""
    rows, cols = _rows_sample(rng, off, 96), _cols_sample(rng, b.shape[1], 12)
    mi, ni = np.repeat(rows, len(cols)), np.tile(cols, len(rows))
    ref = O.grouped_gemm_sampled(a, sa, b, sb, off, mi, ni)
    check_gemm(np_(d)[mi, ni], ref, "exact", True, None, K)


def _kgrouped_check(a, sa, b, sb, koff, d, rng):
    G, M, N = d.shape
    e = np.concatenate([np.arange(G).repeat(8), rng.integers(0, G, 2000)])
    m = np.concatenate([np.tile([0, 255, 256, M - 1, 0, M - 1, 128, 4000 % M], G), rng.integers(0, M, 2000)])
    n = np.concatenate([np.tile([0, 256, 255, N - 1, N - 1, 0, 7, 1000 % N], G), rng.integers(0, N, 2000)])
    ref = O.kgrouped_gemm_sampled(a, sa, b, sb, koff, e, m, n)
    check_gemm(np_(d)[e, m, n], ref, "exact", False, None, None)


def _unpermute_check(y, orm, probs, out, toks):
    """out[toks] against the oracle on just the rows those tokens' slots name."""
    sub = orm[toks]
    rows = np.unique(sub[sub >= 0])
    remap = np.full(y.shape[0], -1, np.int64)
    remap[rows] = np.arange(len(rows))
    rm_sub = np.where(sub >= 0, remap[np.maximum(sub, 0)], -1).astype(np.int32)
    ref = O.unpermute_unpad(np_(y[torch.from_numpy(rows).to(DEV)]), rm_sub, None if probs is None else probs[toks])
    assert np.array_equal(np_(out[torch.from_numpy(toks).to(DEV)]), ref)


def test_moe_layer_forward_backward_full(fgb):
    say("MoE layer at full size, forward and backward, each op against the oracle on sampled outputs")
    rng = np.random.default_rng(0)
    X, idx, probs, W1, W2 = synth.moe(0, device=DEV)
    dO = synth.moe_grad(0, device=DEV)
    T, H = X.shape
    G, N1, F, N2 = W1.shape[0], W1.shape[1], W1.shape[1] // 2, W2.shape[1]
    topk = idx.shape[1]
    M_cap = T * topk + 15 * G
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(DEV)

    # the chain, as the bench runs it
    xq, xs = fgb.fp8_quant_rowwise(X)
    w1q, w1s, w1t, w1ts = fgb.fp8_quant_blockwise_t(W1)
    w2q, w2s, w2t, w2ts = fgb.fp8_quant_blockwise_t(W2)
    pq, ps, rmap, offs = fgb.permute_pad(xq, xs, t(idx), G, 16, M_cap)
    h = fgb.fp8_grouped_gemm(pq, ps, w1q, w1s, offs)
    aq, as_, hq, hs = fgb.swiglu_quant_cache(h, offs)
    y = fgb.fp8_grouped_gemm(aq, as_, w2q, w2s, offs)
    o = fgb.unpermute_unpad(y, rmap, t(probs))
    dyq, dys = fgb.unpermute_backward_quant(dO, rmap, t(probs), M_cap)
    da = fgb.fp8_grouped_gemm(dyq, dys, w2t, w2ts, offs)
    dyt, dyts, koff = fgb.fp8_grouped_direct_transpose(dyq, dys, offs)
    at, ats, _ = fgb.fp8_grouped_direct_transpose(aq, as_, offs)
    dw2 = fgb.fp8_kgrouped_gemm(dyt, dyts, at, ats, koff)
    dhq, dhs = fgb.dswiglu_quant(hq, hs, da, offs)
    dxp = fgb.fp8_grouped_gemm(dhq, dhs, w1t, w1ts, offs)
    dht, dhts, _ = fgb.fp8_grouped_direct_transpose(dhq, dhs, offs)
    xt, xts, _ = fgb.fp8_grouped_direct_transpose(pq, ps, offs)
    dw1 = fgb.fp8_kgrouped_gemm(dht, dhts, xt, xts, koff)
    dx = fgb.unpermute_unpad(dxp, rmap, None)
    torch.cuda.synchronize()

    # quantizers: sampled token rows of X, two 128-row blocks of each weight and their transposed copies
    rows = np.unique(np.concatenate([np.arange(16), T - 16 + np.arange(16), rng.integers(0, T, 32)]))
    oq, os_ = O.quant_rowwise(bits(X[t(rows)].cpu()), 128)
    assert np.array_equal(np_(xq[t(rows)]), oq) and np.array_equal(np_(xs[t(rows)]), os_)
    for W, wq, ws, wt in ((W1, w1q, w1s, w1t), (W2, w2q, w2s, w2t)):
        for e, rb in ((0, 0), (G - 1, W.shape[1] // 128 - 1)):
            bq, bs = O.quant_blockwise(bits(W[e, rb * 128:(rb + 1) * 128].cpu()))
            assert np.array_equal(np_(wq[e, rb * 128:(rb + 1) * 128]), bq), e
            assert np.array_equal(np_(ws[e, rb]), bs[0]), e
            assert np.array_equal(np_(wt[e, :, rb * 128:(rb + 1) * 128]), bq.T), e

    # permute + pad: the layout from the oracle, sampled tokens' rows
    z = np.zeros((T, 128), np.uint8)
    _, _, orm, ooff, used = O.permute_pad(z, z[:, :1], idx, G, 16, M_cap)
    assert np.array_equal(np_(offs), ooff) and np.array_equal(np_(rmap), orm)
    toks = np.unique(np.concatenate([np.arange(8), T - 8 + np.arange(8), rng.integers(0, T, 48)]))
    xqh, xsh = np_(xq[t(toks)]), np_(xs[t(toks)])
    for i, tk in enumerate(toks):
        for r in orm[tk]:
            if r >= 0:
                assert np.array_equal(np_(pq[int(r)]), xqh[i]) and np.array_equal(np_(ps[int(r)]), xsh[i])

    # the host copies the GEMM checks read
    pq_h, ps_h = np_(pq), np_(ps)
    w1q_h, w1s_h, w2q_h, w2s_h = np_(w1q), np_(w1s), np_(w2q), np_(w2s)
    w1t_h, w1ts_h, w2t_h, w2ts_h = np_(w1t), np_(w1ts), np_(w2t), np_(w2ts)

    # fc1, SwiGLU + quant and its cache, fc2, unpermute
    _grouped_check(pq_h, ps_h, w1q_h, w1s_h, ooff, h, rng, H)
    srows = _rows_sample(rng, ooff, 64)
    hsub = np_(h[t(srows)])
    sq, ss = O.swiglu_quant(hsub)
    cq, cs = O.quant_rowwise(hsub, 128)
    assert np.array_equal(np_(aq[t(srows)]), sq) and np.array_equal(np_(as_[t(srows)]), ss)
    assert np.array_equal(np_(hq[t(srows)]), cq) and np.array_equal(np_(hs[t(srows)]), cs)
    aq_h, as_h = np_(aq), np_(as_)
    _grouped_check(aq_h, as_h, w2q_h, w2s_h, ooff, y, rng, F)
    _unpermute_check(y, orm, probs, o, toks)

    # backward: unpermute backward + quant (sampled rows of the padded layout, all of their tokens)
    dyfull = O.unpermute_backward(np_(dO), orm, probs, M_cap)
    pad_rows = rng.integers(used, M_cap, 8) if M_cap > used else np.zeros(0, np.int64)  # rows no slot names
    brows = np.unique(np.concatenate([srows, pad_rows]))
    bq, bs = O.quant_rowwise(dyfull[brows], 128)
    assert np.array_equal(np_(dyq[t(brows)]), bq) and np.array_equal(np_(dys[t(brows)]), bs)
    del dyfull
    dyq_h, dys_h = np_(dyq), np_(dys)
    _grouped_check(dyq_h, dys_h, w2t_h, w2ts_h, ooff, da, rng, H)

    # direct transposes of the segments (sampled 128-column blocks of the transposed copy)
    K_cap = dyt.shape[1]
    for q_h, s_h, qt, st in ((dyq_h, dys_h, dyt, dyts), (aq_h, as_h, at, ats)):
        cols = slice(0, 128) if q_h.shape[1] == 128 else slice(q_h.shape[1] - 128, q_h.shape[1])
        oqt, ost, okoff = O.grouped_direct_transpose(q_h[:, cols], s_h[:, cols.start // 128:cols.start // 128 + 1],
                                                     ooff, K_cap)
        k = int(okoff[-1])
        assert np.array_equal(np_(koff), okoff)
        assert np.array_equal(np_(qt[cols, :k]), oqt[:, :k]) and np.array_equal(np_(st[cols, :k // 128]), ost[:, :k // 128])
    koff_h = np_(koff)
    _kgrouped_check(np_(dyt), np_(dyts), np_(at), np_(ats), koff_h, dw2, rng)

    # dSwiGLU + quant (sampled rows), fc1 Dgrad, fc1 Wgrad, permute backward
    dq, ds = O.dswiglu_quant(np_(hq[t(srows)]), np_(hs[t(srows)]), np_(da[t(srows)]))
    assert np.array_equal(np_(dhq[t(srows)]), dq) and np.array_equal(np_(dhs[t(srows)]), ds)
    _grouped_check(np_(dhq), np_(dhs), w1t_h, w1ts_h, ooff, dxp, rng, N1)
    _kgrouped_check(np_(dht), np_(dhts), np_(xt), np_(xts), koff_h, dw1, rng)
    _unpermute_check(dxp, orm, None, dx, toks)
