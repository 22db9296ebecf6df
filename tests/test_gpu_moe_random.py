"""Seeded random sweep of the MoE data path against the oracle, bit for bit:
random token counts, top-k, expert counts and widths (one 128-column group
up to eight), dropped slots and experts that receive no token.  Each case
chains the entry points the way a layer does: permute + pad of the FP8
activations, the direct transpose of the expert segments, SwiGLU + quant with
its FP8 cache, the SwiGLU backward from that cache, the probs-weighted
unpermute, and the unpermute backward fused with the 1x128 quant."""
import numpy as np
import pytest
import torch

import oracle as O
from test_gpu_parity import DEV, bits, np_, rand_codes, rand_scales, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def fgb():
    import fine_grained_blockwise_amd as m
    return m


def _routing(rng, T, topk, G):
    """topk distinct experts per token; about a third of the cases leave one
    expert without tokens, and about 10% of the slots are dropped (-1)."""
    allowed = np.arange(G)
    if G > topk and rng.random() < 0.35:
        allowed = np.delete(allowed, int(rng.integers(0, G)))
    idx = np.stack([rng.choice(allowed, topk, replace=False) for _ in range(T)]).astype(np.int32)
    idx[rng.random(idx.shape) < 0.1] = -1
    return idx


def _case(fgb, rng, case):
    T = int(rng.integers(1, 301))
    G = int(rng.integers(1, 13))
    topk = int(rng.integers(1, min(G, 8) + 1))
    H = 128 * int(rng.integers(1, 9))
    F = 128 * int(rng.integers(1, 5))
    M_cap = T * topk + 15 * G
    say(f"random moe data path {case}: T={T} topk={topk} G={G} H={H} F={F}")
    seed = 7000 + 10 * case
    idx = _routing(rng, T, topk, G)
    probs = torch.rand(T, topk, generator=torch.Generator().manual_seed(seed)).numpy().astype(np.float32)
    g = torch.Generator().manual_seed(seed + 1)
    xq, xs = rand_codes((T, H), seed + 2), rand_scales((T, H // 128), -20, 4, seed + 3)
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(DEV)

    # permute + pad
    pq, ps, rmap, offs = fgb.permute_pad(t(xq.numpy()), t(xs.numpy()), t(idx), G, 16, M_cap)
    oq, os_, orm, ooff, used = O.permute_pad(xq.numpy(), xs.numpy(), idx, G, 16, M_cap)
    assert np.array_equal(np_(offs), ooff) and np.array_equal(np_(rmap), orm), case
    assert np.array_equal(np_(pq)[:used], oq[:used]) and np.array_equal(np_(ps)[:used], os_[:used]), case

    # direct transpose of the expert segments (the Wgrad operand)
    qt, st, koff = fgb.fp8_grouped_direct_transpose(t(oq), t(os_), t(ooff))
    oqt, ost, okoff = O.grouped_direct_transpose(oq, os_, ooff, qt.shape[1])
    k = int(okoff[-1])
    assert np.array_equal(np_(koff), okoff), case
    assert np.array_equal(np_(qt)[:, :k], oqt[:, :k]) and np.array_equal(np_(st)[:, :k // 128], ost[:, :k // 128]), case

    # SwiGLU + quant and its FP8 cache, over the segments' rows
    h = (torch.randn((M_cap, 2 * F), generator=g) * 3).to(torch.bfloat16)
    q, s, hq, hs = fgb.swiglu_quant_cache(h.to(DEV), offs)
    sq, ss = O.swiglu_quant(bits(h), ooff)
    hq_o, hs_o = O.quant_rowwise(bits(h), 128)
    assert np.array_equal(np_(q)[:used], sq[:used]) and np.array_equal(np_(s)[:used], ss[:used]), case
    assert np.array_equal(np_(hq)[:used], hq_o[:used]) and np.array_equal(np_(hs)[:used], hs_o[:used]), case

    # SwiGLU backward from the cache
    da = (torch.randn((M_cap, F), generator=g) * 0.1).to(torch.bfloat16)
    dq, ds = fgb.dswiglu_quant(t(hq_o), t(hs_o), da.to(DEV), offs)
    dq_o, ds_o = O.dswiglu_quant(hq_o, hs_o, bits(da), ooff)
    assert np.array_equal(np_(dq)[:used], dq_o[:used]) and np.array_equal(np_(ds)[:used], ds_o[:used]), case

    # unpermute (probs-weighted) back to the tokens
    y = torch.randn((M_cap, H), generator=g).to(torch.bfloat16)
    out = fgb.unpermute_unpad(y.to(DEV), t(orm), t(probs))
    assert np.array_equal(np_(out), O.unpermute_unpad(bits(y), orm, probs)), case

    # unpermute backward fused with the 1x128 quant: every row of the padded layout
    dout = torch.randn((T, H), generator=g).to(torch.bfloat16)
    bq, bs = fgb.unpermute_backward_quant(dout.to(DEV), t(orm), t(probs), M_cap)
    bq_o, bs_o = O.quant_rowwise(O.unpermute_backward(bits(dout), orm, probs, M_cap), 128)
    assert np.array_equal(np_(bq), bq_o) and np.array_equal(np_(bs), bs_o), case


def test_random_moe_data_path(fgb):
    rng = np.random.default_rng(4242)
    for case in range(16):
        _case(fgb, rng, case)
