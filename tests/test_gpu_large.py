"""Tensors past 2^32 bytes: every kernel indexes with 64-bit offsets, so an
entry point given a tensor of more than 4 GiB must address its far end
correctly.  Each case builds one such tensor on the device and checks rows
or 128x128 blocks at both ends (and one in the middle) against the oracle
run on just those rows or blocks (each op is row- or block-local): the
row-wise quantizer, the direct transpose, a GEMM whose output passes 4 GiB,
and permute + pad / unpermute through a padded expert layout of over 4 GiB."""
import numpy as np
import pytest
import torch

import oracle as O
from test_gpu_parity import DEV, bits, check_gemm, np_, say

pytestmark = pytest.mark.gpu
GiB4 = 1 << 32


@pytest.fixture(scope="module")
def fgb():
    import fine_grained_blockwise_amd as m
    return m


def _codes_dev(shape, seed):
    g = torch.Generator(device=DEV)
    g.manual_seed(seed)
    q = torch.randint(0, 256, shape, generator=g, dtype=torch.uint8, device=DEV)
    q ^= ((q & 0x7F) == 0x7F).to(torch.uint8)  # no NaN codes (elementwise: masked writes fail past 2^32 elements)
    return q


def _ends(n, k):
    """k indices at the start, k in the middle and k at the end of range(n)."""
    return np.unique(np.concatenate([np.arange(k), n // 2 + np.arange(k), n - k + np.arange(k)]))


def test_quant_rowwise_past_4gib(fgb):
    R, C = (1 << 19) + 37, 8192
    say("quant_rowwise past 4 GiB:", R, C)
    g = torch.Generator(device=DEV)
    g.manual_seed(1)
    x = torch.randn((R, C), generator=g, device=DEV, dtype=torch.bfloat16)
    assert x.numel() * 2 > GiB4
    q, s = fgb.fp8_quant_rowwise(x)
    rows = torch.from_numpy(_ends(R, 48)).to(DEV)
    oq, os_ = O.quant_rowwise(bits(x[rows].cpu()), 128)
    assert np.array_equal(np_(q[rows]), oq) and np.array_equal(np_(s[rows]), os_)
    del x, q, s
    torch.cuda.empty_cache()


def test_direct_transpose_past_4gib(fgb):
    T, C = 1 << 20, 33 * 128
    say("direct transpose past 4 GiB:", T, C)
    q = _codes_dev((T, C), 2)
    assert q.numel() > GiB4
    g = torch.Generator(device=DEV)
    g.manual_seed(3)
    s = torch.randint(127 - 20, 127 + 5, (T, C // 128), generator=g, dtype=torch.uint8, device=DEV)
    qt, st = fgb.fp8_direct_transpose(q, s)
    ntb, ncb = T // 128, C // 128
    for tb, cb in ((0, 0), (ntb // 2, ncb // 2), (ntb - 1, ncb - 1), (ntb - 1, 0), (0, ncb - 1)):
        r, c = slice(tb * 128, (tb + 1) * 128), slice(cb * 128, (cb + 1) * 128)
        oqt, ost = O.direct_transpose(np_(q[r, c]), np_(s[r, cb:cb + 1]))
        assert np.array_equal(np_(qt[c, r]), oqt), (tb, cb)
        assert np.array_equal(np_(st[c, tb:tb + 1]), ost), (tb, cb)
    del q, s, qt, st
    torch.cuda.empty_cache()


def test_gemm_output_past_4gib(fgb):
    M, N, K = (1 << 21) + 5, 1152, 256
    say("gemm with a bf16 output past 4 GiB:", M, N, K)
    a = _codes_dev((M, K), 4)
    g = torch.Generator(device=DEV)
    g.manual_seed(5)
    sa = torch.randint(127 - 6, 127 + 6, (M, K // 128), generator=g, dtype=torch.uint8, device=DEV)
    b = _codes_dev((N, K), 6)
    sb = torch.randint(127 - 6, 127 + 6, ((N + 127) // 128, K // 128), generator=g, dtype=torch.uint8, device=DEV)
    d = fgb.fp8_block_gemm(a, sa, fgb.ROW1x128, b, sb, fgb.BLOCK128)
    assert d.numel() * 2 > GiB4
    rows = _ends(M, 24)
    mi, ni = np.repeat(np.arange(len(rows)), N), np.tile(np.arange(N), len(rows))
    ref = O.block_gemm_sampled(np_(a[torch.from_numpy(rows).to(DEV)]), np_(sa[torch.from_numpy(rows).to(DEV)]),
                               O.ROW1x128, np_(b), np_(sb), O.BLOCK128, mi, ni)
    check_gemm(np_(d[torch.from_numpy(rows).to(DEV)]).ravel(), ref, "exact", True, None, K)
    del a, sa, b, sb, d
    torch.cuda.empty_cache()


def test_permute_unpermute_past_4gib(fgb):
    T, topk, G, H = 1 << 19, 8, 64, 1152
    M_cap = T * topk + 15 * G
    say("permute_pad / unpermute through a padded layout past 4 GiB:", T, topk, G, H)
    assert M_cap * H > GiB4
    rng = np.random.default_rng(7)
    idx = np.argsort(rng.random((T, G)), axis=1)[:, :topk].astype(np.int32)
    idx[rng.random(idx.shape) < 0.02] = -1
    xq = _codes_dev((T, H), 8)
    g = torch.Generator(device=DEV)
    g.manual_seed(9)
    xs = torch.randint(127 - 20, 127 + 4, (T, H // 128), generator=g, dtype=torch.uint8, device=DEV)
    pq, ps, rmap, offs = fgb.permute_pad(xq, xs, torch.from_numpy(idx).to(DEV), G, 16, M_cap)
    # the layout itself (offsets and row map) from the oracle on one 128-column block of zeros
    z = np.zeros((T, 128), np.uint8)
    _, _, orm, ooff, used = O.permute_pad(z, z[:, :1], idx, G, 16, M_cap)
    assert np.array_equal(np_(offs), ooff) and np.array_equal(np_(rmap), orm)
    # sampled tokens: their copies land on the rows the map names
    toks = _ends(T, 32)
    src_q, src_s = np_(xq[torch.from_numpy(toks).to(DEV)]), np_(xs[torch.from_numpy(toks).to(DEV)])
    for i, t in enumerate(toks):
        for k in range(topk):
            r = int(orm[t, k])
            if r >= 0:
                assert np.array_equal(np_(pq[r]), src_q[i]) and np.array_equal(np_(ps[r]), src_s[i]), (t, k)
    # padding rows at the end of the last segments: code 0, scale byte 105
    counts = np.bincount(idx[idx >= 0], minlength=G)
    for e in (G - 2, G - 1):
        lo, hi = int(ooff[e]) + int(counts[e]), int(ooff[e + 1])
        if hi > lo:
            assert np.all(np_(pq[lo:hi]) == 0) and np.all(np_(ps[lo:hi]) == 105), e
    del pq, ps, xq, xs
    torch.cuda.empty_cache()
    # unpermute: expert outputs of the padded layout back to the tokens, probs-weighted
    probs = rng.random((T, topk)).astype(np.float32)
    g.manual_seed(10)
    y = torch.randn((M_cap, H), generator=g, device=DEV, dtype=torch.bfloat16)
    assert y.numel() * 2 > GiB4
    out = fgb.unpermute_unpad(y, rmap, torch.from_numpy(probs).to(DEV))
    sub_rm = orm[toks]
    rows = np.unique(sub_rm[sub_rm >= 0])
    remap = np.full(M_cap, -1, np.int64)
    remap[rows] = np.arange(len(rows))
    y_sub = bits(y[torch.from_numpy(rows).to(DEV)].cpu())
    rm_sub = np.where(sub_rm >= 0, remap[np.maximum(sub_rm, 0)], -1).astype(np.int32)
    ref = O.unpermute_unpad(y_sub, rm_sub, probs[toks])
    assert np.array_equal(np_(out[torch.from_numpy(toks).to(DEV)]), ref)
    del y, out
    torch.cuda.empty_cache()
