"""More experts than one wave has lanes (G = 65, 130, 257): the device-side
expert lookups read the group offsets 64 experts per pass, so these cases
take the multi-pass paths of permute + pad, the M-grouped, masked and
K-grouped GEMMs, the direct transpose of expert segments and SwiGLU + quant,
each checked against the oracle (data movement bit for bit, GEMMs to the
exact mode's tolerance).  About a tenth of the experts receive no token."""
import numpy as np
import pytest
import torch

import oracle as O
from test_gpu_parity import DEV, bits, check_gemm, np_, rand_codes, rand_scales, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def fgb():
    import fine_grained_blockwise_amd as m
    return m


@pytest.mark.parametrize("G", [65, 130, 257])
def test_many_experts(fgb, G):
    rng = np.random.default_rng(G)
    T, topk, H, F, N = 700, 4, 256, 128, 320
    M_cap = T * topk + 15 * G
    say(f"{G} experts: T={T} top-{topk} H={H} F={F} N={N}")
    live = np.sort(rng.choice(G, G - G // 10, replace=False))  # the rest get no token
    idx = np.stack([rng.choice(live, topk, replace=False) for _ in range(T)]).astype(np.int32)
    idx[rng.random(idx.shape) < 0.05] = -1
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(DEV)
    xq, xs = rand_codes((T, H), G + 1).numpy(), rand_scales((T, H // 128), -12, 4, G + 2).numpy()

    # permute + pad
    pq, ps, rmap, offs = fgb.permute_pad(t(xq), t(xs), t(idx), G, 16, M_cap)
    oq, os_, orm, ooff, used = O.permute_pad(xq, xs, idx, G, 16, M_cap)
    assert np.array_equal(np_(offs), ooff) and np.array_equal(np_(rmap), orm)
    assert np.array_equal(np_(pq)[:used], oq[:used]) and np.array_equal(np_(ps)[:used], os_[:used])
    assert int(np.sum(np.diff(ooff) == 0)) >= G // 10  # the empty experts

    # M-grouped GEMM over the segments, every output row of every segment
    b = rand_codes((G, N, H), G + 3).numpy()
    sb = rand_scales((G, (N + 127) // 128, H // 128), -6, 6, G + 4).numpy()
    d = fgb.fp8_grouped_gemm(t(oq), t(os_), t(b), t(sb), t(ooff), out_dtype=torch.float32)
    mi, ni = np.repeat(np.arange(used), N), np.tile(np.arange(N), used)
    ref = O.grouped_gemm_sampled(oq, os_, b, sb, ooff, mi, ni).reshape(used, N)
    check_gemm(np_(d)[:used], ref, "exact", False, None, H)

    # masked layout, G experts of up to 64 rows
    M_max = 64
    masked = rng.integers(0, M_max + 1, G).astype(np.int32)
    masked[rng.choice(G, G // 10, replace=False)] = 0
    a3 = rand_codes((G, M_max, H), G + 5).numpy()
    sa3 = rand_scales((G, M_max, H // 128), -6, 6, G + 6).numpy()
    dm = torch.full((G, M_max, N), 7.0, dtype=torch.float32, device=DEV)
    fgb.fp8_grouped_gemm_masked(t(a3), t(sa3), t(b), t(sb), t(masked), d=dm)
    got = np_(dm)
    for g in range(G):
        assert np.all(got[g, masked[g]:] == np.float32(7.0)), g
        if masked[g]:
            mi, ni = np.repeat(np.arange(masked[g]), N), np.tile(np.arange(N), masked[g])
            r = O.block_gemm_sampled(a3[g], sa3[g], O.ROW1x128, b[g], sb[g], O.BLOCK128, mi, ni)
            check_gemm(got[g, :masked[g]].ravel(), r, "exact", False, None, H)

    # direct transpose of the segments, then the K-grouped GEMM on their K ranges
    qt, st, koff = fgb.fp8_grouped_direct_transpose(t(oq), t(os_), t(ooff))
    oqt, ost, okoff = O.grouped_direct_transpose(oq, os_, ooff, qt.shape[1])
    k = int(okoff[-1])
    assert np.array_equal(np_(koff), okoff)
    assert np.array_equal(np_(qt)[:, :k], oqt[:, :k]) and np.array_equal(np_(st)[:, :k // 128], ost[:, :k // 128])
    Mw = 192
    aw = rand_codes((Mw, qt.shape[1]), G + 7).numpy()
    saw = rand_scales((Mw, qt.shape[1] // 128), -6, 6, G + 8).numpy()
    dw = np_(fgb.fp8_kgrouped_gemm(t(aw), t(saw), qt, st, koff))  # D_e [Mw, H]
    empty = np.diff(okoff) == 0
    assert np.all(dw[empty] == 0.0)
    s = 4000
    ei, mi, ni = rng.integers(0, G, s), rng.integers(0, Mw, s), rng.integers(0, H, s)
    ref = O.kgrouped_gemm_sampled(aw, saw, oqt, ost, okoff, ei, mi, ni)
    check_gemm(dw[ei, mi, ni], ref, "exact", False, None, None)

    # SwiGLU + quant over the segments
    h = (torch.randn((M_cap, 2 * F), generator=torch.Generator().manual_seed(G + 9)) * 3).to(torch.bfloat16)
    q, s_ = fgb.swiglu_quant(h.to(DEV), t(ooff))
    sq, ss = O.swiglu_quant(bits(h), ooff)
    assert np.array_equal(np_(q)[:used], sq[:used]) and np.array_equal(np_(s_)[:used], ss[:used])
