"""GPU parity at the workloads' full sizes, for the steps and shapes that the
smaller parity cases do not reach: the Linear's Dgrad and Wgrad at the
DeepSeek-V3 shapes, the Wgrad through the direct transpose contracting over
32768 tokens, the MOSS two-level quantization and its MX GEMM at the weight's
full shape, the fc2 expert GEMM, and the weight quantizer's transposed copy
for every expert.

Every oracle input is the seeded synthetic tensor itself (quantized by the
oracle where a step needs FP8 operands); the GPU runs on the same bytes, and
its own quantizers and transposes are checked bit for bit against the
oracle's.  GEMMs are compared on sampled outputs that include the corners and
the rows and columns on both sides of every 256-wide tile edge, to the
tolerance of the mode: max|d - ref| / max|ref| <= 1e-5 for FP32 output, one
bf16 ulp (or 1e-5 * max|ref|) for BF16 output in exact mode; the FP8
matrix unit's derived bound in fast mode."""
import functools
import sys

import numpy as np
import pytest
import torch

import oracle as O
import synth

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
MODES = ["exact", "fast"]


def say(*a):
    print("[case]", *a, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def fgb():
    import fine_grained_blockwise_amd as m
    return m


def np_(t):
    t = t.detach().cpu()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    return t.numpy()


def dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


def ulp_bf16(x):
    x = np.abs(np.asarray(x, np.float64))
    e = np.floor(np.log2(np.maximum(x, 2.0 ** -133)))
    return np.exp2(np.maximum(e, -133) - 7)


def check_gemm(got, ref, mode, bf16, bounds=None, K=None):
    if bf16:
        gv = torch.from_numpy(np.ascontiguousarray(got).view(np.int16)).view(torch.bfloat16).float().numpy()
        gv = gv.astype(np.float64)
    else:
        gv = np.asarray(got, np.float64)
    d = np.abs(gv - ref)
    if mode == "exact":
        if bf16:
            ok = (d <= ulp_bf16(ref)) | (d <= 1e-5 * np.max(np.abs(ref)))
            assert ok.all(), f"{(~ok).sum()} elements beyond 1 bf16 ulp; worst {d[~ok].max()}"
        else:
            err = d.max() / np.max(np.abs(ref))
            assert err <= 1e-5, f"max rel err {err:.3e}"
    else:
        rm, asum = bounds
        tol = 2.0 ** -10 * rm + (K / 8 + 4) * 2.0 ** -24 * asum
        if bf16:
            tol = tol + ulp_bf16(np.abs(ref) + tol)
        ok = d <= tol
        assert ok.all(), f"{(~ok).sum()} elements beyond the FP8-unit bound"
    return d.max() / max(np.max(np.abs(ref)), 1e-300)


def tile_edge_samples(M, N, n, seed, tile=256):
    """n random (m, n) pairs, the four corners, and the rows/columns on both
    sides of every tile edge (each paired with random partners)."""
    rng = np.random.default_rng(seed)
    me = np.unique(np.clip(np.concatenate([np.arange(tile, M, tile) - 1, np.arange(tile, M, tile),
                                           [0, M - 1]]), 0, M - 1))
    ne = np.unique(np.clip(np.concatenate([np.arange(tile, N, tile) - 1, np.arange(tile, N, tile),
                                           [0, N - 1]]), 0, N - 1))
    mi = np.concatenate([rng.integers(0, M, n), me, rng.integers(0, M, ne.size), [0, 0, M - 1, M - 1]])
    ni = np.concatenate([rng.integers(0, N, n), rng.integers(0, N, me.size), ne, [0, N - 1, 0, N - 1]])
    return mi.astype(np.int64), ni.astype(np.int64)


# ---------------------------------------------------------------------------
# DeepSeek-V3-shaped Linear: Dgrad (8192 x 7168 x 2048) and Wgrad (2048 x 7168 x 8192), BF16 out
# ---------------------------------------------------------------------------
@functools.lru_cache(maxsize=1)
def _dsv3_operands():
    X, W, dY = synth.linear_dsv3(0)
    xq, xs = O.quant_rowwise(synth.bf16_bits(X))
    wq, ws = O.quant_blockwise(synth.bf16_bits(W))
    gq, gs = O.quant_rowwise(synth.bf16_bits(dY))
    xqt, xst = O.direct_transpose(xq, xs)
    gqt, gst = O.direct_transpose(gq, gs)
    return dict(X=X, W=W, dY=dY, xq=xq, xs=xs, wq=wq, ws=ws, gq=gq, gs=gs, xqt=xqt, xst=xst, gqt=gqt, gst=gst)


def test_dsv3_linear_quant_and_transposes_full(fgb):
    say("DeepSeek-V3 Linear: GPU quantizers and direct transposes at full size vs the oracle")
    o = _dsv3_operands()
    gq, gs = fgb.fp8_quant_rowwise(o["dY"].to(DEV))
    assert np.array_equal(np_(gq), o["gq"]) and np.array_equal(np_(gs), o["gs"])
    wq, ws = fgb.fp8_quant_blockwise(o["W"].to(DEV))
    assert np.array_equal(np_(wq), o["wq"]) and np.array_equal(np_(ws), o["ws"])
    for q, s, qt, st in [("xq", "xs", "xqt", "xst"), ("gq", "gs", "gqt", "gst")]:
        gt, gst = fgb.fp8_direct_transpose(dev(o[q]), dev(o[s]))
        assert np.array_equal(np_(gst), o[st]) and np.array_equal(np_(gt), o[qt]), q


@pytest.mark.parametrize("mode", MODES)
@pytest.mark.parametrize("which", ["dgrad", "wgrad"])
def test_dsv3_linear_dgrad_wgrad_full_sampled(fgb, which, mode):
    o = _dsv3_operands()
    if which == "dgrad":  # dX [8192, 7168] = dY [8192, 2048] . W [2048, 7168]: B = W^T, 128x128 blocks
        a, sa, ag = o["gq"], o["gs"], O.ROW1x128
        b, sb, bg = o["wq"].T.copy(), o["ws"].T.copy(), O.BLOCK128
    else:  # dW [2048, 7168] = dY^T . X, both direct-transposed, 1x128 scales on both sides
        a, sa, ag = o["gqt"], o["gst"], O.ROW1x128
        b, sb, bg = o["xqt"], o["xst"], O.ROW1x128
    M, K = a.shape
    N = b.shape[0]
    say(f"DeepSeek-V3 Linear {which} {M}x{N}x{K}, bf16 out, sampled", mode)
    d = np_(fgb.fp8_block_gemm(dev(a), dev(sa), ag, dev(b), dev(sb), bg, out_dtype=torch.bfloat16,
                               mode=fgb.GEMM_EXACT if mode == "exact" else fgb.GEMM_FAST))
    mi, ni = tile_edge_samples(M, N, 3000, 11)
    ref = O.block_gemm_sampled(a, sa, ag, b, sb, bg, mi, ni)
    bounds = O.gemm_run_bounds_sampled(a, sa, ag, b, sb, bg, mi, ni) if mode == "fast" else None
    err = check_gemm(d[mi, ni], ref, mode, True, bounds, K)
    say("   max|d|/max|ref|", err)


# ---------------------------------------------------------------------------
# Wgrad through the direct transpose: X, dY codes [32768, 7168], [32768, 2048], K = 32768, FP32 out
# ---------------------------------------------------------------------------
@functools.lru_cache(maxsize=1)
def _wgrad_operands():
    xq, xs = synth.wgrad_codes(32768, 7168, 0, 41)
    gq, gs = synth.wgrad_codes(32768, 2048, 0, 42)
    xqt, xst = O.direct_transpose(xq.numpy(), xs.numpy())
    gqt, gst = O.direct_transpose(gq.numpy(), gs.numpy())
    return xq, xs, gq, gs, xqt, xst, gqt, gst


def test_wgrad_k32768_transposes_full(fgb):
    say("Wgrad path: GPU direct transposes of X [32768, 7168] and dY [32768, 2048] in full vs the oracle")
    xq, xs, gq, gs, xqt, xst, gqt, gst = _wgrad_operands()
    t, st = fgb.fp8_direct_transpose(xq.to(DEV), xs.to(DEV))
    assert np.array_equal(np_(st), xst) and np.array_equal(np_(t), xqt)
    t, st = fgb.fp8_direct_transpose(gq.to(DEV), gs.to(DEV))
    assert np.array_equal(np_(st), gst) and np.array_equal(np_(t), gqt)


@pytest.mark.parametrize("mode", MODES)
def test_wgrad_k32768_fp32_full_sampled(fgb, mode):
    say("Wgrad 2048x7168x32768 on the direct-transposed codes, FP32 out, sampled", mode)
    _, _, _, _, xqt, xst, gqt, gst = _wgrad_operands()
    d = np_(fgb.fp8_block_gemm(dev(gqt), dev(gst), fgb.ROW1x128, dev(xqt), dev(xst), fgb.ROW1x128,
                               out_dtype=torch.float32, mode=fgb.GEMM_EXACT if mode == "exact" else fgb.GEMM_FAST))
    mi, ni = tile_edge_samples(2048, 7168, 1500, 12)
    ref = O.block_gemm_sampled(gqt, gst, O.ROW1x128, xqt, xst, O.ROW1x128, mi, ni)
    bounds = O.gemm_run_bounds_sampled(gqt, gst, O.ROW1x128, xqt, xst, O.ROW1x128, mi, ni) if mode == "fast" else None
    err = check_gemm(d[mi, ni], ref, mode, False, bounds, 32768)
    say("   max|d|/max|ref|", err)


# ---------------------------------------------------------------------------
# MOSS: two-level quantization of W [8192, 28672] and of W^T [28672, 8192]; MX GEMM 4096 x 28672 x 8192
# ---------------------------------------------------------------------------
@functools.lru_cache(maxsize=1)
def _moss_operands():
    W, A = synth.moss(0)
    Wt = W.t().contiguous()
    return W, Wt, A


@pytest.mark.parametrize("layout", ["W [8192, 28672]", "W^T [28672, 8192]"])
def test_mx2_quant_dequant_full(fgb, layout):
    say("MOSS mx2_quant at full size, layout", layout)
    W, Wt, _ = _moss_operands()
    x = W if layout.startswith("W [") else Wt
    q, s2, s1 = fgb.mx2_quant(x.to(DEV), 10240)
    oq, os2, os1 = O.mx2_quant(synth.bf16_bits(x), 10240)
    assert np.array_equal(np_(s1).view(np.uint32), os1.view(np.uint32))
    assert np.array_equal(np_(s2), os2)
    assert np.array_equal(np_(q), oq)
    # dequantization of a band of rows (every level-1 group of them), fp32 bit for bit
    rows = slice(0, 256)
    xh = np_(fgb.mx2_dequant(q[rows].contiguous(), s2[rows].contiguous(), s1[rows].contiguous(), 10240))
    oxh = O.mx2_dequant(oq[rows], os2[rows], os1[rows], 10240)
    assert np.array_equal(xh.view(np.uint32), oxh.view(np.uint32))
    xf = (synth.bf16_bits(x[rows]).astype(np.uint32) << 16).view(np.float32)
    snr = O.snr_db(xf, oxh)
    say(f"   SNR of rows 0-255: {snr:.3f} dB")
    assert snr > 25.0


@pytest.mark.parametrize("mode", MODES)
def test_moss_mx_gemm_full_sampled(fgb, mode):
    say("MOSS MX GEMM 4096x28672x8192: 1x32 A, two-level W^T with the level-1 factor, FP32 out, sampled", mode)
    _, Wt, A = _moss_operands()
    bq, bs2, bs1 = O.mx2_quant(synth.bf16_bits(Wt), 10240)  # one level-1 group per row (K = 8192)
    aq, as_ = O.quant_rowwise(synth.bf16_bits(A), 32)
    l1 = np.ascontiguousarray(bs1[:, 0])
    d = np_(fgb.fp8_block_gemm(dev(aq), dev(as_), fgb.ROW1x32, dev(bq), dev(bs2), fgb.ROW1x32, b_l1=dev(l1),
                               g1=10240, out_dtype=torch.float32,
                               mode=fgb.GEMM_EXACT if mode == "exact" else fgb.GEMM_FAST))
    mi, ni = tile_edge_samples(4096, 28672, 2000, 13)
    ref = O.block_gemm_sampled(aq, as_, O.ROW1x32, bq, bs2, O.ROW1x32, mi, ni, b_l1=bs1, g1=10240)
    bounds = (O.gemm_run_bounds_sampled(aq, as_, O.ROW1x32, bq, bs2, O.ROW1x32, mi, ni, b_l1=l1)
              if mode == "fast" else None)
    err = check_gemm(d[mi, ni], ref, mode, False, bounds, 8192)
    say("   max|d|/max|ref|", err)


# ---------------------------------------------------------------------------
# MoE: fc2 (N = 7168, K = 2048) over the 32 experts; the expert weights' transposed copies
# ---------------------------------------------------------------------------
def _moe_offsets(T=16384, G=32):
    idx, _ = synth.routing(T, G, 8, 1.1, 0)
    counts = np.bincount(idx.ravel(), minlength=G)
    off = np.concatenate([[0], np.cumsum((counts + 15) // 16 * 16)]).astype(np.int32)
    return off, T * 8 + 15 * G


def _codes(shape, seed):
    g = torch.Generator().manual_seed(seed)
    q = torch.randint(0, 256, shape, generator=g, dtype=torch.int32).to(torch.uint8)
    q[(q & 0x7F) == 0x7F] ^= 1
    return q


def _scales(shape, lo, hi, seed):
    g = torch.Generator().manual_seed(seed)
    return torch.randint(lo + 127, hi + 128, shape, generator=g, dtype=torch.int32).to(torch.uint8)


@pytest.mark.parametrize("mode", MODES)
def test_grouped_gemm_moe_fc2_sampled(fgb, mode):
    say("grouped gemm: fc2 of the 32-expert layer (N=7168, K=2048), sampled at segment and tile edges", mode)
    G, N, K = 32, 7168, 2048
    off, M_cap = _moe_offsets()
    a, sa = _codes((M_cap, K), 61), _scales((M_cap, K // 128), -6, 2, 62)
    b, sb = _codes((G, N, K), 63), _scales((G, N // 128, K // 128), -12, -4, 64)
    d = np_(fgb.fp8_grouped_gemm(a.to(DEV), sa.to(DEV), b.to(DEV), sb.to(DEV), dev(off),
                                 mode=fgb.GEMM_EXACT if mode == "exact" else fgb.GEMM_FAST))
    rng = np.random.default_rng(14)
    mi = np.concatenate([rng.integers(0, off[G], 3000), off[1:G] - 1, off[:G], off[:G] + 255, off[:G] + 256])
    mi = mi[mi < off[G]]
    ni = np.concatenate([rng.integers(0, N, mi.size - 64), np.repeat([0, 255, 256, N - 1], 16)])
    assert ni.size == mi.size
    an, san, bn, sbn = a.numpy(), sa.numpy(), b.numpy(), sb.numpy()
    ref = O.grouped_gemm_sampled(an, san, bn, sbn, off, mi, ni)
    bounds = None
    if mode == "fast":
        rm, asum = np.zeros(mi.size), np.zeros(mi.size)
        for g in range(G):
            sel = (mi >= off[g]) & (mi < off[g + 1])
            if sel.any():
                rm[sel], asum[sel] = O.gemm_run_bounds_sampled(an, san, O.ROW1x128, bn[g], sbn[g], O.BLOCK128,
                                                               mi[sel], ni[sel])
        bounds = (rm, asum)
    err = check_gemm(d[mi, ni], ref, mode, True, bounds, K)
    say("   max|d|/max|ref|", err)


def test_quant_blockwise_t_every_expert(fgb):
    say("quant_blockwise_t: all 32 experts of W2 [32, 7168, 2048] (bf16 N(0, 0.02))")
    W2 = synth.normal((32, 7168, 2048), 0.02, 0, 33, "cpu", torch.bfloat16)
    q, s, qt, st = fgb.fp8_quant_blockwise_t(W2.to(DEV))
    q, s, qt, st = np_(q), np_(s), np_(qt), np_(st)
    for e in range(32):
        oq, os_ = O.quant_blockwise(synth.bf16_bits(W2[e]))
        oqt, ost = O.block_transpose(oq, os_)
        assert np.array_equal(s[e], os_) and np.array_equal(q[e], oq), e
        assert np.array_equal(st[e], ost) and np.array_equal(qt[e], oqt), e
