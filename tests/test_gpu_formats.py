"""GPU parity of the format variants against the CPU oracle on the same bytes:
E5M2 device encoding, the format/rule-aware quantizer and dequantizer, the
E5M2 direct transpose, the MX floor rule in the MOSS quantizer, the GEMM
with an E5M2 gradient operand, and the masked grouped GEMM.  Bit-exact for
codes and scales; GEMMs to the tolerance of the main parity suite."""
import numpy as np
import pytest
import torch

import oracle as O
import synth
from test_gpu_parity import DEV, MODES, _mode, check_gemm, np_, rand_codes, rand_scales, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def fgb():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import fine_grained_blockwise_amd as m
    return m


def bits(t):
    return t.contiguous().view(torch.int16).numpy().view(np.uint16)


def rand_e5m2(shape, seed):
    g = torch.Generator().manual_seed(seed)
    q = torch.randint(0, 256, shape, generator=g, dtype=torch.int32).to(torch.uint8)
    q[((q >> 2) & 31) == 31] ^= 0x04  # no Inf / NaN codes
    return q


# ---------------------------------------------------------------------------
def test_device_encode_e5m2_all_bf16_ties_and_sweep(fgb):
    say("encode E5M2: all bf16, every tie and neighbours, strided fp32 sweep")
    b = (np.arange(65536, dtype=np.uint32) << 16).view(np.float32)
    b = b[np.isfinite(b)]
    tab = O.fp8_decode_all(O.E5M2)
    mags = np.sort(np.unique(np.abs(tab[np.isfinite(tab)])))
    mids = ((mags[1:] + mags[:-1]) / 2).astype(np.float32)
    near = np.concatenate([mids, np.nextafter(mids, np.float32(0)), np.nextafter(mids, np.float32(1e9)),
                           mags.astype(np.float32)])
    lo = int(np.float32(2.0 ** -19).view(np.uint32))
    hi = int(np.float32(2.0 ** 16).view(np.uint32))
    sweep = np.arange(lo, hi, 7, dtype=np.uint32).view(np.float32)
    x = np.concatenate([b, near, -near, sweep, -sweep[::5],
                        np.float32([0.0, -0.0, 57344, 57345, 61440, 1e30, -1e30, 1e-45])]).astype(np.float32)
    got = np_(fgb.fgb_fp8_encode(torch.from_numpy(x).to(DEV), fgb.E5M2))
    assert np.array_equal(got, O.fp8_encode(x, O.E5M2))
    # E4M3 through the generic entry is the E4M3 encoder
    y = np.concatenate([b, near[:1000]]).astype(np.float32)
    assert np.array_equal(np_(fgb.fgb_fp8_encode(torch.from_numpy(y).to(DEV), fgb.E4M3)), O.e4m3_encode(y))


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("fmt,rule,group", [("e5m2", "ceil", 128), ("e5m2", "ceil", 32), ("e4m3", "floor", 32),
                                            ("e4m3", "floor", 128), ("e5m2", "floor", 32)])
@pytest.mark.parametrize("rows,cols", [(3, 384), (67, 1024), (257, 7168)])
def test_quant_rowwise_fmt(fgb, dtype, fmt, rule, group, rows, cols):
    say("quant_rowwise_fmt", dtype, fmt, rule, group, rows, cols)
    F = O.E5M2 if fmt == "e5m2" else O.E4M3
    R = O.SCALE_OCP_FLOOR if rule == "floor" else O.SCALE_CEIL
    g = torch.Generator().manual_seed(rows * 7 + cols + F * 3 + R)
    x = torch.randn(rows, cols, generator=g) * torch.exp2(torch.randint(-40, 20, (rows, 1), generator=g).float())
    x[0, :group] = 0.0
    x[-1, 3] = 1e-42  # a subnormal among normals
    x = x.to(dtype)
    q, s = fgb.fp8_quant_rowwise_fmt(x.to(DEV), group, F, R)
    xin = bits(x) if dtype == torch.bfloat16 else x.numpy()
    oq, os_ = O.quant_rowwise_fmt(xin, group, F, R)
    assert np.array_equal(np_(s), os_)
    assert np.array_equal(np_(q), oq)
    d = np_(fgb.fp8_dequant_fmt(q, s, fgb.ROW1x128 if group == 128 else fgb.ROW1x32, F))
    assert np.array_equal(d.astype(np.float64), O.dequant_fmt(oq, os_, group, F))


def test_quant_rowwise_e5m2_dsv3_grad(fgb):
    say("quant_rowwise_fmt: E5M2 dY [8192, 2048] of the DeepSeek-V3-shaped Linear")
    _, _, dY = synth.linear_dsv3(0)
    q, s = fgb.fp8_quant_rowwise_fmt(dY.to(DEV), 128, fgb.E5M2, fgb.SCALE_CEIL)
    oq, os_ = O.quant_rowwise_fmt(bits(dY), 128, O.E5M2, O.SCALE_CEIL)
    assert np.array_equal(np_(s), os_) and np.array_equal(np_(q), oq)


@pytest.mark.parametrize("T,C", [(128, 128), (384, 256), (32768, 2048)])
def test_direct_transpose_e5m2(fgb, T, C):
    say("direct transpose E5M2", T, C)
    q = rand_e5m2((T, C), T + C)
    s = rand_scales((T, C // 128), -29, 4, T + C + 1)
    qt, st = fgb.fp8_direct_transpose_fmt(q.to(DEV), s.to(DEV), fgb.E5M2)
    oqt, ost = O.direct_transpose_fmt(q.numpy(), s.numpy(), O.E5M2)
    assert np.array_equal(np_(st), ost)
    assert np.array_equal(np_(qt), oqt)


def test_mx2_floor_rule(fgb):
    for R, Cc, g1 in [(5, 1024 + 96, 512), (64, 28672, 10240)]:
        say("mx2 floor rule", R, Cc, g1)
        W, _ = synth.moss(seed=1, R=R, C=Cc, M=1)
        W[1, :g1] = 0.0
        q, s2, s1 = fgb.mx2_quant_rule(W.to(DEV), g1, fgb.SCALE_OCP_FLOOR)
        oq, os2, os1 = O.mx2_quant(bits(W), g1, O.SCALE_OCP_FLOOR)
        assert np.array_equal(np_(s1), os1) and np.array_equal(np_(s2), os2)
        assert np.array_equal(np_(q), oq)


# ---------------------------------------------------------------------------
def test_gemm_e5m2_conversion_is_exact(fgb):
    """Exact mode: with B the identity (code 1.0, scale 2^0), each output is one
    E5M2 value times its scale: every finite code at scales 2^-29..2^10 must come
    out exactly (the bf16 conversion of the matrix path)."""
    say("gemm E5M2: one-hot B, every code and scale")
    codes = np.array([c for c in range(256) if ((c >> 2) & 31) != 31], np.uint8)
    K = 256
    M = 40
    a = np.zeros((M, K), np.uint8)
    for r in range(M):
        a[r, :len(codes)] = codes  # 248 finite codes in the first 248 columns
    sa = np.array([[127 - 29 + r, 127 - 29 + r] for r in range(M)], np.uint8)
    b = np.zeros((K, K), np.uint8)
    b[np.arange(K), np.arange(K)] = 0x38  # E4M3 1.0
    sb = np.full((2, 2), 127, np.uint8)
    t = lambda x: torch.from_numpy(np.ascontiguousarray(x)).to(DEV)
    d = np_(fgb.fp8_block_gemm_fmt(t(a), t(sa), fgb.ROW1x128, fgb.E5M2, t(b), t(sb), fgb.BLOCK128, fgb.E4M3,
                                   out_dtype=torch.float32, mode=fgb.GEMM_EXACT))
    want = O.dequant_fmt(a, sa, 128, O.E5M2)
    assert np.array_equal(d.astype(np.float64), want)


@pytest.mark.parametrize("mode", MODES)
@pytest.mark.parametrize("bgran", ["block", "row"])
def test_gemm_e5m2_small(fgb, mode, bgran):
    say("gemm E5M2 A x E4M3 B, ragged", mode, bgran)
    M, N, K = 300, 320, 512
    a = rand_e5m2((M, K), 81)
    sa = rand_scales((M, K // 128), -20, -8, 82)  # gradient-like scales
    b = rand_codes((N, K), 83)
    if bgran == "block":
        sb = rand_scales(((N + 127) // 128, K // 128), -8, 2, 84)
        BG, OBG = fgb.BLOCK128, O.BLOCK128
    else:
        sb = rand_scales((N, K // 128), -8, 2, 84)
        BG, OBG = fgb.ROW1x128, O.ROW1x128
    d = np_(fgb.fp8_block_gemm_fmt(a.to(DEV), sa.to(DEV), fgb.ROW1x128, fgb.E5M2, b.to(DEV), sb.to(DEV), BG,
                                   fgb.E4M3, out_dtype=torch.float32, mode=_mode(fgb, mode)))
    mi, ni = np.repeat(np.arange(M), N), np.tile(np.arange(N), M)
    an, san, bn, sbn = a.numpy(), sa.numpy(), b.numpy(), sb.numpy()
    ref = O.block_gemm_fmt_sampled(an, san, O.ROW1x128, O.E5M2, bn, sbn, OBG, O.E4M3, mi, ni)
    bounds = None
    if mode == "fast":
        bounds = O.gemm_run_bounds_fmt_sampled(an, san, O.ROW1x128, O.E5M2, bn, sbn, OBG, O.E4M3, mi, ni)
    check_gemm(d.ravel(), ref, mode, False, bounds, K)


@pytest.mark.parametrize("mode", MODES)
def test_gemm_e5m2_dsv3_dgrad_sampled(fgb, mode):
    """Dgrad of the DeepSeek-V3-shaped Linear with an E5M2 gradient: dX = dY x W,
    A = dY [8192, 2048] (E5M2, 1x128), B = W^T [7168, 2048] (E4M3, 128x128)."""
    say("gemm E5M2 dgrad 8192x7168x2048, sampled", mode)
    X, W, dY = synth.linear_dsv3(0)
    gq, gs = O.quant_rowwise_fmt(bits(dY), 128, O.E5M2, O.SCALE_CEIL)
    wq, ws = O.quant_blockwise(bits(W))
    wqt, wst = np.ascontiguousarray(wq.T), np.ascontiguousarray(ws.T)
    t = lambda x: torch.from_numpy(np.ascontiguousarray(x)).to(DEV)
    d = np_(fgb.fp8_block_gemm_fmt(t(gq), t(gs), fgb.ROW1x128, fgb.E5M2, t(wqt), t(wst), fgb.BLOCK128, fgb.E4M3,
                                   out_dtype=torch.bfloat16, mode=_mode(fgb, mode)))
    rng = np.random.default_rng(2)
    mi = np.concatenate([rng.integers(0, 8192, 2000), [0, 8191]])
    ni = np.concatenate([rng.integers(0, 7168, 2000), [7167, 0]])
    ref = O.block_gemm_fmt_sampled(gq, gs, O.ROW1x128, O.E5M2, wqt, wst, O.BLOCK128, O.E4M3, mi, ni)
    bounds = None
    if mode == "fast":
        bounds = O.gemm_run_bounds_fmt_sampled(gq, gs, O.ROW1x128, O.E5M2, wqt, wst, O.BLOCK128, O.E4M3, mi, ni)
    check_gemm(d[mi, ni], ref, mode, True, bounds, 2048)


# ---------------------------------------------------------------------------
def _masked_ref(a, sa, b, sb, masked, gi, mi, ni):
    out = np.empty(len(gi))
    for g in np.unique(gi):
        sel = gi == g
        out[sel] = O.block_gemm_sampled(a[g], sa[g], O.ROW1x128, b[g], sb[g], O.BLOCK128, mi[sel], ni[sel])
    return out


def _masked_bounds(a, sa, b, sb, gi, mi, ni):
    rm, asum = np.zeros(len(gi)), np.zeros(len(gi))
    for g in np.unique(gi):
        sel = gi == g
        rm[sel], asum[sel] = O.gemm_run_bounds_sampled(a[g], sa[g], O.ROW1x128, b[g], sb[g], O.BLOCK128,
                                                       mi[sel], ni[sel])
    return rm, asum


@pytest.mark.parametrize("mode", MODES)
def test_grouped_gemm_masked_small(fgb, mode):
    say("masked grouped gemm: empty, partial, full and over-long masks", mode)
    G, M_max, N, K = 4, 300, 320, 512
    masked = np.array([0, 17, 300, 1000], np.int32)  # the last clamps to M_max
    a = rand_codes((G, M_max, K), 91)
    sa = rand_scales((G, M_max, K // 128), -6, 6, 92)
    b = rand_codes((G, N, K), 93)
    sb = rand_scales((G, (N + 127) // 128, K // 128), -6, 6, 94)
    d = torch.full((G, M_max, N), 7.0, dtype=torch.float32, device=DEV)
    fgb.fp8_grouped_gemm_masked(a.to(DEV), sa.to(DEV), b.to(DEV), sb.to(DEV), torch.from_numpy(masked).to(DEV), d=d,
                                mode=_mode(fgb, mode))
    got = np_(d)
    valid = np.minimum(masked, M_max)
    for g in range(G):
        assert np.all(got[g, valid[g]:] == 7.0)
    gi = np.concatenate([np.full(valid[g] * N, g) for g in range(G)])
    mi = np.concatenate([np.repeat(np.arange(valid[g]), N) for g in range(G)])
    ni = np.concatenate([np.tile(np.arange(N), valid[g]) for g in range(G)])
    an, san, bn, sbn = a.numpy(), sa.numpy(), b.numpy(), sb.numpy()
    ref = _masked_ref(an, san, bn, sbn, masked, gi, mi, ni)
    bounds = _masked_bounds(an, san, bn, sbn, gi, mi, ni) if mode == "fast" else None
    check_gemm(got[gi, mi, ni], ref, mode, False, bounds, K)


@pytest.mark.parametrize("mode", MODES)
def test_grouped_gemm_masked_every_valid_tile_count(fgb, mode):
    """Valid row counts that give each wave of a 256-row tile every count of
    valid 32-row tiles (0 to 4, the upper and lower 128 rows), with partial
    32-row tiles; every valid output checked, the rows past each mask untouched."""
    say("masked grouped gemm: 0-4 valid 32-row tiles per wave", mode)
    masked = np.array([32, 61, 96, 128, 129, 190, 224, 256], np.int32)
    G, M_max, N, K = masked.size, 256, 192, 384
    a = rand_codes((G, M_max, K), 111)
    sa = rand_scales((G, M_max, K // 128), -6, 6, 112)
    b = rand_codes((G, N, K), 113)
    sb = rand_scales((G, (N + 127) // 128, K // 128), -6, 6, 114)
    for bf16 in (False, True):
        fill = 7.0
        d = torch.full((G, M_max, N), fill, dtype=torch.bfloat16 if bf16 else torch.float32, device=DEV)
        fgb.fp8_grouped_gemm_masked(a.to(DEV), sa.to(DEV), b.to(DEV), sb.to(DEV), torch.from_numpy(masked).to(DEV),
                                    d=d, mode=_mode(fgb, mode))
        got = np_(d)  # fp32 values, or bf16 bit patterns
        untouched = np.uint16(0x40E0) if bf16 else np.float32(fill)  # 7.0
        for g in range(G):
            assert np.all(got[g, masked[g]:] == untouched), g
        gi = np.concatenate([np.full(masked[g] * N, g) for g in range(G)])
        mi = np.concatenate([np.repeat(np.arange(masked[g]), N) for g in range(G)])
        ni = np.concatenate([np.tile(np.arange(N), masked[g]) for g in range(G)])
        an, san, bn, sbn = a.numpy(), sa.numpy(), b.numpy(), sb.numpy()
        ref = _masked_ref(an, san, bn, sbn, masked, gi, mi, ni)
        bounds = _masked_bounds(an, san, bn, sbn, gi, mi, ni) if mode == "fast" else None
        check_gemm(got[gi, mi, ni], ref, mode, bf16, bounds, K)


@pytest.mark.parametrize("mode", MODES)
def test_grouped_gemm_masked_decode_sampled(fgb, mode):
    """Decode-shaped: 32 experts of fc1 (N=4096, K=7168), M_max = 512 rows each
    (a token reaches an expert at most once), valid counts from top-8 routing
    of 512 tokens."""
    say("masked grouped gemm: decode fc1 32 experts, sampled", mode)
    G, M_max, N, K = 32, 512, 4096, 7168
    idx, _ = synth.routing(512, G, 8, 1.1, 3)
    masked = np.bincount(idx.ravel(), minlength=G).astype(np.int32)
    a = rand_codes((G, M_max, K), 101)
    sa = rand_scales((G, M_max, K // 128), -8, 2, 102)
    b = rand_codes((G, N, K), 103)
    sb = rand_scales((G, N // 128, K // 128), -12, -4, 104)
    d = np_(fgb.fp8_grouped_gemm_masked(a.to(DEV), sa.to(DEV), b.to(DEV), sb.to(DEV),
                                        torch.from_numpy(masked).to(DEV), mode=_mode(fgb, mode)))
    rng = np.random.default_rng(4)
    gi = rng.integers(0, G, 1500)
    gi = gi[masked[gi] > 0]
    mi = (rng.integers(0, 1 << 30, gi.size) % masked[gi]).astype(np.int64)
    ni = rng.integers(0, N, gi.size)
    an, san, bn, sbn = a.numpy(), sa.numpy(), b.numpy(), sb.numpy()
    ref = _masked_ref(an, san, bn, sbn, masked, gi, mi, ni)
    bounds = _masked_bounds(an, san, bn, sbn, gi, mi, ni) if mode == "fast" else None
    check_gemm(d[gi, mi, ni], ref, mode, True, bounds, K)
