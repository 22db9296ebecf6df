"""GPU parity: every HIP entry point against the CPU oracle on the same bytes.

Bit-exact for codes, scales, data movement and the bf16 unpermute fold; GEMMs
within max|d - ref| / max|ref| <= 1e-5 (FP32 output) or, elementwise, one bf16
ulp of |ref| or 1e-5 * max|ref| (BF16 output)."""
import functools
import sys

import numpy as np
import pytest
import torch

import oracle as O
import synth

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


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


def bits(t):
    """bf16 CPU tensor -> uint16 numpy bits."""
    return t.contiguous().view(torch.int16).numpy().view(np.uint16)


def ulp_bf16(x):
    x = np.abs(np.asarray(x, np.float64))
    e = np.floor(np.log2(np.maximum(x, 2.0 ** -133)))
    return np.exp2(np.maximum(e, -133) - 7)


def check_fp32(got, ref, tol=1e-5):
    got = np.asarray(got, np.float64)
    scale = np.max(np.abs(ref))
    err = np.max(np.abs(got - ref)) / scale if scale > 0 else np.max(np.abs(got))
    assert err <= tol, f"max rel err {err:.3e}"
    return err


def rand_codes(shape, seed):
    g = torch.Generator().manual_seed(seed)
    q = torch.randint(0, 256, shape, generator=g, dtype=torch.int32).to(torch.uint8)
    q[(q & 0x7F) == 0x7F] ^= 1  # no NaN codes
    return q


def rand_scales(shape, lo, hi, seed):
    g = torch.Generator().manual_seed(seed)
    return torch.randint(lo + 127, hi + 128, shape, generator=g, dtype=torch.int32).to(torch.uint8)


# ---------------------------------------------------------------------------
# E4M3 device conversion
# ---------------------------------------------------------------------------
def test_device_encode_all_bf16_and_ties(fgb):
    say("encode: all bf16, every tie and neighbours")
    b = (np.arange(65536, dtype=np.uint32) << 16).view(np.float32)
    b = b[np.isfinite(b)]
    tab = O.e4m3_decode_table()
    mags = np.sort(np.unique(np.abs(tab[np.isfinite(tab)])))
    mids = ((mags[1:] + mags[:-1]) / 2).astype(np.float32)
    near = np.concatenate([mids, np.nextafter(mids, np.float32(0)), np.nextafter(mids, np.float32(1e9)),
                           mags.astype(np.float32)])
    x = np.concatenate([b, near, -near, np.float32([0.0, -0.0, 448, 449, 500, -1e30, 1e-40, -1e-40])])
    x = x.astype(np.float32)
    got = np_(fgb.fgb_e4m3_encode(torch.from_numpy(x).to(DEV)))
    assert np.array_equal(got, O.e4m3_encode(x))


def test_device_encode_dense_fp32_range(fgb):
    say("encode: strided sweep of fp32 in [2^-12, 2^9]")
    lo = int(np.float32(2.0 ** -12).view(np.uint32))
    hi = int(np.float32(2.0 ** 9).view(np.uint32))
    bitsv = np.arange(lo, hi, 5, dtype=np.uint32)
    x = bitsv.view(np.float32)
    x = np.concatenate([x, -x[::7]])
    got = np_(fgb.fgb_e4m3_encode(torch.from_numpy(x).to(DEV)))
    assert np.array_equal(got, O.e4m3_encode(x))


# ---------------------------------------------------------------------------
# 1 x g quantization
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("group", [128, 32])
@pytest.mark.parametrize("rows,cols", [(1, 128), (3, 384), (67, 1024), (257, 7168)])
def test_quant_rowwise_small(fgb, dtype, group, rows, cols):
    say("quant_rowwise", dtype, group, rows, cols)
    g = torch.Generator().manual_seed(rows * 31 + cols)
    x = torch.randn(rows, cols, generator=g) * torch.exp2(torch.randint(-30, 30, (rows, 1), generator=g).float())
    x[0, :group] = 0.0
    if rows > 2:
        x[1, :group] = -0.0
        x[2, :min(cols, 256)] *= 1e-38  # subnormal fp32 / bf16 values
    x = x.to(dtype)
    q, s = fgb.fp8_quant_rowwise(x.to(DEV), group)
    xr = bits(x) if dtype == torch.bfloat16 else x.numpy()
    oq, os_ = O.quant_rowwise(xr, group)
    assert np.array_equal(np_(q), oq) and np.array_equal(np_(s), os_)


def test_quant_rowwise_strided_ld(fgb):
    say("quant_rowwise ld != cols")
    x = torch.randn(100, 1024).to(torch.bfloat16)
    xs = x[:, :640]
    q = torch.full((100, 768), 0xAA, dtype=torch.uint8, device=DEV)
    s = torch.full((100, 9), 0xAA, dtype=torch.uint8, device=DEV)
    fgb.fp8_quant_rowwise(x.to(DEV)[:, :640], 128, q[:, :640], s[:, :5])
    oq, os_ = O.quant_rowwise(bits(xs.contiguous()), 128)
    assert np.array_equal(np_(q)[:, :640], oq) and np.all(np_(q)[:, 640:] == 0xAA)
    assert np.array_equal(np_(s)[:, :5], os_) and np.all(np_(s)[:, 5:] == 0xAA)


def test_quant_linear_tiny(fgb):
    say("quant: tiny linear X, dY (fp32), W (fp32 blocks)")
    X, W, dY = synth.linear_tiny(0)
    for t in (X, dY):
        q, s = fgb.fp8_quant_rowwise(t.to(DEV))
        oq, os_ = O.quant_rowwise(t.numpy())
        assert np.array_equal(np_(q), oq) and np.array_equal(np_(s), os_)
    q, s = fgb.fp8_quant_blockwise(W.to(DEV))
    oq, os_ = O.quant_blockwise(W.numpy())
    assert np.array_equal(np_(q), oq) and np.array_equal(np_(s), os_)


def test_quant_dsv3_full(fgb):
    say("quant: DeepSeek-V3 X [8192, 7168] bf16 rowwise, W [2048, 7168] blockwise")
    X, W, dY = synth.linear_dsv3(0)
    q, s = fgb.fp8_quant_rowwise(X.to(DEV))
    oq, os_ = O.quant_rowwise(bits(X))
    assert np.array_equal(np_(s), os_)
    assert np.array_equal(np_(q), oq)
    q, s = fgb.fp8_quant_blockwise(W.to(DEV))
    oq, os_ = O.quant_blockwise(bits(W))
    assert np.array_equal(np_(q), oq) and np.array_equal(np_(s), os_)


@pytest.mark.parametrize("rows", [1, 100, 2112])
def test_quant_blockwise_partial(fgb, rows):
    say("quant_blockwise rows", rows)
    g = torch.Generator().manual_seed(rows)
    w = (torch.randn(rows, 512, generator=g) * 0.02).to(torch.bfloat16)
    q, s = fgb.fp8_quant_blockwise(w.to(DEV))
    oq, os_ = O.quant_blockwise(bits(w))
    assert np.array_equal(np_(q), oq) and np.array_equal(np_(s), os_)


def test_dequant(fgb):
    say("dequant")
    q = rand_codes((256, 512), 1)
    for gran, sshape in [(fgb.ROW1x128, (256, 4)), (fgb.ROW1x32, (256, 16)), (fgb.BLOCK128, (2, 4))]:
        s = rand_scales(sshape, -40, 40, 2)
        ref = O.dequant(q.numpy(), s.numpy(), gran)
        out = np_(fgb.fp8_dequant(q.to(DEV), s.to(DEV), gran, torch.float32))
        assert np.array_equal(out.astype(np.float64), ref)


# ---------------------------------------------------------------------------
# direct transpose
# ---------------------------------------------------------------------------
def test_transpose_exhaustive_codes_and_shifts(fgb):
    say("transpose: 256 codes x k in 0..127")
    q = torch.arange(256, dtype=torch.int32).to(torch.uint8).repeat(256, 1)  # [256 rows, 256 cols]
    s = torch.zeros((256, 2), dtype=torch.uint8)
    for t in range(256):
        k = t % 128
        s[t, :] = 240 - k
    qt, st = fgb.fp8_direct_transpose(q.to(DEV), s.to(DEV))
    oqt, ost = O.direct_transpose(q.numpy(), s.numpy())
    nan = np.isin(np.arange(256), [0x7F, 0xFF])
    assert np.array_equal(np_(qt)[~nan], oqt[~nan])
    assert np.array_equal(np_(st), ost)


@pytest.mark.parametrize("T,C", [(128, 128), (256, 512), (384, 2048), (1280, 384), (2176, 256)])
def test_transpose_random(fgb, T, C):
    say("transpose", T, C)
    q, s = synth.wgrad_codes(T, C, seed=T + C)
    qt, st = fgb.fp8_direct_transpose(q.to(DEV), s.to(DEV))
    oqt, ost = O.direct_transpose(q.numpy(), s.numpy())
    assert np.array_equal(np_(qt), oqt) and np.array_equal(np_(st), ost)


def test_transpose_wgrad_dy_full(fgb):
    say("transpose: Wgrad dY codes [32768, 2048] with scales 2^-20..2^4")
    q, s = synth.wgrad_codes(32768, 2048, seed=0, stream=42)
    qt, st = fgb.fp8_direct_transpose(q.to(DEV), s.to(DEV))
    oqt, ost = O.direct_transpose(q.numpy(), s.numpy())
    assert np.array_equal(np_(st), ost)
    assert np.array_equal(np_(qt), oqt)


@pytest.mark.parametrize("T,C", [(128, 128), (256, 512), (384, 2048), (32768, 2048)])
def test_naive_transpose(fgb, T, C):
    say("three-pass transpose", T, C)
    q, s = synth.wgrad_codes(T, C, seed=T + C + 1)
    qt, st = fgb.fp8_naive_transpose(q.to(DEV), s.to(DEV))
    oqt, ost = O.naive_transpose(q.numpy(), s.numpy())
    assert np.array_equal(np_(st), ost)
    assert np.array_equal(np_(qt), oqt)


@pytest.mark.parametrize("G,R,C", [(8, 512, 256), (3, 1664, 384)])
def test_block_transpose_batched(fgb, G, R, C):
    say(f"transpose: batched expert weight blocks [{G}, {R}, {C}]")
    q = rand_codes((G, R, C), 15)
    s = rand_scales((G, R // 128, C // 128), -30, 10, 16)
    qt, st = fgb.fp8_block_transpose_batched(q.to(DEV), s.to(DEV))
    oqt, ost = O.block_transpose_batched(q.numpy(), s.numpy())
    assert np.array_equal(np_(qt), oqt) and np.array_equal(np_(st), ost)


@pytest.mark.parametrize("T,C", [(300, 256), (2500, 384), (16384, 2048)])
def test_grouped_direct_transpose(fgb, T, C):
    say("grouped direct transpose of expert segments", T, C)
    topk, G = 8, 32
    idx, _ = synth.routing(T=T, E=G, topk=topk, seed=T + 7)
    xq, xs = synth.wgrad_codes(T, C, seed=T + 8)
    # the permuted, padded layout both sides start from (rows past off[G] stay 0xCD)
    pq, ps, _, offs, _ = O.permute_pad(xq.numpy(), xs.numpy(), idx, G, 16)
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(DEV)
    qt, st, koff = fgb.fp8_grouped_direct_transpose(t(pq), t(ps), t(offs))
    K_cap = qt.shape[1]
    oqt, ost, okoff = O.grouped_direct_transpose(pq, ps, offs, K_cap)
    k = int(okoff[-1])
    assert np.array_equal(np_(koff), okoff)
    assert np.array_equal(np_(st)[:, :k // 128], ost[:, :k // 128])
    assert np.array_equal(np_(qt)[:, :k], oqt[:, :k])


@pytest.mark.parametrize("G,rows,cols", [(1, 128, 128), (3, 256, 384), (32, 2048, 7168)])
def test_quant_blockwise_t(fgb, G, rows, cols):
    say("quant_blockwise with transposed copy", G, rows, cols)
    g = torch.Generator().manual_seed(G + rows + cols)
    w = (torch.randn(G, rows, cols, generator=g) * 0.02
         * torch.exp2(torch.randint(-20, 8, (G, rows // 128, 1, cols // 128, 1), generator=g).float())
         .expand(G, rows // 128, 128, cols // 128, 128).reshape(G, rows, cols)).to(torch.bfloat16)
    w[0, :128, :128] = 0.0  # an all-zero block
    q, s, qt, st = fgb.fp8_quant_blockwise_t(w.to(DEV))
    for e in sorted({0, G - 1, G // 2}):
        oq, os_ = O.quant_blockwise(bits(w[e]))
        oqt, ost = O.block_transpose(oq, os_)
        assert np.array_equal(np_(s[e]), os_) and np.array_equal(np_(q[e]), oq), e
        assert np.array_equal(np_(st[e]), ost) and np.array_equal(np_(qt[e]), oqt), e


def test_transpose_block_weights(fgb):
    say("transpose: 128x128-block weight transpose")
    q = rand_codes((2048, 1024), 5)
    s = rand_scales((16, 8), -30, 10, 6)
    qt, st = fgb.fp8_direct_transpose(q.to(DEV), s.to(DEV), fgb.BLOCK128)
    assert np.array_equal(np_(qt), q.numpy().T) and np.array_equal(np_(st), s.numpy().T)


# ---------------------------------------------------------------------------
# GEMMs
#
# EXACT mode: max|d - ref| / max|ref| <= 1e-5 (FP32 out); BF16 out elementwise
# within one bf16 ulp of |ref| or 1e-5 * max|ref|.
# FAST mode (FP8 matrix unit): the bound derived from its measured product-sum
# behaviour -- each product of a run of 8 consecutive K is cut toward zero to
# 13 bits below the run's largest, so |d - ref| <= 2^-10 * sum_runs max|p|
# plus FP32 rounding of the sums (<= (K/8 + 4) * 2^-24 * sum |p|), plus the
# bf16 rounding of the output.
# ---------------------------------------------------------------------------
MODES = ["exact", "fast"]


def _mode(fgb, name):
    return fgb.GEMM_EXACT if name == "exact" else fgb.GEMM_FAST


def check_gemm(got, ref, mode, bf16, bounds=None, K=None):
    """got: numpy (fp32 values or bf16 bits) at the sampled/full positions; ref fp64."""
    if bf16:
        gv = torch.from_numpy(np.ascontiguousarray(got).view(np.int16)).view(torch.bfloat16).float().numpy().astype(np.float64)
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
        return d.max() / max(np.max(np.abs(ref)), 1e-300)
    rm, asum = bounds
    tol = 2.0 ** -10 * rm + (K / 8 + 4) * 2.0 ** -24 * asum
    if bf16:
        tol = tol + ulp_bf16(np.abs(ref) + tol)
    ok = d <= tol
    assert ok.all(), f"{(~ok).sum()} elements beyond the FP8-unit bound; worst excess {np.max(d - tol)}"
    return d.max() / max(np.max(np.abs(ref)), 1e-300)


def _all_pairs(M, N):
    return np.repeat(np.arange(M), N), np.tile(np.arange(N), M)


@pytest.mark.parametrize("mode", MODES)
def test_gemm_linear_tiny_three_gemms(fgb, mode):
    say("gemm: tiny linear Fprop / Dgrad / Wgrad (fp32 out)", mode)
    X, W, dY = synth.linear_tiny(0)
    oxq, oxs = O.quant_rowwise(X.numpy())
    owq, ows = O.quant_blockwise(W.numpy())
    ogq, ogs = O.quant_rowwise(dY.numpy())
    oxqt, oxst = O.direct_transpose(oxq, oxs)
    ogqt, ogst = O.direct_transpose(ogq, ogs)
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(DEV)
    cases = [(oxq, oxs, O.ROW1x128, owq, ows, O.BLOCK128),
             (ogq, ogs, O.ROW1x128, owq.T.copy(), ows.T.copy(), O.BLOCK128),
             (ogqt, ogst, O.ROW1x128, oxqt, oxst, O.ROW1x128)]
    for a, sa, ag, b, sb, bg in cases:
        d = fgb.fp8_block_gemm(t(a), t(sa), ag, t(b), t(sb), bg, out_dtype=torch.float32, mode=_mode(fgb, mode))
        ref = O.block_gemm(a, sa, ag, b, sb, bg)
        bounds = None
        if mode == "fast":
            mi, ni = _all_pairs(a.shape[0], b.shape[0])
            bounds = [x.reshape(ref.shape) for x in O.gemm_run_bounds_sampled(a, sa, ag, b, sb, bg, mi, ni)]
        err = check_gemm(np_(d), ref, mode, False, bounds, a.shape[1])
        say("  max rel err", err)


@pytest.mark.parametrize("mode", MODES)
@pytest.mark.parametrize("M,N,K", [(1, 1, 128), (300, 2112, 512), (513, 260, 384)])
@pytest.mark.parametrize("bg", ["block", "row"])
def test_gemm_ragged(fgb, M, N, K, bg, mode):
    say("gemm ragged", M, N, K, bg, mode)
    a = rand_codes((M, K), M)
    b = rand_codes((N, K), N)
    sa = rand_scales((M, K // 128), -10, 10, 3)
    if bg == "block":
        sb = rand_scales(((N + 127) // 128, K // 128), -10, 10, 4)
        gran = fgb.BLOCK128
    else:
        sb = rand_scales((N, K // 128), -10, 10, 4)
        gran = fgb.ROW1x128
    ref = O.block_gemm(a.numpy(), sa.numpy(), O.ROW1x128, b.numpy(), sb.numpy(), gran)
    bounds = None
    if mode == "fast":
        mi, ni = _all_pairs(M, N)
        bounds = [x.reshape(ref.shape) for x in
                  O.gemm_run_bounds_sampled(a.numpy(), sa.numpy(), O.ROW1x128, b.numpy(), sb.numpy(), gran, mi, ni)]
    for bf16 in (False, True):
        d = fgb.fp8_block_gemm(a.to(DEV), sa.to(DEV), fgb.ROW1x128, b.to(DEV), sb.to(DEV), gran,
                               out_dtype=torch.bfloat16 if bf16 else torch.float32, mode=_mode(fgb, mode))
        check_gemm(np_(d), ref, mode, bf16, bounds, K)


def test_gemm_empty_and_k0(fgb):
    """M = 0 writes nothing; K = 0 is the empty sum: D = 0, or D unchanged when accumulating."""
    say("gemm: M = 0 and K = 0")
    M, N, K = 300, 260, 256
    b = rand_codes((N, K), 5).to(DEV)
    sb = rand_scales(((N + 127) // 128, K // 128), -4, 4, 6).to(DEV)
    a0 = torch.empty((0, K), dtype=torch.uint8, device=DEV)
    sa0 = torch.empty((0, K // 128), dtype=torch.uint8, device=DEV)
    for dt in (torch.float32, torch.bfloat16):
        assert fgb.fp8_block_gemm(a0, sa0, fgb.ROW1x128, b, sb, fgb.BLOCK128, out_dtype=dt).shape == (0, N)
    e = lambda r: torch.empty((r, 0), dtype=torch.uint8, device=DEV)
    ak, sak, bk, sbk = e(M), e(M), e(N), e((N + 127) // 128)
    for mode in MODES:
        for dt in (torch.float32, torch.bfloat16):
            d = torch.full((M, N), 3.0, dtype=dt, device=DEV)
            fgb.fp8_block_gemm(ak, sak, fgb.ROW1x128, bk, sbk, fgb.BLOCK128, d=d, mode=_mode(fgb, mode))
            assert torch.count_nonzero(d).item() == 0, (mode, dt)
        base = torch.randn(M, N, device=DEV) + 0.5  # no -0.0 (the empty sum adds +0.0)
        d = base.clone()
        fgb.fp8_block_gemm(ak, sak, fgb.ROW1x128, bk, sbk, fgb.BLOCK128, d=d, accumulate=True, mode=_mode(fgb, mode))
        assert torch.equal(d, base), mode


def test_gemm_accumulate_and_ldd(fgb):
    say("gemm accumulate into strided fp32 D")
    M, N, K = 256, 384, 256
    a, b = rand_codes((M, K), 1), rand_codes((N, K), 2)
    sa, sb = rand_scales((M, 2), -5, 5, 3), rand_scales((N, 2), -5, 5, 4)
    ref = O.block_gemm(a.numpy(), sa.numpy(), O.ROW1x128, b.numpy(), sb.numpy(), O.ROW1x128)
    base = torch.randn(M, 512, dtype=torch.float32)
    d = base.clone().to(DEV)
    fgb.fp8_block_gemm(a.to(DEV), sa.to(DEV), fgb.ROW1x128, b.to(DEV), sb.to(DEV), fgb.ROW1x128,
                       d=d[:, :N], accumulate=True)
    got = np_(d)
    check_fp32(got[:, :N] - base.numpy()[:, :N].astype(np.float64), ref, tol=1e-5)
    assert np.array_equal(got[:, N:], base.numpy()[:, N:])


@pytest.mark.parametrize("mode", MODES)
def test_gemm_k4096_accumulation_control(fgb, mode):
    say("gemm: K=4096 random FP8 precision control", mode)
    g = torch.Generator().manual_seed(9)
    x = torch.randn(256, 4096, generator=g)
    y = torch.randn(512, 4096, generator=g)
    qa, sa = O.quant_rowwise(x.numpy())
    qb, sb = O.quant_rowwise(y.numpy())
    ref = O.block_gemm(qa, sa, O.ROW1x128, qb, sb, O.ROW1x128)
    t = lambda a: torch.from_numpy(a).to(DEV)
    d = np_(fgb.fp8_block_gemm(t(qa), t(sa), fgb.ROW1x128, t(qb), t(sb), fgb.ROW1x128, out_dtype=torch.float32,
                               mode=_mode(fgb, mode)))
    bounds = None
    if mode == "fast":
        mi, ni = _all_pairs(256, 512)
        bounds = [x.reshape(ref.shape) for x in O.gemm_run_bounds_sampled(qa, sa, O.ROW1x128, qb, sb, O.ROW1x128, mi, ni)]
    err = check_gemm(d, ref, mode, False, bounds, 4096)
    say("K=4096 max relative error", mode, err)


@pytest.mark.parametrize("mode", MODES)
def test_gemm_mx_per32_with_level1(fgb, mode):
    say("gemm: 1x32 E8M0 scales on both sides + fp32 level-1 factor", mode)
    M, N, K = 192, 320, 1024
    a, b = rand_codes((M, K), 11), rand_codes((N, K), 12)
    sa, sb = rand_scales((M, K // 32), -20, 20, 13), rand_scales((N, K // 32), -20, 20, 14)
    l1 = torch.rand(N, generator=torch.Generator().manual_seed(15)) * 2 + 0.1
    l1n = l1.numpy().reshape(N, 1)
    ref = O.block_gemm(a.numpy(), sa.numpy(), O.ROW1x32, b.numpy(), sb.numpy(), O.ROW1x32, l1n, 10240)
    bounds = None
    if mode == "fast":
        mi, ni = _all_pairs(M, N)
        bounds = [x.reshape(ref.shape) for x in
                  O.gemm_run_bounds_sampled(a.numpy(), sa.numpy(), O.ROW1x32, b.numpy(), sb.numpy(), O.ROW1x32, mi, ni,
                                            b_l1=l1.numpy())]
    for bf16 in (False, True):  # the level-1 factor is applied in both epilogues
        d = fgb.fp8_block_gemm(a.to(DEV), sa.to(DEV), fgb.ROW1x32, b.to(DEV), sb.to(DEV), fgb.ROW1x32,
                               b_l1=l1.to(DEV), g1=10240, out_dtype=torch.bfloat16 if bf16 else torch.float32,
                               mode=_mode(fgb, mode))
        check_gemm(np_(d), ref, mode, bf16, bounds, K)


def test_gemm_mx_scale_byte_zero_exact(fgb):
    """E8M0 byte 0 means 2^-127 on the GPU as in the oracle: an A operand whose every 1x32 scale is byte 0
    (the scale the 1x32 quantizer gives a group with amax <= 448 * 2^-127), with codes whose value times
    2^-127 has a bf16 representation (exponent field >= 4), gives outputs near 2^-110 that the exact mode
    must reproduce; reading byte 0 as 2^-126 would double them."""
    say("gemm exact: 1x32 A scales all byte 0 (2^-127)")
    M, N, K = 96, 160, 512
    g = torch.Generator().manual_seed(21)
    a = torch.randint(0, 256, (M, K), generator=g, dtype=torch.int32).to(torch.uint8)
    a = (a & 0x87) | ((torch.randint(4, 16, (M, K), generator=g, dtype=torch.int32).to(torch.uint8)) << 3)
    a[(a & 0x7F) == 0x7F] ^= 1
    b = rand_codes((N, K), 22)
    sa = torch.zeros((M, K // 32), dtype=torch.uint8)
    sb = rand_scales((N, K // 32), -8, 8, 23)
    ref = O.block_gemm(a.numpy(), sa.numpy(), O.ROW1x32, b.numpy(), sb.numpy(), O.ROW1x32)
    assert 0 < np.max(np.abs(ref)) < 2.0 ** -90
    d = fgb.fp8_block_gemm(a.to(DEV), sa.to(DEV), fgb.ROW1x32, b.to(DEV), sb.to(DEV), fgb.ROW1x32,
                           out_dtype=torch.float32, mode=fgb.GEMM_EXACT)
    check_gemm(np_(d), ref, "exact", False)


def _sample(M, N, n, seed):
    rng = np.random.default_rng(seed)
    mi = np.concatenate([rng.integers(0, M, n), [0, M - 1, M - 1]])
    ni = np.concatenate([rng.integers(0, N, n), [0, N - 1, 0]])
    return mi, ni


@pytest.mark.parametrize("mode", MODES)
def test_gemm_dsv3_linear_realistic(fgb, mode):
    say("gemm: DeepSeek-V3 Linear data (Student-t channels), 512-token slice, three GEMMs", mode)
    X, W, dY = synth.linear_dsv3(0, T=512)
    xq, xs = O.quant_rowwise(synth.bf16_bits(X))
    wq, ws = O.quant_blockwise(synth.bf16_bits(W))
    gq, gs = O.quant_rowwise(synth.bf16_bits(dY))
    xqt, xst = O.direct_transpose(xq, xs)
    gqt, gst = O.direct_transpose(gq, gs)
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(DEV)
    cases = [("fprop", xq, xs, O.ROW1x128, wq, ws, O.BLOCK128),
             ("dgrad", gq, gs, O.ROW1x128, wq.T.copy(), ws.T.copy(), O.BLOCK128),
             ("wgrad", gqt, gst, O.ROW1x128, xqt, xst, O.ROW1x128)]
    for name, a, sa, ag, b, sb, bg in cases:
        d = np_(fgb.fp8_block_gemm(t(a), t(sa), ag, t(b), t(sb), bg, out_dtype=torch.bfloat16, mode=_mode(fgb, mode)))
        mi, ni = _sample(a.shape[0], b.shape[0], 4000, 5)
        ref = O.block_gemm_sampled(a, sa, ag, b, sb, bg, mi, ni)
        bounds = O.gemm_run_bounds_sampled(a, sa, ag, b, sb, bg, mi, ni) if mode == "fast" else None
        err = check_gemm(d[mi, ni], ref, mode, True, bounds, a.shape[1])
        say("  ", name, "max |d|/max|ref|", err)


@functools.lru_cache(maxsize=1)
def _dsv3_quantized():
    X, W, dY = synth.linear_dsv3(0)
    xq, xs = O.quant_rowwise(synth.bf16_bits(X))
    wq, ws = O.quant_blockwise(synth.bf16_bits(W))
    return xq, xs, wq, ws


@pytest.mark.parametrize("mode", MODES)
def test_gemm_dsv3_fprop_full_sampled(fgb, mode):
    say("gemm: DeepSeek-V3 Fprop 8192x2048x7168, bf16 out, sampled", mode)
    xq, xs, wq, ws = _dsv3_quantized()
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(DEV)
    d = np_(fgb.fp8_block_gemm(t(xq), t(xs), fgb.ROW1x128, t(wq), t(ws), fgb.BLOCK128, mode=_mode(fgb, mode)))
    mi, ni = _sample(8192, 2048, 3000, 1)
    ref = O.block_gemm_sampled(xq, xs, O.ROW1x128, wq, ws, O.BLOCK128, mi, ni)
    bounds = O.gemm_run_bounds_sampled(xq, xs, O.ROW1x128, wq, ws, O.BLOCK128, mi, ni) if mode == "fast" else None
    check_gemm(d[mi, ni], ref, mode, True, bounds, 7168)


# ---------------------------------------------------------------------------
# MoE
# ---------------------------------------------------------------------------
def _moe_small(T=700, topk=4, G=6, H=512, seed=0):
    g = torch.Generator().manual_seed(seed)
    xq = rand_codes((T, H), seed + 1)
    xs = rand_scales((T, H // 128), -20, 4, seed + 2)
    idx = torch.stack([torch.randperm(G, generator=g)[:topk] for _ in range(T)]).to(torch.int32)
    idx[idx == 2] = -1  # expert 2 empty, slots dropped
    return xq, xs, idx


def test_permute_pad_small(fgb):
    say("permute_pad small (empty expert, dropped slots)")
    xq, xs, idx = _moe_small()
    G = 6
    oq, os_, orm, ooff, used = O.permute_pad(xq.numpy(), xs.numpy(), idx.numpy(), G, 16)
    q, s, rm, off = fgb.permute_pad(xq.to(DEV), xs.to(DEV), idx.to(DEV), G, 16)
    assert np.array_equal(np_(off), ooff) and np.array_equal(np_(rm), orm)
    assert np.array_equal(np_(q)[:used], oq[:used]) and np.array_equal(np_(s)[:used], os_[:used])


def test_permute_pad_moe_full(fgb):
    say("permute_pad: 16384 tokens top-8 of 32 experts, H=7168")
    T, H, G = 16384, 7168, 32
    idx, probs = synth.routing(T, G, 8, 1.1, 0)
    xq = rand_codes((T, H), 31)
    xs = rand_scales((T, H // 128), -20, 4, 32)
    oq, os_, orm, ooff, used = O.permute_pad(xq.numpy(), xs.numpy(), idx, G, 16)
    q, s, rm, off = fgb.permute_pad(xq.to(DEV), xs.to(DEV), torch.from_numpy(idx).to(DEV), G, 16)
    assert np.array_equal(np_(off), ooff) and np.array_equal(np_(rm), orm)
    assert np.array_equal(np_(s)[:used], os_[:used])
    assert np.array_equal(np_(q)[:used], oq[:used])


def test_unpermute_small_and_full(fgb):
    for T, topk, H, with_p in [(50, 3, 64, False), (300, 8, 7168, True), (16384, 8, 7168, True)]:
        say("unpermute", T, topk, H, with_p)
        g = torch.Generator().manual_seed(T)
        M = T * topk + 15 * 8
        y = torch.randn(M, H, generator=g).to(torch.bfloat16)
        rm = torch.randperm(M, generator=g)[: T * topk].reshape(T, topk).to(torch.int32)
        rm[0, 0] = -1
        probs = torch.rand(T, topk, generator=g) if with_p else None
        out = fgb.unpermute_unpad(y.to(DEV), rm.to(DEV), None if probs is None else probs.to(DEV))
        ref = O.unpermute_unpad(bits(y), rm.numpy(), None if probs is None else probs.numpy())
        assert np.array_equal(np_(out), ref)


@pytest.mark.parametrize("T,H,weighted", [(64, 256, True), (2048, 7168, True), (300, 512, False)])
def test_unpermute_backward(fgb, T, H, weighted):
    say("unpermute_backward", T, H, weighted)
    topk, G = 8, 32
    idx, probs = synth.routing(T=T, E=G, topk=topk, seed=T)
    M_cap = T * topk + 15 * G
    # the row map of the forward permute (codes irrelevant here: one 128-column block)
    z = np.zeros((T, 128), np.uint8)
    _, _, rmap, _, _ = O.permute_pad(z, z[:, :1], idx, G, 16, M_cap)
    g = torch.Generator().manual_seed(T + H)
    dout = torch.randn((T, H), generator=g).to(torch.bfloat16)
    pr = torch.from_numpy(probs).to(DEV) if weighted else None
    dy = fgb.unpermute_backward(dout.to(DEV), torch.from_numpy(rmap).to(DEV), pr, M_cap)
    ref = O.unpermute_backward(bits(dout), rmap, probs if weighted else None, M_cap)
    assert np.array_equal(np_(dy), ref)


def test_swiglu_quant(fgb):
    for M, F, use_off in [(64, 256, False), (1000, 2048, True)]:
        say("swiglu_quant", M, F, use_off)
        g = torch.Generator().manual_seed(M)
        h = (torch.randn(M, 2 * F, generator=g) * 4).to(torch.bfloat16)
        h[0, :F] = 0.0
        h[1, :F] = -100.0  # exp(-g) overflows
        off = torch.tensor([0, 48, 96, 96, M - 40], dtype=torch.int32) if use_off else None
        q0 = torch.zeros((M, F), dtype=torch.uint8, device=DEV)
        s0 = torch.zeros((M, F // 128), dtype=torch.uint8, device=DEV)
        q, s = fgb.swiglu_quant(h.to(DEV), None if off is None else off.to(DEV), q0, s0)
        oq, os_ = O.swiglu_quant(bits(h), None if off is None else off.numpy())
        assert np.array_equal(np_(s), os_)
        assert np.array_equal(np_(q), oq)


@pytest.mark.parametrize("M,F,use_off", [(70, 256, True), (1000, 2048, False)])
def test_swiglu_quant_cache(fgb, M, F, use_off):
    say("swiglu_quant_cache", M, F, use_off)
    g = torch.Generator().manual_seed(M + 3)
    h = (torch.randn(M, 2 * F, generator=g) * 4).to(torch.bfloat16)
    h[0] = 0.0                      # all-zero groups: scale byte 105
    h[1, :F] = -100.0               # exp(-g) overflows
    h[2, F:] = 1e-38                # tiny up values
    h[3, :128] = -448.0 * 2.0 ** 40  # a large group
    off = np.array([0, 16, 16, 48, 64], np.int32) if use_off else None
    t_off = None if off is None else torch.from_numpy(off).to(DEV)
    q, s, hq, hs = fgb.swiglu_quant_cache(h.to(DEV), t_off)
    oq, os_ = O.swiglu_quant(bits(h), off)
    ohq, ohs = O.quant_rowwise(bits(h), 128)
    rows = M if off is None else int(off[-1])
    assert np.array_equal(np_(s)[:rows], os_[:rows]) and np.array_equal(np_(q)[:rows], oq[:rows])
    assert np.array_equal(np_(hs)[:rows], ohs[:rows]) and np.array_equal(np_(hq)[:rows], ohq[:rows])
    # the plain entry point on the same input gives the same activation codes
    q2, s2 = fgb.swiglu_quant(h.to(DEV), t_off)
    assert np.array_equal(np_(q2)[:rows], np_(q)[:rows]) and np.array_equal(np_(s2)[:rows], np_(s)[:rows])


@pytest.mark.parametrize("T,H,weighted", [(64, 256, True), (2048, 7168, True), (300, 512, False)])
def test_unpermute_backward_quant(fgb, T, H, weighted):
    say("unpermute_backward_quant", T, H, weighted)
    topk, G = 8, 32
    idx, probs = synth.routing(T=T, E=G, topk=topk, seed=T + 1)
    M_cap = T * topk + 15 * G
    z = np.zeros((T, 128), np.uint8)
    _, _, rmap, _, _ = O.permute_pad(z, z[:, :1], idx, G, 16, M_cap)
    rmap[0, 1] = -1  # a dropped slot: its row is never referenced
    g = torch.Generator().manual_seed(T + H + 1)
    dout = torch.randn((T, H), generator=g).to(torch.bfloat16)
    dout[1] = 0.0
    pr = torch.from_numpy(probs).to(DEV) if weighted else None
    q, s = fgb.unpermute_backward_quant(dout.to(DEV), torch.from_numpy(rmap).to(DEV), pr, M_cap)
    dy = O.unpermute_backward(bits(dout), rmap, probs if weighted else None, M_cap)
    oq, os_ = O.quant_rowwise(dy, 128)
    assert np.array_equal(np_(s), os_)
    assert np.array_equal(np_(q), oq)


@pytest.mark.parametrize("M,F,use_off", [(37, 256, True), (4096, 2048, False)])
def test_dswiglu_quant(fgb, M, F, use_off):
    say("dswiglu_quant", M, F, use_off)
    g = torch.Generator().manual_seed(M + F)
    h = (torch.randn((M, 2 * F), generator=g) * 3).to(torch.bfloat16)
    hq, hs = O.quant_rowwise(bits(h), 128)
    da = (torch.randn((M, F), generator=g) * 0.1).to(torch.bfloat16)
    off = np.array([0, 16, 24, 32], np.int32) if use_off else None
    dq, ds = fgb.dswiglu_quant(torch.from_numpy(hq).to(DEV), torch.from_numpy(hs).to(DEV), da.to(DEV),
                               None if off is None else torch.from_numpy(off).to(DEV))
    oq, os_ = O.dswiglu_quant(hq, hs, bits(da), off)
    rows = M if off is None else int(off[-1])
    assert np.array_equal(np_(ds)[:rows], os_[:rows])
    assert np.array_equal(np_(dq)[:rows], oq[:rows])


def test_dswiglu_quant_smallest_scale_bytes(fgb):
    """Cache scale bytes 0..3 (2^-127..2^-124: decoded inputs in the fp32
    subnormal range) and the largest bytes the rule allows beside ordinary
    ones: the scale byte is read as 2^(byte - 127) for every byte, as the
    oracle reads it."""
    say("dswiglu_quant smallest scale bytes")
    M, F = 64, 256
    g = torch.Generator().manual_seed(7)
    hq = torch.randint(0, 256, (M, 2 * F), dtype=torch.uint8, generator=g)
    hq[(hq & 0x7F) == 0x7F] = 0x11  # no NaN codes
    choices = torch.tensor([0, 1, 2, 3, 100, 120, 127, 130], dtype=torch.uint8)
    hs = choices[torch.randint(0, len(choices), (M, 2 * F // 128), generator=g)]
    da = (torch.randn((M, F), generator=g) * 0.1).to(torch.bfloat16)
    dq, ds = fgb.dswiglu_quant(hq.to(DEV), hs.to(DEV), da.to(DEV), None)
    oq, os_ = O.dswiglu_quant(hq.numpy(), hs.numpy(), bits(da), None)
    assert np.array_equal(np_(ds), os_)
    assert np.array_equal(np_(dq), oq)


def _every_swiglu_input():
    """Every g the SwiGLU kernels can see: all finite bf16 values (the forward's
    input) and every finite E4M3 code times every 1x128 scale 2^-22..2^127
    (the backward's dequantized cache)."""
    b = np.arange(65536, dtype=np.uint32)
    gb = (b << 16).view(np.float32)
    gb = gb[np.isfinite(gb)]
    codes = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], np.uint8)
    dec = O.fp8_decode_all(O.E4M3)[codes].astype(np.float64)
    g8 = dec[None, :] * np.ldexp(1.0, np.arange(-22, 128))[:, None]
    g8 = g8[np.abs(g8) <= np.finfo(np.float32).max].astype(np.float32)  # finite in fp32
    return np.concatenate([gb, g8])


def test_swiglu_elementwise_exhaustive(fgb):
    """The fp32 values swiglu_quant and dswiglu_quant quantize, for every input
    g they can see, bit for bit against the oracle (random bf16 u and da, and
    u = da = 1)."""
    say("swiglu / dswiglu fp32 element values, every possible g")
    g = _every_swiglu_input()
    rng = np.random.default_rng(9)
    for kind in ("random", "ones"):
        if kind == "random":
            u = torch.from_numpy(rng.standard_normal(g.size).astype(np.float32)).to(torch.bfloat16).float().numpy()
            da = torch.from_numpy((rng.standard_normal(g.size) * 0.1).astype(np.float32)).to(torch.bfloat16).float().numpy()
        else:
            u = np.ones_like(g)
            da = np.ones_like(g)
        gd, ud, dad = (torch.from_numpy(np.ascontiguousarray(x)).to(DEV) for x in (g, u, da))
        a = np_(fgb.swiglu_f32(gd, ud))
        assert np.array_equal(a.view(np.uint32), O.swiglu_f32(g, u).view(np.uint32))
        du, dg = fgb.dswiglu_f32(gd, ud, dad)
        rdu, rdg = O.dswiglu_f32(g, u, da)
        assert np.array_equal(np_(du).view(np.uint32), rdu.view(np.uint32))
        assert np.array_equal(np_(dg).view(np.uint32), rdg.view(np.uint32))


@pytest.mark.parametrize("mode", MODES)
def test_grouped_gemm_small(fgb, mode):
    say("grouped gemm small, one empty expert, ragged segments", mode)
    G, N, K = 4, 384, 512
    off = np.array([0, 48, 48, 336, 352], np.int32)
    M_cap = 400
    a = rand_codes((M_cap, K), 41)
    sa = rand_scales((M_cap, K // 128), -6, 6, 42)
    b = rand_codes((G, N, K), 43)
    sb = rand_scales((G, (N + 127) // 128, K // 128), -6, 6, 44)
    d = torch.full((M_cap, N), 7.0, dtype=torch.float32, device=DEV)
    fgb.fp8_grouped_gemm(a.to(DEV), sa.to(DEV), b.to(DEV), sb.to(DEV), torch.from_numpy(off).to(DEV), d=d,
                         mode=_mode(fgb, mode))
    got = np_(d)
    mi = np.repeat(np.arange(352), N)
    ni = np.tile(np.arange(N), 352)
    ref = O.grouped_gemm_sampled(a.numpy(), sa.numpy(), b.numpy(), sb.numpy(), off, mi, ni).reshape(352, N)
    bounds = None
    if mode == "fast":
        rm = np.zeros(mi.size)
        asum = np.zeros(mi.size)
        for g in range(G):
            sel = (mi >= off[g]) & (mi < off[g + 1])
            if sel.any():
                r1, r2 = O.gemm_run_bounds_sampled(a.numpy(), sa.numpy(), O.ROW1x128, b.numpy()[g], sb.numpy()[g],
                                                   O.BLOCK128, mi[sel], ni[sel])
                rm[sel], asum[sel] = r1, r2
        bounds = (rm.reshape(352, N), asum.reshape(352, N))
    check_gemm(got[:352], ref, mode, False, bounds, K)
    assert np.all(got[352:] == 7.0)


@pytest.mark.parametrize("mode", MODES)
def test_grouped_gemm_all_experts_empty(fgb, mode):
    say("grouped gemm: every expert empty (no tile exists, nothing written)", mode)
    G, N, K, M_cap = 5, 256, 256, 300
    off = np.zeros(G + 1, np.int32)
    a = rand_codes((M_cap, K), 61)
    sa = rand_scales((M_cap, K // 128), -4, 4, 62)
    b = rand_codes((G, N, K), 63)
    sb = rand_scales((G, N // 128, K // 128), -4, 4, 64)
    d = torch.full((M_cap, N), 7.0, dtype=torch.bfloat16, device=DEV)
    fgb.fp8_grouped_gemm(a.to(DEV), sa.to(DEV), b.to(DEV), sb.to(DEV), torch.from_numpy(off).to(DEV), d=d,
                         mode=_mode(fgb, mode))
    assert bool((d == 7.0).all())


@pytest.mark.parametrize("mode", MODES)
def test_grouped_gemm_past_one_chunk_group(fgb, mode):
    """272 tiles: one full group of 8 x 32 tiles spread over the XCDs plus a
    partial group of 16; every segment boundary row and sampled interior rows."""
    say("grouped gemm: 3 experts, 17 m-tiles x 16 n-tiles, sampled + boundaries", mode)
    G, N, K = 3, 4096, 256
    off = np.array([0, 2000, 3504, 4208], np.int32)  # 2000, 1504, 704 rows: 8 + 6 + 3 m-tiles
    M_cap = 4400
    a = rand_codes((M_cap, K), 71)
    sa = rand_scales((M_cap, K // 128), -6, 6, 72)
    b = rand_codes((G, N, K), 73)
    sb = rand_scales((G, N // 128, K // 128), -6, 6, 74)
    d = torch.full((M_cap, N), 7.0, dtype=torch.float32, device=DEV)
    fgb.fp8_grouped_gemm(a.to(DEV), sa.to(DEV), b.to(DEV), sb.to(DEV), torch.from_numpy(off).to(DEV), d=d,
                         mode=_mode(fgb, mode))
    got = np_(d)
    assert np.all(got[off[G]:] == 7.0)
    rng = np.random.default_rng(7)
    edge = np.concatenate([off[:G], off[1:] - 1, off[:G] + 255, off[:G] + 256])
    mi = np.concatenate([rng.integers(0, off[G], 6000), edge[edge < off[G]]])
    mi = np.repeat(mi, 4)
    ni = np.concatenate([rng.integers(0, N, mi.size - 8), [0, 255, 256, 2047, 2048, 3839, 3840, N - 1]])
    ref = O.grouped_gemm_sampled(a.numpy(), sa.numpy(), b.numpy(), sb.numpy(), off, mi, ni)
    bounds = None
    if mode == "fast":
        rm = np.zeros(mi.size)
        asum = np.zeros(mi.size)
        for g in range(G):
            sel = (mi >= off[g]) & (mi < off[g + 1])
            if sel.any():
                rm[sel], asum[sel] = O.gemm_run_bounds_sampled(a.numpy(), sa.numpy(), O.ROW1x128, b.numpy()[g],
                                                               sb.numpy()[g], O.BLOCK128, mi[sel], ni[sel])
        bounds = (rm, asum)
    check_gemm(got[mi, ni], ref, mode, False, bounds, K)


@pytest.mark.parametrize("mode", MODES)
def test_grouped_gemm_moe_fc1_sampled(fgb, mode):
    say("grouped gemm: fc1 of the 32-expert layer (N=4096, K=7168), sampled", mode)
    T, G, N, K = 16384, 32, 4096, 7168
    idx, _ = synth.routing(T, G, 8, 1.1, 0)
    counts = np.bincount(idx.ravel(), minlength=G)
    off = np.concatenate([[0], np.cumsum((counts + 15) // 16 * 16)]).astype(np.int32)
    M_cap = T * 8 + 15 * G
    a = rand_codes((M_cap, K), 51)
    sa = rand_scales((M_cap, K // 128), -8, 2, 52)
    b = rand_codes((G, N, K), 53)
    sb = rand_scales((G, N // 128, K // 128), -12, -4, 54)
    d = np_(fgb.fp8_grouped_gemm(a.to(DEV), sa.to(DEV), b.to(DEV), sb.to(DEV), torch.from_numpy(off).to(DEV),
                                 mode=_mode(fgb, mode)))
    rng = np.random.default_rng(3)
    mi = np.concatenate([rng.integers(0, off[G], 3000), off[1:G] - 1, off[:G]])
    mi = mi[mi < off[G]]
    ni = rng.integers(0, N, mi.size)
    ref = O.grouped_gemm_sampled(a.numpy(), sa.numpy(), b.numpy(), sb.numpy(), off, mi, ni)
    bounds = None
    if mode == "fast":
        rm = np.zeros(mi.size)
        asum = np.zeros(mi.size)
        an, san, bn, sbn = a.numpy(), sa.numpy(), b.numpy(), sb.numpy()
        for g in range(G):
            sel = (mi >= off[g]) & (mi < off[g + 1])
            if sel.any():
                rm[sel], asum[sel] = O.gemm_run_bounds_sampled(an, san, O.ROW1x128, bn[g], sbn[g], O.BLOCK128,
                                                               mi[sel], ni[sel])
        bounds = (rm, asum)
    check_gemm(d[mi, ni], ref, mode, True, bounds, K)


def _kgrouped_bounds(a, sa, b, sb, koff, ei, mi, ni):
    """FP8-unit error bounds of the sampled K-grouped products, expert by expert."""
    rm = np.zeros(mi.size)
    asum = np.zeros(mi.size)
    for e in range(len(koff) - 1):
        sel = ei == e
        k0, k1 = int(koff[e]), int(koff[e + 1])
        if sel.any() and k1 > k0:
            rm[sel], asum[sel] = O.gemm_run_bounds_sampled(
                a[:, k0:k1], sa[:, k0 // 128:k1 // 128], O.ROW1x128, b[:, k0:k1], sb[:, k0 // 128:k1 // 128],
                O.ROW1x128, mi[sel], ni[sel])
    return rm, asum


@pytest.mark.parametrize("mode", MODES)
@pytest.mark.parametrize("accumulate", [False, True])
def test_kgrouped_gemm_small(fgb, mode, accumulate):
    say("k-grouped gemm small: ragged M and N, one empty expert", mode, accumulate)
    M, N, K_cap = 300, 320, 1024
    koff = np.array([0, 128, 128, 512, 896], np.int32)  # columns past 896 are never read
    G = len(koff) - 1
    a = rand_codes((M, K_cap), 61)
    sa = rand_scales((M, K_cap // 128), -6, 6, 62)
    b = rand_codes((N, K_cap), 63)
    sb = rand_scales((N, K_cap // 128), -6, 6, 64)
    init = torch.randn((G, M, N), generator=torch.Generator().manual_seed(65))
    d = init.clone().to(DEV)
    fgb.fp8_kgrouped_gemm(a.to(DEV), sa.to(DEV), b.to(DEV), sb.to(DEV), torch.from_numpy(koff).to(DEV), d=d,
                          accumulate=accumulate, mode=_mode(fgb, mode))
    got = np_(d).astype(np.float64).ravel()
    if accumulate:
        got = got - init.numpy().astype(np.float64).ravel()  # exact: |d| is far above the product's rounding
    ei = np.repeat(np.arange(G), M * N)
    mi = np.tile(np.repeat(np.arange(M), N), G)
    ni = np.tile(np.arange(N), G * M)
    ref = O.kgrouped_gemm_sampled(a.numpy(), sa.numpy(), b.numpy(), sb.numpy(), koff, ei, mi, ni)
    assert np.all(got.reshape(G, M, N)[1] == 0.0)  # the empty expert
    bounds = None
    if mode == "fast":
        bounds = _kgrouped_bounds(a.numpy(), sa.numpy(), b.numpy(), sb.numpy(), koff, ei, mi, ni)
    if accumulate:
        # D += P rounds once more in FP32: allow one FP32 ulp of |init + P| on top
        tol = np.abs(init.numpy().ravel().astype(np.float64)) * 2.0 ** -23 + np.abs(ref) * 2.0 ** -23
        if mode == "exact":
            assert np.all(np.abs(got - ref) <= tol + 1e-5 * np.max(np.abs(ref)))
        else:
            rm, asum = bounds
            assert np.all(np.abs(got - ref) <= tol + 2.0 ** -10 * rm + (K_cap / 8 + 4) * 2.0 ** -24 * asum)
    else:
        check_gemm(got, ref, mode, False, bounds, K_cap)


@pytest.mark.parametrize("mode", MODES)
def test_kgrouped_gemm_moe_wgrad_sampled(fgb, mode):
    say("k-grouped gemm: Wgrad of fc1 of the 32-expert layer (M=4096, N=7168), sampled", mode)
    T, G, topk, M, N = 16384, 32, 8, 4096, 7168
    idx, _ = synth.routing(T, G, topk, 1.1, 0)
    seg = (np.bincount(idx.ravel(), minlength=G) + 15) // 16 * 16  # padded expert segments
    koff = np.concatenate([[0], np.cumsum((seg + 127) // 128 * 128)]).astype(np.int32)
    K_cap = fgb.grouped_k_cap(T * topk + 15 * G, G)
    assert koff[-1] <= K_cap
    a = rand_codes((M, K_cap), 71)
    sa = rand_scales((M, K_cap // 128), -20, 4, 72)
    b = rand_codes((N, K_cap), 73)
    sb = rand_scales((N, K_cap // 128), -8, 2, 74)
    d = np_(fgb.fp8_kgrouped_gemm(a.to(DEV), sa.to(DEV), b.to(DEV), sb.to(DEV), torch.from_numpy(koff).to(DEV),
                                  out_dtype=torch.bfloat16, mode=_mode(fgb, mode)))
    rng = np.random.default_rng(5)
    ei = np.concatenate([rng.integers(0, G, 1500), np.arange(G), np.arange(G)])
    mi = np.concatenate([rng.integers(0, M, 1500), np.zeros(G, np.int64), np.full(G, M - 1)])
    ni = np.concatenate([rng.integers(0, N, 1500), np.full(G, N - 1), np.zeros(G, np.int64)])
    ref = O.kgrouped_gemm_sampled(a.numpy(), sa.numpy(), b.numpy(), sb.numpy(), koff, ei, mi, ni)
    bounds = None
    if mode == "fast":
        bounds = _kgrouped_bounds(a.numpy(), sa.numpy(), b.numpy(), sb.numpy(), koff, ei, mi, ni)
    check_gemm(d[ei, mi, ni], ref, mode, True, bounds, int(np.max(np.diff(koff))))


# ---------------------------------------------------------------------------
# MOSS two-level
# ---------------------------------------------------------------------------
def test_mx2_small_and_rows_of_full(fgb):
    for R, Cc, g1 in [(5, 1024 + 96, 512), (64, 28672, 10240)]:
        say("mx2", R, Cc, g1)
        W, _ = synth.moss(seed=0, R=R, C=Cc, M=1)
        W[1, :g1] = 0.0
        q, s2, s1 = fgb.mx2_quant(W.to(DEV), g1)
        oq, os2, os1 = O.mx2_quant(bits(W), g1)
        assert np.array_equal(np_(s1), os1) and np.array_equal(np_(s2), os2)
        assert np.array_equal(np_(q), oq)
        xh = np_(fgb.mx2_dequant(q, s2, s1, g1))
        assert np.array_equal(xh, O.mx2_dequant(oq, os2, os1, g1))


def test_determinism_every_kernel_family(fgb):
    """Each kernel family twice on the same device inputs: identical bytes (no
    float atomics, no order-dependent reductions anywhere)."""
    say("determinism: every kernel family run twice")
    torch.manual_seed(11)
    T, H, F, G, topk = 1024, 1024, 512, 8, 4
    x = torch.randn(T, H, device=DEV).to(torch.bfloat16)
    w = (torch.randn(G, 2 * F, H, device=DEV) * 0.02).to(torch.bfloat16)
    idx = torch.stack([torch.randperm(G)[:topk] for _ in range(T)]).to(torch.int32).to(DEV)
    probs = torch.rand(T, topk, device=DEV)
    h = (torch.randn(T * topk + 15 * G, 2 * F, device=DEV) * 3).to(torch.bfloat16)
    yb = torch.randn(T * topk + 15 * G, H, device=DEV).to(torch.bfloat16)

    def run():
        out = []
        xq, xs = fgb.fp8_quant_rowwise(x)
        wq, ws, wqt, wst = fgb.fp8_quant_blockwise_t(w)
        xt, xts = fgb.fp8_direct_transpose(xq, xs)
        out += [xq, xs, wq, ws, wqt, wst, xt, xts]
        for mode in (fgb.GEMM_EXACT, fgb.GEMM_FAST):
            for od in (torch.bfloat16, torch.float32):
                out.append(fgb.fp8_block_gemm(xq, xs, fgb.ROW1x128, wq[0], ws[0], fgb.BLOCK128, out_dtype=od,
                                              mode=mode))
        pq, ps, rmap, offs = fgb.permute_pad(xq, xs, idx, G, 16)
        n = int(offs[-1])  # rows at or past off[G] are not written
        out += [pq[:n], ps[:n], rmap, offs]
        for mode in (fgb.GEMM_EXACT, fgb.GEMM_FAST):
            y = fgb.fp8_grouped_gemm(pq, ps, wq, ws, offs, mode=mode)
            out.append(y[:int(offs[-1])])
        q, s, hq, hs = fgb.swiglu_quant_cache(h[:pq.shape[0]], offs)
        out += [q[:n], s[:n], hq[:n], hs[:n]]
        dq, ds = fgb.dswiglu_quant(hq, hs, h[:pq.shape[0], :F].contiguous(), offs)
        out += [dq[:n], ds[:n]]
        out.append(fgb.unpermute_unpad(yb, rmap, probs))
        uq, us = fgb.unpermute_backward_quant(x, rmap, probs, pq.shape[0])
        out += [uq, us]
        qt, st, koff = fgb.fp8_grouped_direct_transpose(uq, us, offs)
        kend = int(koff[-1])
        out += [qt[:, :kend], st[:, :kend // 128], koff]
        for mode in (fgb.GEMM_EXACT, fgb.GEMM_FAST):
            out.append(fgb.fp8_kgrouped_gemm(qt[:256], st[:256], qt, st, koff, mode=mode))
        mq, m2, m1 = fgb.mx2_quant(x, 640)
        out += [mq, m2, m1]
        torch.cuda.synchronize()
        return [t.clone() for t in out]

    a, b = run(), run()
    for i, (u, v) in enumerate(zip(a, b)):
        assert u.shape == v.shape and torch.equal(u.view(torch.uint8) if u.dtype.is_floating_point else u,
                                                  v.view(torch.uint8) if v.dtype.is_floating_point else v), i
