"""The fast GEMM mode computes what the FP8 matrix-unit model
(tests/fp8_unit_model.py) says, bit for bit on codes quantized from
continuous data, in every layout the library offers: 1D1D and 1D2D scales,
1x32 E8M0 scales with the level-1 factor, E5M2 A operands, the M-grouped and
K-grouped forms, accumulation into D, FP32 and BF16 output; on uniformly
random codes, within a few FP32 roundings.  Each case also reports the fast result's distance from
the oracle (the method's FP32 accumulation of exact products), which exceeds
1e-5 of max|ref| on these workloads: the fast mode is the FP8 unit's
arithmetic, not the method's."""
import sys

import numpy as np
import pytest
import torch

import oracle as O
import synth
from fp8_unit_model import BLOCK128, E5M2, ROW1x32, ROW1x128, fp8_unit_accumulate, fp8_unit_gemm_sampled

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def say(*a):
    print("[case]", *a, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def fgb():
    import fine_grained_blockwise_amd as m
    return m


def dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


def raw(t):
    """fp32 -> uint32 bits, bf16 -> uint16 bits (CPU numpy)."""
    t = t.detach().cpu().contiguous()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    return t.numpy().view(np.uint32)


def check(name, got_bits, want_bits, ref=None, got_vals=None):
    bad = got_bits != want_bits
    assert not bad.any(), f"{name}: {int(bad.sum())} of {bad.size} outputs differ from the FP8-unit model"
    if ref is not None:
        err = np.max(np.abs(np.asarray(got_vals, np.float64) - ref)) / np.max(np.abs(ref))
        say(f"   {name}: bit-exact with the FP8-unit model; distance from the FP32 oracle {err:.2e} of max|ref|")


def test_fast_matches_model_k4096_1d1d_and_1x32(fgb):
    say("fast GEMM vs FP8-unit model: K=4096 N(0,1) control, 1x128 and 1x32 scales, fp32 and bf16 out")
    X = torch.randn(192, 4096, generator=torch.Generator().manual_seed(1))
    Y = torch.randn(320, 4096, generator=torch.Generator().manual_seed(2))
    for g, gran in ((128, ROW1x128), (32, ROW1x32)):
        xq, xs = O.quant_rowwise(X.numpy(), g)
        yq, ys = O.quant_rowwise(Y.numpy(), g)
        l1 = (np.random.default_rng(3).random(320) * 2 + 0.1).astype(np.float32) if g == 32 else None
        mi, ni = np.repeat(np.arange(192), 320), np.tile(np.arange(320), 192)
        ref = O.block_gemm_sampled(xq, xs, gran, yq, ys, gran, mi, ni,
                                   b_l1=None if l1 is None else l1.reshape(-1, 1), g1=10240 if l1 is not None else 0)
        for out, dt in (("f32", torch.float32), ("bf16", torch.bfloat16)):
            d = fgb.fp8_block_gemm(dev(xq), dev(xs), gran, dev(yq), dev(ys), gran,
                                   b_l1=None if l1 is None else dev(l1), g1=10240 if l1 is not None else 0,
                                   out_dtype=dt, mode=fgb.GEMM_FAST)
            want = fp8_unit_gemm_sampled(xq, xs, gran, yq, ys, gran, mi, ni, b_l1=l1, out=out)
            check(f"K=4096 1x{g} {out}", raw(d).ravel(), want.view(np.uint32) if out == "f32" else want, ref,
                  d.float().cpu().numpy().ravel())


def test_fast_matches_model_tiny_linear_three_gemms(fgb):
    say("fast GEMM vs FP8-unit model: the tiny Linear's Fprop, Dgrad, Wgrad")
    X, W, dY = synth.linear_tiny(0)
    xq, xs = O.quant_rowwise(X.numpy())
    wq, ws = O.quant_blockwise(W.numpy())
    gq, gs = O.quant_rowwise(dY.numpy())
    xqt, xst = O.direct_transpose(xq, xs)
    gqt, gst = O.direct_transpose(gq, gs)
    for name, a, sa, ag, b, sb, bg in [("fprop", xq, xs, ROW1x128, wq, ws, BLOCK128),
                                       ("dgrad", gq, gs, ROW1x128, wq.T.copy(), ws.T.copy(), BLOCK128),
                                       ("wgrad", gqt, gst, ROW1x128, xqt, xst, ROW1x128)]:
        M, N = a.shape[0], b.shape[0]
        mi, ni = np.repeat(np.arange(M), N), np.tile(np.arange(N), M)
        ref = O.block_gemm_sampled(a, sa, ag, b, sb, bg, mi, ni)
        d = fgb.fp8_block_gemm(dev(a), dev(sa), ag, dev(b), dev(sb), bg, out_dtype=torch.float32, mode=fgb.GEMM_FAST)
        want = fp8_unit_gemm_sampled(a, sa, ag, b, sb, bg, mi, ni)
        check(name, raw(d).ravel(), want.view(np.uint32), ref, d.cpu().numpy().ravel())
        # accumulate: D_out = fp32(D_in + unit result)
        d0 = torch.randn(M, N, generator=torch.Generator().manual_seed(5)).to(DEV)
        d1 = d0.clone()
        fgb.fp8_block_gemm(dev(a), dev(sa), ag, dev(b), dev(sb), bg, out_dtype=torch.float32, d=d1,
                           accumulate=True, mode=fgb.GEMM_FAST)
        want_acc = (d0.cpu().numpy().ravel().astype(np.float64) + want.astype(np.float64)).astype(np.float32)
        check(name + " accumulate", raw(d1).ravel(), want_acc.view(np.uint32))


def test_fast_matches_model_dsv3_fprop_full_sampled(fgb):
    say("fast GEMM vs FP8-unit model: DeepSeek-V3 Fprop 8192x2048x7168, bf16 out, sampled")
    X, W, _ = synth.linear_dsv3(0)
    xq, xs = O.quant_rowwise(synth.bf16_bits(X))
    wq, ws = O.quant_blockwise(synth.bf16_bits(W))
    d = raw(fgb.fp8_block_gemm(dev(xq), dev(xs), ROW1x128, dev(wq), dev(ws), BLOCK128, mode=fgb.GEMM_FAST))
    rng = np.random.default_rng(7)
    mi = np.concatenate([rng.integers(0, 8192, 1500), [0, 8191, 255, 256]])
    ni = np.concatenate([rng.integers(0, 2048, 1500), [2047, 0, 255, 256]])
    want = fp8_unit_gemm_sampled(xq, xs, ROW1x128, wq, ws, BLOCK128, mi, ni, out="bf16")
    check("dsv3 fprop bf16", d[mi, ni], want)


def test_fast_matches_model_e5m2_gradient(fgb):
    say("fast GEMM vs FP8-unit model: Dgrad with an E5M2 gradient (256 tokens of the DeepSeek-V3 Linear)")
    _, W, dY = synth.linear_dsv3(0, T=256)
    gq, gs = O.quant_rowwise_fmt(synth.bf16_bits(dY), 128, 1, 0)
    wq, ws = O.quant_blockwise(synth.bf16_bits(W))
    b, sb = wq.T.copy(), ws.T.copy()
    M, N = gq.shape[0], b.shape[0]
    rng = np.random.default_rng(8)
    mi, ni = rng.integers(0, M, 3000), rng.integers(0, N, 3000)
    d = fgb.fp8_block_gemm_fmt(dev(gq), dev(gs), ROW1x128, fgb.E5M2, dev(b), dev(sb), BLOCK128,
                               out_dtype=torch.float32, mode=fgb.GEMM_FAST)
    want = fp8_unit_gemm_sampled(gq, gs, ROW1x128, b, sb, BLOCK128, mi, ni, a_fmt=E5M2)
    check("e5m2 dgrad", raw(d)[mi, ni], want.view(np.uint32))


def _quantized_normal(rows, K, seed, std=1.0):
    x = torch.randn(rows, K, generator=torch.Generator().manual_seed(seed)) * std
    return O.quant_rowwise(x.numpy())


def test_fast_matches_model_grouped_forms(fgb):
    say("fast GEMM vs FP8-unit model: M-grouped (6 experts, bf16 out) and K-grouped (fp32 out)")
    G, N, K = 6, 384, 512
    lens = [48, 0, 272, 16, 96, 160]
    off = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    M_cap = int(off[-1]) + 32
    a, sa = _quantized_normal(M_cap, K, 31)
    bq = [O.quant_blockwise((torch.randn(N, K, generator=torch.Generator().manual_seed(40 + e)) * 0.02).numpy())
          for e in range(G)]
    b = np.stack([q for q, _ in bq])
    sb = np.stack([s for _, s in bq])
    d = raw(fgb.fp8_grouped_gemm(dev(a), dev(sa), dev(b), dev(sb), dev(off), mode=fgb.GEMM_FAST))
    for e in range(G):
        if lens[e] == 0:
            continue
        rows = np.arange(off[e], off[e + 1])
        mi, ni = np.repeat(rows, N), np.tile(np.arange(N), rows.size)
        want = fp8_unit_gemm_sampled(a, sa, ROW1x128, b[e], sb[e], BLOCK128, mi, ni, out="bf16")
        check(f"M-grouped expert {e}", d[mi, ni], want)
    # K-grouped: D_e = A[:, koff[e]:koff[e+1]] B[:, koff[e]:koff[e+1]]^T
    Mk, Nk, Kc = 256, 384, 1024
    koff = np.array([0, 256, 256, 640, 1024], np.int32)
    ka, ksa = _quantized_normal(Mk, Kc, 32)
    kb, ksb = _quantized_normal(Nk, Kc, 33)
    dk = raw(fgb.fp8_kgrouped_gemm(dev(ka), dev(ksa), dev(kb), dev(ksb), dev(koff), mode=fgb.GEMM_FAST))
    mi, ni = np.repeat(np.arange(Mk), Nk), np.tile(np.arange(Nk), Mk)
    for e in range(len(koff) - 1):
        if koff[e + 1] == koff[e]:
            assert not dk[e].any(), e  # an empty K range gives D_e = 0
            continue
        want = fp8_unit_accumulate(ka, ksa, ROW1x128, kb, ksb, ROW1x128, mi, ni, k0=int(koff[e]), k1=int(koff[e + 1]))
        check(f"K-grouped expert {e}", dk[e].ravel(), want.view(np.uint32))


def test_fast_within_rounding_of_model_on_uniformly_random_codes(fgb):
    """Every code equally likely (subnormals included): the unit's own adder ends a few FP32 roundings
    away from the model in a few percent of outputs; the runs' cut, which moves the result away from the
    exact sum, is the model's."""
    say("fast GEMM vs FP8-unit model: uniformly random codes, 1x128 and 1x32 scales")
    g = torch.Generator().manual_seed(19)
    M, N, K = 128, 256, 512

    def codes(shape):
        q = torch.randint(0, 256, shape, generator=g, dtype=torch.int32).to(torch.uint8)
        q[(q & 0x7F) == 0x7F] ^= 1
        return q.numpy()

    a, b = codes((M, K)), codes((N, K))
    mi, ni = np.repeat(np.arange(M), N), np.tile(np.arange(N), M)
    for grp, gran in ((128, ROW1x128), (32, ROW1x32)):
        sa = torch.randint(121, 130, (M, K // grp), generator=g, dtype=torch.int32).to(torch.uint8).numpy()
        sb = torch.randint(117, 126, (N, K // grp), generator=g, dtype=torch.int32).to(torch.uint8).numpy()
        d = fgb.fp8_block_gemm(dev(a), dev(sa), gran, dev(b), dev(sb), gran, out_dtype=torch.float32,
                               mode=fgb.GEMM_FAST).cpu().numpy().ravel().astype(np.float64)
        f = fp8_unit_gemm_sampled(a, sa, gran, b, sb, gran, mi, ni).astype(np.float64)
        _, asum = O.gemm_run_bounds_sampled(a, sa, gran, b, sb, gran, mi, ni)
        x = np.abs(d - f) / (2.0 ** -24 * asum)
        same = float(np.mean(d == f))
        say(f"   1x{grp}: {100 * same:.1f}% bit-identical; worst |gpu - model| = {x.max():.2f} x 2^-24 sum|p|")
        assert x.max() <= 8.0
        assert same >= 0.9
