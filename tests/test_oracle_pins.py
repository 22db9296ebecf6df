"""Pins for the CPU oracle: each test checks the oracle against something other
than itself -- printed values, exhaustive brute force, a library codec,
closed forms or exact integer arithmetic.  CPU only."""
import math
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle as O
import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def golden_values():
    vals = {}
    for line in open(os.path.join(GOLDEN, "pages_values.txt")):
        line = line.split("#")[0].strip()
        if line:
            k, v = [x.strip() for x in line.split("=")]
            vals[k] = v
    return vals


# --------------------------------------------------------------------------
# independent references built in the test
# --------------------------------------------------------------------------
def torch_decode_table():
    """E4M3FN decode by torch's float8_e4m3fn dtype (a library implementation)."""
    c = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    return c.view(torch.float8_e4m3fn).to(torch.float64).numpy()


def brute_encode(x):
    """Nearest finite E4M3 value by search over the sorted table of magnitudes;
    ties to the even code; >= 448 saturates; sign kept.  x: float64 array."""
    tab = torch_decode_table()
    codes = np.arange(0x7F)  # 0x00..0x7E: non-negative finite magnitudes, increasing
    mags = tab[codes]
    assert np.all(np.diff(mags) > 0)
    a = np.abs(x)
    i = np.searchsorted(mags, a, side="left")  # mags[i-1] < a <= mags[i]
    i = np.clip(i, 1, len(mags) - 1)
    lo, hi = mags[i - 1], mags[i]
    dlo, dhi = a - lo, hi - a
    pick_hi = (dhi < dlo) | ((dhi == dlo) & (codes[i] % 2 == 0))
    code = np.where(pick_hi, codes[i], codes[i - 1])
    code = np.where(a == 0, 0, code)
    code = np.where(a >= 448.0, 0x7E, code)
    sign = np.signbit(x).astype(np.int64) << 7
    return (code | sign).astype(np.uint8)


def code_int_value(c):
    """Integer n with decode(c) = n * 2^-9 (Python ints), sign included."""
    s, E, m = c >> 7, (c >> 3) & 15, c & 7
    mag = m if E == 0 else (8 + m) << (E - 1)
    return -mag if s else mag


def shift_code(c, k):
    """The pages' exponent-shift rule, done on the integer fields: decrement the
    exponent field by k when the result stays normal; otherwise shift the
    integer magnitude right by k with round-to-nearest-even (mantissa
    recombination into a subnormal)."""
    s, E, m = c & 0x80, (c >> 3) & 15, c & 7
    if k == 0:
        return c
    if E - k >= 1:
        return s | ((E - k) << 3) | m
    mag = m if E == 0 else (8 + m) << (E - 1)  # units of 2^-9
    q, r = mag >> k, mag & ((1 << k) - 1)
    half = 1 << (k - 1)
    if r > half or (r == half and (q & 1)):
        q += 1
    return s | q  # q <= 8, and 8 is exactly the code of 2^-6


def scale_exp_bits(amax_f32):
    """Closed form on the fp32 bits: 448 = 1.75 * 2^8, so for a normal amax with
    unbiased exponent Ea and mantissa field f, e = Ea - 8 + (f > 0x600000)."""
    b = np.asarray(amax_f32, np.float32).view(np.uint32).astype(np.int64)
    Ea = ((b >> 23) & 255) - 127
    f = b & 0x7FFFFF
    return (Ea - 8 + (f > 0x600000)).astype(np.int64)


# --------------------------------------------------------------------------
# E4M3 codec
# --------------------------------------------------------------------------
def test_decode_matches_library_codec_and_printed_range():
    g = golden_values()
    t = O.e4m3_decode_table()
    ref = torch_decode_table()
    fin = ~np.isnan(ref)
    assert np.array_equal(np.isnan(t), np.isnan(ref))
    assert np.array_equal(t[fin], ref[fin])
    assert np.array_equal(np.signbit(t[fin]), np.signbit(ref[fin]))
    assert np.nanmax(t) == float(g["e4m3_max"]) == t[0x7E]
    assert not np.isinf(t).any() and int(g["e4m3_has_inf"]) == 0
    assert set(np.flatnonzero(np.isnan(t))) == {0x7F, 0xFF}
    assert t[0x08] == 2.0 ** -6 and t[0x01] == 2.0 ** -9 and t[0x38] == 1.0
    assert len(set(np.abs(t[fin]))) == 127  # 0 plus 126 non-zero magnitudes


def test_encode_exhaustive_bf16():
    bits = np.arange(65536, dtype=np.uint32)
    f = (bits << 16).view(np.float32)
    f = f[np.isfinite(f)]
    assert np.array_equal(O.e4m3_encode(f), brute_encode(f.astype(np.float64)))


def test_encode_exhaustive_fp32_range():
    """Every fp32 value in [2^-12, 2^9] (covers all subnormal codes, every tie
    and the saturation edge) against brute force; both signs checked on a
    strided subset."""
    lo = np.float32(2.0 ** -12).view(np.uint32)
    hi = np.float32(2.0 ** 9).view(np.uint32)
    step = 1 << 23
    for start in range(int(lo), int(hi) + 1, step):
        b = np.arange(start, min(start + step, int(hi) + 1), dtype=np.uint32)
        f = b.view(np.float32)
        assert np.array_equal(O.e4m3_encode(f), brute_encode(f.astype(np.float64))), start
    b = np.arange(0, 0x44000000, 997, dtype=np.uint32) | np.uint32(0x80000000)
    f = b.view(np.float32)
    assert np.array_equal(O.e4m3_encode(f), brute_encode(f.astype(np.float64)))


def test_encode_matches_library_cast_below_saturation():
    """torch's float -> float8_e4m3fn cast rounds to nearest even; it agrees
    with the oracle wherever no saturation is involved (|v| < 464)."""
    rng = np.random.default_rng(7)
    x = (rng.standard_normal(1 << 20) * rng.choice([1e-3, 1e-1, 1, 30, 200], 1 << 20)).astype(np.float32)
    x = x[np.abs(x) < 464]
    ref = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(O.e4m3_encode(x), ref)


def test_encode_special_cases():
    v = np.array([0.0, -0.0, 448.0, -448.0, 449.0, 1e30, -1e30, 2.0 ** -10, -(2.0 ** -10),
                  3 * 2.0 ** -10, 1.0, 224.5, 432.0], np.float32)
    exp = np.array([0x00, 0x80, 0x7E, 0xFE, 0x7E, 0x7E, 0xFE, 0x00, 0x80, 0x02, 0x38, 0x76, 0x7E],
                   np.uint8)
    assert np.array_equal(O.e4m3_encode(v), exp)
    # encode(decode(c)) == c for all finite codes
    t = O.e4m3_decode_table()
    codes = np.array([c for c in range(256) if c not in (0x7F, 0xFF)])
    assert np.array_equal(O.e4m3_encode(t[codes].astype(np.float32)), codes.astype(np.uint8))


# --------------------------------------------------------------------------
# Scale rule
# --------------------------------------------------------------------------
def test_scale_rule_worked_cases():
    for line in open(os.path.join(GOLDEN, "scale_rule_worked.txt")):
        line = line.split("#")[0].strip()
        if not line:
            continue
        a, e, emin = line.split()
        a32 = np.float32(float(a))
        want = int(e)
        fr = Fraction(float(a32))
        if fr > 0 and want > int(emin):  # the hand value satisfies the defining inequality
            assert fr <= 448 * Fraction(2) ** want and fr > 448 * Fraction(2) ** (want - 1)
        assert O.scale_exp(np.array([a32]), int(emin))[0] == want, line


def test_scale_rule_closed_form_all_bf16_and_threshold_sweep():
    bits = np.arange(1, 0x7F80, dtype=np.uint32) << 16  # every positive finite bf16
    a = bits.view(np.float32)
    normal = a >= np.float32(2.0 ** -126)
    e = O.scale_exp(a, -22)
    ref = np.maximum(scale_exp_bits(a), -22)
    assert np.array_equal(e[normal], ref[normal])
    assert np.all(e[~normal] == -22)
    # mantissas around the 1.75 threshold for every exponent, and random fp32
    ex = np.arange(1, 255, dtype=np.uint32)
    mant = np.array([0, 1, 0x5FFFFF, 0x600000, 0x600001, 0x7FFFFF], np.uint32)
    b = (ex[:, None] << 23 | mant[None, :]).ravel()
    rng = np.random.default_rng(3)
    b = np.concatenate([b, rng.integers(0x00800000, 0x7F800000, 1 << 20, dtype=np.uint32)])
    a = b.view(np.float32)
    for emin in (-22, -127):
        assert np.array_equal(O.scale_exp(a, emin), np.maximum(scale_exp_bits(a), emin))


def test_scale_floor_is_the_printed_clamp():
    """The -22 floor reproduces the 1e-4 amax clamp: ceil(log2(max(amax,1e-4)/448))."""
    g = golden_values()
    clamp = float(g["amax_clamp"])
    rng = np.random.default_rng(5)
    a = np.concatenate([np.float32(10.0) ** rng.uniform(-9, 3, 100000).astype(np.float32),
                        np.zeros(3, np.float32)]).astype(np.float32)
    ref = np.array([math.ceil(math.log2(max(float(v), clamp) / 448.0)) for v in a])
    # exact comparison only where log2 is not within rounding of an integer
    exact_int = np.array([abs(math.log2(max(float(v), clamp) / 448.0) - round(math.log2(max(float(v), clamp) / 448.0))) < 1e-9 for v in a])
    e = O.scale_exp(a, -22)
    assert np.array_equal(e[~exact_int], ref[~exact_int])


# --------------------------------------------------------------------------
# Quantization
# --------------------------------------------------------------------------
def test_roundtrip_exact_for_every_code_and_scale():
    """quant(decode(c) * 2^e) recovers c at scale e for every finite code c and
    every e with an fp32-representable tile (the tile's max code fixes e)."""
    t = O.e4m3_decode_table()
    codes = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], np.int64)
    codes = np.concatenate([codes, np.full(256 - len(codes), 0x7E)])  # 256 per row
    for e in range(-22, 119):
        row = np.ldexp(t[codes], e).astype(np.float32)
        x = row.reshape(2, 128)
        x[:, 0] = np.float32(np.ldexp(448.0, e))  # pin amax of each tile
        q, s = O.quant_rowwise(x, 128)
        want = codes.reshape(2, 128).copy()
        want[:, 0] = 0x7E
        assert np.array_equal(q, want.astype(np.uint8)), e
        assert np.all(s == e + 127)


def test_quant_rowwise_against_brute_force():
    rng = np.random.default_rng(11)
    x = (rng.standard_normal((16, 384)) * np.float32(10.0) ** rng.integers(-6, 4, (16, 1))).astype(np.float32)
    x[3, 128:256] = 0.0
    x[4, :128] = -0.0
    for group in (128, 32):
        q, s = O.quant_rowwise(x, group)
        emin = -22 if group == 128 else -127
        tiles = x.reshape(16, -1, group)
        amax = np.abs(tiles).max(-1)
        e = np.maximum(scale_exp_bits(amax), emin)
        e[amax == 0] = emin
        assert np.array_equal(s.astype(np.int64) - 127, e)
        scaled = tiles.astype(np.float64) * np.ldexp(1.0, -e)[..., None]
        assert np.array_equal(q, brute_encode(scaled).reshape(16, -1))
    # bf16 input path equals the fp32 path on the same values
    xb = torch.from_numpy(x).to(torch.bfloat16)
    bits = xb.view(torch.int16).numpy().view(np.uint16)
    qb, sb = O.quant_rowwise(bits, 128)
    qf, sf = O.quant_rowwise(xb.float().numpy(), 128)
    assert np.array_equal(qb, qf) and np.array_equal(sb, sf)


def test_quant_blockwise_against_brute_force_partial_block():
    rng = np.random.default_rng(12)
    rows, cols = 200, 256  # partial last row block (72 rows)
    w = (rng.standard_normal((rows, cols)) * 0.02).astype(np.float32)
    w[128:, 128:] *= 1e5
    q, s = O.quant_blockwise(w)
    assert s.shape == (2, 2)
    for rb in range(2):
        for cb in range(2):
            blk = w[rb * 128:(rb + 1) * 128, cb * 128:(cb + 1) * 128]
            e = max(int(scale_exp_bits(np.abs(blk).max())), -22)
            assert s[rb, cb] == e + 127
            assert np.array_equal(q[rb * 128:(rb + 1) * 128, cb * 128:(cb + 1) * 128],
                                  brute_encode(blk.astype(np.float64) * 2.0 ** -e))


def test_dequant_is_code_times_scale():
    rng = np.random.default_rng(13)
    q = rng.integers(0, 256, (128, 256)).astype(np.uint8)
    q[q == 0x7F] = 0x7E
    q[q == 0xFF] = 0xFE
    s = rng.integers(100, 140, (128, 2)).astype(np.uint8)
    out = O.dequant(q, s, O.ROW1x128)
    ref = torch_decode_table()[q] * np.ldexp(1.0, np.repeat(s.astype(np.int64) - 127, 128, axis=1))
    assert np.array_equal(out, ref)


# --------------------------------------------------------------------------
# Direct transpose
# --------------------------------------------------------------------------
def _transpose_case(e_top, ks):
    """128 x 256 row-wise block pair where row t holds all 256 codes and has scale e_top - ks[t]."""
    q = np.tile(np.arange(256, dtype=np.uint8), (128, 1))
    s = np.zeros((128, 2), np.uint8)
    for t in range(128):
        s[t, :] = e_top - ks[t] + 127
    return q, s


def test_direct_transpose_exhaustive_table_against_exponent_shift():
    ks = list(range(41)) + [0] * 87
    q, s = _transpose_case(100, ks)
    qt, st = O.direct_transpose(q, s)
    assert qt.shape == (256, 128) and st.shape == (256, 1)
    assert np.all(st == 227)
    for t in range(41):
        for c in range(256):
            if c in (0x7F, 0xFF):
                continue
            assert qt[c, t] == shift_code(c, ks[t]), (hex(c), ks[t])


def test_direct_transpose_worked_cases():
    for line in open(os.path.join(GOLDEN, "transpose_worked.txt")):
        line = line.split("#")[0].strip()
        if not line:
            continue
        c, k, want = [int(x, 0) for x in line.split()]
        ks = [0] * 128
        ks[1] = k
        q, s = _transpose_case(0, ks)
        qt, _ = O.direct_transpose(q, s)
        assert qt[c, 1] == want, line
        assert shift_code(c, k) == want, line  # the test's own rule agrees with the hand values


def test_direct_transpose_invariants():
    rng = np.random.default_rng(21)
    T, Cc = 256, 384
    q = rng.integers(0, 256, (T, Cc)).astype(np.uint8)
    q[(q & 0x7F) == 0x7F] = 0x7E
    s_eq = np.full((T, Cc // 128), 130, np.uint8)
    qt, st = O.direct_transpose(q, s_eq)
    assert np.array_equal(qt, q.T)  # equal row scales -> pure byte transpose
    s = rng.integers(107, 131, (T, Cc // 128)).astype(np.uint8)
    qt, st = O.direct_transpose(q, s)
    # output scale = block max of the row scales, replicated
    for tb in range(T // 128):
        for cb in range(Cc // 128):
            assert np.all(st[cb * 128:(cb + 1) * 128, tb] == s[tb * 128:(tb + 1) * 128, cb].max())
    # value check: dequantized transpose equals the original wherever no underflow occurs
    d0 = O.dequant(q, s, O.ROW1x128)
    d1 = O.dequant(qt, st, O.ROW1x128).T
    E = (q >> 3) & 15
    k = (np.repeat(st.T, 128, axis=1)[:, :Cc] if False else None)
    kk = np.zeros((T, Cc), np.int64)
    for tb in range(T // 128):
        for cb in range(Cc // 128):
            blk = s[tb * 128:(tb + 1) * 128, cb].astype(np.int64)
            kk[tb * 128:(tb + 1) * 128, cb * 128:(cb + 1) * 128] = (blk.max() - blk)[:, None]
    safe = E.astype(np.int64) - kk >= 1
    assert np.array_equal(d0[safe], d1[safe])
    # applying it again to the output (now equal scales per block) is a byte transpose
    qtt, stt = O.direct_transpose(qt, st)
    assert np.array_equal(qtt, qt.T)


# --------------------------------------------------------------------------
# three-pass (naive) transpose, and the sf = amax/448 rule of the study
# --------------------------------------------------------------------------
def brute_rowwise_pow2(x):
    """1x128 power-of-two quantization of a float64 array whose tile maxima are
    fp32 numbers: closed-form exponent and brute-force encoding."""
    rows, cols = x.shape
    tiles = x.reshape(rows, -1, 128)
    amax = np.abs(tiles).max(-1)
    e = np.full(amax.shape, -22, np.int64)
    nz = amax > 0
    e[nz] = np.maximum(scale_exp_bits(amax[nz].astype(np.float32)), -22)
    q = brute_encode(tiles * np.ldexp(1.0, -e)[..., None]).reshape(rows, cols)
    return q, (e + 127).astype(np.uint8)


def test_naive_transpose_is_dequant_transpose_requant():
    rng = np.random.default_rng(81)
    T, Cc = 256, 384
    x = (rng.standard_normal((T, Cc)) * np.float32(10.0) ** rng.integers(-3, 3, (T, 1))).astype(np.float32)
    q, s = O.quant_rowwise(x)
    qt, st = O.naive_transpose(q, s)
    xh = torch_decode_table()[q] * np.ldexp(1.0, np.repeat(s.astype(np.int64) - 127, 128, axis=1))
    qe, se = brute_rowwise_pow2(np.ascontiguousarray(xh.T))
    assert np.array_equal(qt, qe) and np.array_equal(st, se)


def test_naive_equals_direct_when_every_column_reaches_the_block_max():
    # every column of each 128x128 block holds a 448 and the block's rows share
    # one scale: the column scale is the block scale, nothing is re-rounded,
    # and both conversions give the byte transpose
    rng = np.random.default_rng(82)
    T, Cc = 256, 256
    q = (rng.integers(0, 0x7F, (T, Cc)) | (rng.integers(0, 2, (T, Cc)) << 7)).astype(np.uint8)
    q[(q & 0x7F) == 0x7F] = 0
    q[5, :] = 0x7E
    q[128 + 77, :] = 0xFE
    s = np.repeat(rng.integers(106, 140, (2, Cc // 128)), 128, axis=0).astype(np.uint8)  # e >= -21, above the floor
    qn, sn = O.naive_transpose(q, s)
    qd, sd = O.direct_transpose(q, s)
    assert np.array_equal(qn, q.T) and np.array_equal(qn, qd) and np.array_equal(sn, sd)


def test_naive_scale_never_exceeds_the_direct_block_scale():
    # the column maximum of a dequantized block is at most the block maximum, so
    # the three-pass scales are <= the direct transpose's block-max scales and
    # its dequantized result is at least as close to the input, element by element
    rng = np.random.default_rng(83)
    x = (rng.standard_normal((256, 256)) * np.exp(rng.standard_normal((256, 1)) * 3)).astype(np.float32)
    q, s = O.quant_rowwise(x)
    qn, sn = O.naive_transpose(q, s)
    qd, sd = O.direct_transpose(q, s)
    assert np.all(sn <= sd)
    ref = O.dequant(q, s, O.ROW1x128).T
    en = np.abs(O.dequant(qn, sn, O.ROW1x128) - ref)
    ed = np.abs(O.dequant(qd, sd, O.ROW1x128) - ref)
    assert np.all(en <= ed)


def test_quant_rowwise_sf_rule():
    rng = np.random.default_rng(84)
    x = (rng.standard_normal((8, 256)) * np.float32(10.0) ** rng.integers(-4, 4, (8, 1))).astype(np.float32)
    x[2, :128] = 0.0
    q, sf = O.quant_rowwise_sf(x)
    tiles = x.reshape(8, 2, 128)
    amax = np.abs(tiles).max(-1)
    f = np.where(amax > 0, (amax / np.float32(448.0)).astype(np.float32), np.float32(1.0)).astype(np.float32)
    assert np.array_equal(sf, f)
    y = (tiles / f[..., None]).astype(np.float32)  # fp32 division, correctly rounded
    assert np.array_equal(q, brute_encode(y.astype(np.float64)).reshape(8, 256))
    big = np.abs(tiles).argmax(-1)
    for r in range(8):
        for j in range(2):
            if amax[r, j] > 0:
                assert q[r, j * 128 + big[r, j]] & 0x7F == 0x7E  # the tile maximum codes to 448
    xd = O.dequant_sf(q, sf)
    assert np.array_equal(xd, (torch_decode_table()[q].astype(np.float32) * np.repeat(sf, 128, axis=1)).astype(np.float32))


def test_naive_transpose_sf_composition():
    rng = np.random.default_rng(85)
    x = (rng.standard_normal((256, 384)) * 3).astype(np.float32)
    q, sf = O.quant_rowwise_sf(x)
    qt, sft = O.naive_transpose_sf(q, sf)
    xt = np.ascontiguousarray((torch_decode_table()[q].astype(np.float32) * np.repeat(sf, 128, axis=1)).astype(np.float32).T)
    tiles = xt.reshape(384, 2, 128)
    amax = np.abs(tiles).max(-1)
    f = np.where(amax > 0, (amax / np.float32(448.0)).astype(np.float32), np.float32(1.0)).astype(np.float32)
    assert np.array_equal(sft, f)
    assert np.array_equal(qt, brute_encode((tiles / f[..., None]).astype(np.float32).astype(np.float64)).reshape(384, 256))


def test_grouped_direct_transpose_against_per_segment_direct_transpose():
    """Each expert segment's block equals the direct transpose of that segment,
    extended (when short) by absent rows of code 0 with scale byte 0, which can
    never hold the block maximum; koff is the scan of the 128-rounded lengths."""
    rng = np.random.default_rng(86)
    lens = [256, 48, 0, 128, 144, 16]
    off = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    M, Cc = int(off[-1]), 256
    q, s = synth.wgrad_codes(M, Cc, seed=86)
    q, s = q.numpy(), s.numpy()
    Kc = 1024
    qt, st, koff = O.grouped_direct_transpose(q, s, off, Kc)
    assert list(koff) == list(np.concatenate([[0], np.cumsum([(l + 127) // 128 * 128 for l in lens])]))
    for e, l in enumerate(lens):
        if l == 0:
            continue
        n = (l + 127) // 128 * 128
        qe = np.zeros((n, Cc), np.uint8)
        se = np.zeros((n, Cc // 128), np.uint8)
        qe[:l] = q[off[e]:off[e + 1]]
        se[:l] = s[off[e]:off[e + 1]]
        dq, ds = O.direct_transpose(qe, se)
        assert np.array_equal(qt[:, koff[e]:koff[e] + n], dq)
        assert np.array_equal(st[:, koff[e] // 128:(koff[e] + n) // 128], ds)


def test_kgrouped_gemm_against_per_expert_block_gemm():
    rng = np.random.default_rng(87)
    koff = np.array([0, 256, 256, 640, 768], np.int32)
    Kc, M, N = 896, 40, 24
    a = rng.integers(0, 0x7F, (M, Kc)).astype(np.uint8)
    b = (rng.integers(0, 0x7F, (N, Kc)) | 0x80 * rng.integers(0, 2, (N, Kc))).astype(np.uint8)
    sa = rng.integers(110, 135, (M, Kc // 128)).astype(np.uint8)
    sb = rng.integers(110, 135, (N, Kc // 128)).astype(np.uint8)
    ei, mi, ni = np.meshgrid(np.arange(4), np.arange(M), np.arange(N), indexing="ij")
    got = O.kgrouped_gemm_sampled(a, sa, b, sb, koff, ei.ravel(), mi.ravel(), ni.ravel()).reshape(4, M, N)
    for e in range(4):
        k0, k1 = koff[e], koff[e + 1]
        if k1 == k0:
            assert np.all(got[e] == 0)
            continue
        ref = O.block_gemm(np.ascontiguousarray(a[:, k0:k1]), np.ascontiguousarray(sa[:, k0 // 128:k1 // 128]),
                           O.ROW1x128, np.ascontiguousarray(b[:, k0:k1]),
                           np.ascontiguousarray(sb[:, k0 // 128:k1 // 128]), O.ROW1x128)
        assert np.array_equal(got[e], ref)


def test_block_transpose_exact():
    rng = np.random.default_rng(22)
    q = rng.integers(0, 256, (256, 384)).astype(np.uint8)
    s = rng.integers(100, 140, (2, 3)).astype(np.uint8)
    qt, st = O.block_transpose(q, s)
    assert np.array_equal(qt, q.T) and np.array_equal(st, s.T)


# --------------------------------------------------------------------------
# GEMM
# --------------------------------------------------------------------------
def _rand_codes(rng, shape):
    q = rng.integers(0, 256, shape).astype(np.uint8)
    q[(q & 0x7F) == 0x7F] ^= 0x01  # no NaN codes
    return q


def test_gemm_exact_integer_arithmetic_tiny():
    rng = np.random.default_rng(31)
    M, N, K = 5, 7, 256
    a = _rand_codes(rng, (M, K))
    b = _rand_codes(rng, (N, K))
    sa = rng.integers(110, 140, (M, K // 128)).astype(np.uint8)
    sb = rng.integers(110, 140, (1, K // 128)).astype(np.uint8)
    d = O.block_gemm(a, sa, O.ROW1x128, b, sb, O.BLOCK128)
    for m in range(M):
        for n in range(N):
            exact = Fraction(0)
            terms_abs = Fraction(0)
            for kb in range(K // 128):
                p = sum(code_int_value(int(a[m, k])) * code_int_value(int(b[n, k]))
                        for k in range(kb * 128, kb * 128 + 128))
                term = Fraction(p) * Fraction(2) ** (int(sa[m, kb]) + int(sb[0, kb]) - 254 - 18)
                exact += term
                terms_abs += abs(term)
            err = abs(Fraction(d[m, n]) - exact)
            assert err <= terms_abs * Fraction(2) ** -52, (m, n)


def test_gemm_equals_fp64_matmul_of_dequantized():
    rng = np.random.default_rng(32)
    M, N, K = 64, 300, 512
    a = _rand_codes(rng, (M, K))
    b = _rand_codes(rng, (N, K))
    tab = torch_decode_table()
    for a_gran, b_gran, ga, gb in [(O.ROW1x128, O.BLOCK128, 128, 128), (O.ROW1x128, O.ROW1x128, 128, 128),
                                   (O.ROW1x32, O.ROW1x32, 32, 32)]:
        sa = rng.integers(115, 135, (M, K // ga)).astype(np.uint8)
        if b_gran == O.BLOCK128:
            sb = rng.integers(115, 135, ((N + 127) // 128, K // 128)).astype(np.uint8)
            eb = np.repeat(np.repeat(sb.astype(np.int64) - 127, 128, 0)[:N], 128, 1)
        else:
            sb = rng.integers(115, 135, (N, K // gb)).astype(np.uint8)
            eb = np.repeat(sb.astype(np.int64) - 127, gb, 1)
        ea = np.repeat(sa.astype(np.int64) - 127, ga, 1)
        A = tab[a] * np.ldexp(1.0, ea)
        B = tab[b] * np.ldexp(1.0, eb)
        ref = A @ B.T
        d = O.block_gemm(a, sa, a_gran, b, sb, b_gran)
        assert np.max(np.abs(d - ref)) <= 1e-12 * np.max(np.abs(ref))
        mi = rng.integers(0, M, 50)
        ni = rng.integers(0, N, 50)
        ds = O.block_gemm_sampled(a, sa, a_gran, b, sb, b_gran, mi, ni)
        assert np.array_equal(ds, d[mi, ni])


def test_gemm_special_cases():
    K = 512
    a = np.full((3, K), 0x38, np.uint8)
    b = np.full((4, K), 0x38, np.uint8)
    sa = np.full((3, K // 128), 127, np.uint8)
    sb = np.full((1, K // 128), 127, np.uint8)
    assert np.all(O.block_gemm(a, sa, O.ROW1x128, b, sb, O.BLOCK128) == K)
    # one-hot rows select single products, scales multiply exactly
    a = np.zeros((2, K), np.uint8)
    a[0, 5] = 0x40    # 2.0
    a[1, 300] = 0xC8  # -4.0
    b = np.zeros((2, K), np.uint8)
    b[:, 5] = 0x30    # 0.5
    b[:, 300] = 0x38  # 1.0
    sa = np.full((2, K // 128), 127, np.uint8)
    sa[1, 2] = 130
    sb = np.full((1, K // 128), 127, np.uint8)
    sb[0, 0] = 125
    d = O.block_gemm(a, sa, O.ROW1x128, b, sb, O.BLOCK128)
    assert d[0, 0] == 2.0 * 0.5 * 2.0 ** -2 and d[1, 0] == -4.0 * 8.0


def test_gemm_level1_factor():
    rng = np.random.default_rng(33)
    M, N, K, g1 = 8, 16, 512, 256
    a = _rand_codes(rng, (M, K))
    b = _rand_codes(rng, (N, K))
    sa = rng.integers(120, 130, (M, K // 32)).astype(np.uint8)
    sb = rng.integers(120, 130, (N, K // 32)).astype(np.uint8)
    l1 = rng.uniform(0.5, 2.0, (N, 2)).astype(np.float32)
    d = O.block_gemm(a, sa, O.ROW1x32, b, sb, O.ROW1x32, l1, g1)
    d0 = O.block_gemm(a[:, :256], sa[:, :8], O.ROW1x32, b[:, :256], sb[:, :8], O.ROW1x32)
    d1 = O.block_gemm(a[:, 256:], sa[:, 8:], O.ROW1x32, b[:, 256:], sb[:, 8:], O.ROW1x32)
    ref = d0 * l1[:, 0].astype(np.float64)[None, :] + d1 * l1[:, 1].astype(np.float64)[None, :]
    assert np.max(np.abs(d - ref)) <= 1e-13 * np.max(np.abs(ref))


def test_fp32_accumulation_control():
    """The pages report that ~14-bit accumulation gives ~2% max relative error at
    K = 4096.  Here: the oracle vs a float32 sequential accumulation of the same
    products stays ~1e-6 while a 14-bit-truncated accumulation is orders worse --
    the oracle is not itself a low-precision accumulator."""
    rng = np.random.default_rng(34)
    M, N, K = 4, 64, 4096
    x = rng.standard_normal((M, K)).astype(np.float32)
    y = rng.standard_normal((N, K)).astype(np.float32)
    qa, sa = O.quant_rowwise(x, 128)
    qb, sb = O.quant_rowwise(y, 128)
    d = O.block_gemm(qa, sa, O.ROW1x128, qb, sb, O.ROW1x128)
    tab = torch_decode_table()
    A = (tab[qa] * np.ldexp(1.0, np.repeat(sa.astype(np.int64) - 127, 128, 1))).astype(np.float32)
    B = (tab[qb] * np.ldexp(1.0, np.repeat(sb.astype(np.int64) - 127, 128, 1))).astype(np.float32)
    acc32 = np.zeros((M, N), np.float32)
    acc14 = np.zeros((M, N), np.float64)
    for k in range(K):
        prod = (A[:, k:k + 1] * B[None, :, k]).astype(np.float32)
        acc32 = (acc32 + prod).astype(np.float32)
        s = acc14 + prod
        ex = np.floor(np.log2(np.maximum(np.abs(s), 1e-300)))
        q = np.exp2(ex - 13)
        acc14 = np.trunc(s / q) * q
    rel32 = np.max(np.abs(acc32 - d)) / np.max(np.abs(d))
    rel14 = np.max(np.abs(acc14 - d)) / np.max(np.abs(d))
    assert rel32 < 1e-5 and rel14 > 30 * rel32


# --------------------------------------------------------------------------
# MoE data movement
# --------------------------------------------------------------------------
def test_permute_pad_invariants():
    rng = np.random.default_rng(41)
    T, topk, G, H = 300, 4, 8, 256
    xq = rng.integers(0, 256, (T, H)).astype(np.uint8)
    xs = rng.integers(100, 140, (T, H // 128)).astype(np.uint8)
    idx = np.stack([rng.permutation(G)[:topk] for _ in range(T)]).astype(np.int32)
    idx[rng.integers(0, T, 50), rng.integers(0, topk, 50)] = -1  # dropped slots
    idx[idx == 7] = -1  # expert 7 gets no tokens
    out_q, out_s, rm, off, used = O.permute_pad(xq, xs, idx, G, 16)
    g = golden_values()
    assert int(g["pad_multiple"]) == 16
    counts = np.array([(idx == e).sum() for e in range(G)])
    assert off[0] == 0 and np.all(np.diff(off) == ((counts + 15) // 16) * 16)
    assert np.all(off % 16 == 0) and used == off[G] and off[8] == off[7]
    seen = np.zeros(used, bool)
    for t in range(T):
        for k in range(topk):
            e, r = idx[t, k], rm[t, k]
            if e < 0:
                assert r == -1
                continue
            assert off[e] <= r < off[e] + counts[e]
            assert np.array_equal(out_q[r], xq[t]) and np.array_equal(out_s[r], xs[t])
            seen[r] = True
    for e in range(G):
        rows = rm[idx == e]
        assert np.array_equal(np.sort(rows), np.arange(off[e], off[e] + counts[e]))
        # ascending token order inside the expert
        toks = np.nonzero((idx == e).any(1))[0]
        assert np.array_equal(rm[toks][idx[toks] == e], np.arange(off[e], off[e] + counts[e]))
        pad = slice(off[e] + counts[e], off[e + 1])
        assert np.all(out_q[pad] == 0) and np.all(out_s[pad] == 105)
        # the padding looks exactly like a quantized all-zero row
        zq, zs = O.quant_rowwise(np.zeros((1, H), np.float32), 128)
        assert np.all(out_q[pad] == zq) and np.all(out_s[pad] == zs)
        assert not seen[pad].any()
    assert np.all(out_q[used:] == 0xCD)  # rows past the end untouched


def test_unpermute_inverts_permute():
    rng = np.random.default_rng(42)
    T, G, H = 200, 6, 128
    x = torch.randn(T, H).to(torch.bfloat16)
    xb = x.view(torch.int16).numpy().view(np.uint16)
    idx = rng.integers(0, G, (T, 1)).astype(np.int32)
    xq = np.zeros((T, H), np.uint8)
    xs = np.zeros((T, 1), np.uint8)
    _, _, rm, off, used = O.permute_pad(xq, xs, idx, G, 16)
    y = np.zeros((T + 15 * G, H), np.uint16)
    y[rm[:, 0]] = xb
    assert np.array_equal(O.unpermute_unpad(y, rm), xb)


def test_unpermute_backward_is_the_adjoint():
    """dy = unpermute_backward(dout) satisfies <unpermute_unpad(y), dout> =
    <y, dy> for the exact linear maps (checked in fp64 with bf16-exact weights
    and values, where no rounding occurs), copies dout exactly without probs,
    and leaves every padding row zero."""
    rng = np.random.default_rng(43)
    T, topk, G, H = 96, 4, 8, 128
    idx = np.stack([rng.permutation(G)[:topk] for _ in range(T)]).astype(np.int32)
    _, _, rm, off, used = O.permute_pad(np.zeros((T, H), np.uint8), np.zeros((T, 1), np.uint8), idx, G, 16)
    M_cap = T * topk + 15 * G
    # small-integer bf16 values and power-of-two probs: every product and sum is exact
    dout = torch.from_numpy(rng.integers(-8, 9, (T, H)).astype(np.float32)).to(torch.bfloat16)
    db = dout.view(torch.int16).numpy().view(np.uint16)
    probs = np.ldexp(1.0, rng.integers(-3, 1, (T, topk))).astype(np.float32)
    dy = O.unpermute_backward(db, rm, probs, M_cap)
    dyf = torch.from_numpy(dy.view(np.int16)).view(torch.bfloat16).double().numpy()
    y = torch.from_numpy(rng.integers(-8, 9, (M_cap, H)).astype(np.float32)).to(torch.bfloat16)
    out = O.unpermute_unpad(y.view(torch.int16).numpy().view(np.uint16), rm, probs)
    outf = torch.from_numpy(out.view(np.int16)).view(torch.bfloat16).double().numpy()
    assert np.sum(outf * dout.double().numpy()) == np.sum(y.double().numpy() * dyf)
    # without probs: the rows are copies; padding rows (and rows past used) are zero
    dy1 = O.unpermute_backward(db, rm, None, M_cap)
    for t in range(T):
        for k in range(topk):
            assert np.array_equal(dy1[rm[t, k]], db[t])
    mask = np.zeros(M_cap, bool)
    mask[rm.ravel()] = True
    assert np.all(dy1[~mask] == 0) and np.all(dy[~mask] == 0)


def test_unpermute_weighted_fold_small_integers_and_fma():
    # small integers: every fma exact, result exact
    T, topk, H = 3, 3, 8
    y = torch.arange(12 * H, dtype=torch.float32).reshape(12, H).remainder(7).to(torch.bfloat16)
    yb = y.view(torch.int16).numpy().view(np.uint16)
    rm = np.array([[0, 5, -1], [2, 3, 4], [11, 10, 9]], np.int32)
    probs = np.array([[1, 2, 3], [0.5, 0.25, 2], [1, 1, 1]], np.float32)
    out = O.unpermute_unpad(yb, rm, probs)
    yf = y.float().numpy()
    ref = np.zeros((T, H), np.float64)
    for t in range(T):
        for k in range(topk):
            if rm[t, k] >= 0:
                ref[t] += probs[t, k] * yf[rm[t, k]]
    ref_b = torch.from_numpy(ref.astype(np.float32)).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(out, ref_b)
    # general values: fp32 fma fold emulated exactly with fractions, then RNE to bf16
    rng = np.random.default_rng(43)
    y = torch.from_numpy(rng.standard_normal((16, 4)).astype(np.float32)).to(torch.bfloat16)
    yb = y.view(torch.int16).numpy().view(np.uint16)
    rm = rng.integers(0, 16, (5, 8)).astype(np.int32)
    probs = rng.uniform(0, 1, (5, 8)).astype(np.float32)
    out = O.unpermute_unpad(yb, rm, probs)
    yf = y.float().numpy()
    for t in range(5):
        for h in range(4):
            acc = np.float32(0)
            for k in range(8):
                exact = Fraction(float(probs[t, k])) * Fraction(float(yf[rm[t, k], h])) + Fraction(float(acc))
                acc = np.float32(_round_f32(exact))
            want = torch.tensor([float(acc)], dtype=torch.float32).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)[0]
            assert out[t, h] == want


def _round_f32(fr):
    """Round a rational to the nearest fp32 (ties to even), via float64 neighbours."""
    f = np.float32(float(fr))
    cands = [np.nextafter(f, np.float32(-np.inf)), f, np.nextafter(f, np.float32(np.inf))]
    best = None
    for c in cands:
        d = abs(Fraction(float(c)) - fr)
        if best is None or d < best[0] or (d == best[0] and (np.float32(c).view(np.uint32) & 1) == 0):
            best = (d, c)
    return best[1]


# --------------------------------------------------------------------------
# SwiGLU
# --------------------------------------------------------------------------
def _ulp_f32(x):
    x = np.abs(np.asarray(x, np.float32))
    return np.nextafter(x, np.float32(np.inf)) - x


def test_expf_within_two_ulp_of_long_double():
    x = np.linspace(-87.0, 88.7, 1 << 20, dtype=np.float32)
    x = np.concatenate([x, np.float32([0, -0.0, 1e-8, -1e-8, 0.5, -0.5, 88.72, -87.33])])
    y = O.expf(x)
    ref = np.exp(x.astype(np.longdouble))
    err = np.abs(y.astype(np.longdouble) - ref) / _ulp_f32(ref.astype(np.float32)).astype(np.longdouble)
    assert err.max() <= 2.0
    assert O.expf(np.float32([0.0]))[0] == 1.0
    assert np.isinf(O.expf(np.float32([89.0]))[0]) and O.expf(np.float32([-105.0]))[0] == 0.0


def test_swiglu_quant_composition():
    """swiglu_quant = 1x128 quant of fp32 (g / (1 + exp(-g))) * u, gate first;
    here the activation is formed with numpy fp32 operations (IEEE, elementwise)
    around the oracle's exp, and quantized by the rowwise quant."""
    rng = np.random.default_rng(51)
    M, F = 48, 256
    h = torch.from_numpy((rng.standard_normal((M, 2 * F)) * 3).astype(np.float32)).to(torch.bfloat16)
    hb = h.view(torch.int16).numpy().view(np.uint16)
    g = h[:, :F].float().numpy()
    u = h[:, F:].float().numpy()
    e = O.expf(-g)
    a = ((g / (np.float32(1.0) + e)).astype(np.float32) * u).astype(np.float32)
    q_ref, s_ref = O.quant_rowwise(a, 128)
    q, s = O.swiglu_quant(hb)
    assert np.array_equal(q, q_ref) and np.array_equal(s, s_ref)
    # silu(0) == 0 exactly
    z = np.zeros((1, 2 * F), np.uint16)
    q0, s0 = O.swiglu_quant(z)
    assert np.all(q0 == 0) and np.all(s0 == 105)
    # rows past off[G] are not written
    off = np.array([0, 16, 32], np.int32)
    q2, s2 = O.swiglu_quant(hb, off)
    assert np.array_equal(q2[:32], q[:32]) and np.all(q2[32:] == 0)


def _dswiglu_inputs(seed, M, F):
    rng = np.random.default_rng(seed)
    h = (rng.standard_normal((M, 2 * F)) * 3).astype(np.float32)
    hq, hs = O.quant_rowwise(h, 128)
    da = torch.from_numpy(rng.standard_normal((M, F)).astype(np.float32)).to(torch.bfloat16)
    return hq, hs, da


def test_dswiglu_formula_is_the_derivative():
    """sg * (1 + g * (1 - sg)) with sg = 1/(1+e^-g) is d/dg [g * sigmoid(g)]:
    central differences in fp64 over a wide range of g."""
    g = np.linspace(-30, 30, 2001)
    silu = lambda x: x / (1.0 + np.exp(-x))
    h = 1e-5
    fd = (silu(g + h) - silu(g - h)) / (2 * h)
    sg = 1.0 / (1.0 + np.exp(-g))
    assert np.max(np.abs(sg * (1 + g * (1 - sg)) - fd)) < 1e-8


def test_dswiglu_quant_against_fp64_gradient():
    """Dequantized [dg | du] is within the E4M3 rounding bound of the fp64
    gradient of a = silu(g) * u at the dequantized cached input."""
    M, F = 24, 384
    hq, hs, da = _dswiglu_inputs(61, M, F)
    dab = da.view(torch.int16).numpy().view(np.uint16)
    dq, ds = O.dswiglu_quant(hq, hs, dab)
    h = O.dequant(hq, hs, O.ROW1x128)
    g, u = h[:, :F], h[:, F:]
    a = da.double().numpy()
    sg = 1.0 / (1.0 + np.exp(-g))
    exact = np.concatenate([a * u * sg * (1 + g * (1 - sg)), a * g * sg], axis=1)
    got = O.dequant(dq, ds, O.ROW1x128)
    step = np.ldexp(1.0, np.repeat(ds.astype(np.int64) - 127, 128, axis=1))  # 2^e per element
    bound = np.maximum(np.abs(exact) * 2.0 ** -4, step * 2.0 ** -10) * (1 + 1e-5) + np.abs(exact) * 1e-6
    assert np.all(np.abs(got - exact) <= bound)


def test_dswiglu_quant_composition_and_special_cases():
    """Layout and operation order: the gradient formed with numpy fp32 operations
    around the oracle's exp, dg then du, quantized 1x128."""
    M, F = 16, 256
    hq, hs, da = _dswiglu_inputs(62, M, F)
    dab = da.view(torch.int16).numpy().view(np.uint16)
    h = O.dequant(hq, hs, O.ROW1x128).astype(np.float32)
    g, u = h[:, :F], h[:, F:]
    a = da.float().numpy()
    one = np.float32(1.0)
    d = (one + O.expf(-g)).astype(np.float32)
    sg = (one / d).astype(np.float32)
    silu = (g / d).astype(np.float32)
    du = (a * silu).astype(np.float32)
    dsilu = (sg * (one + (g * (one - sg)).astype(np.float32)).astype(np.float32)).astype(np.float32)
    dg = ((a * u).astype(np.float32) * dsilu).astype(np.float32)
    q_ref, s_ref = O.quant_rowwise(np.concatenate([dg, du], axis=1), 128)
    dq, ds = O.dswiglu_quant(hq, hs, dab)
    assert np.array_equal(dq, q_ref) and np.array_equal(ds, s_ref)
    # g = 0: silu = 0 (du = 0) and dsilu = 1/2 exactly
    hz = hq.copy()
    hz[:, :F] = 0
    dq0, ds0 = O.dswiglu_quant(hz, hs, dab)
    assert np.all((dq0[:, F:] & 0x7F) == 0)  # +-0 (the sign of da is kept)
    ref0, rs0 = O.quant_rowwise((a * O.dequant(hz, hs, O.ROW1x128)[:, F:].astype(np.float32) * np.float32(0.5)).astype(np.float32), 128)
    assert np.array_equal(dq0[:, :F], ref0) and np.array_equal(ds0[:, :F // 128], rs0)
    # rows past off[G] are not written
    off = np.array([0, 8, 12], np.int32)
    dq2, _ = O.dswiglu_quant(hq, hs, dab, off)
    assert np.array_equal(dq2[:12], dq[:12]) and np.all(dq2[12:] == 0)


def test_swiglu_f32_forms_are_the_quantized_paths_values():
    """orc_swiglu_f32 and orc_dswiglu_f32 give exactly the fp32 values that
    orc_swiglu_quant and orc_dswiglu_quant quantize: their 1x128 quantization
    reproduces those outputs bit for bit."""
    rng = np.random.default_rng(53)
    M, F = 32, 256
    h = torch.from_numpy((rng.standard_normal((M, 2 * F)) * 3).astype(np.float32)).to(torch.bfloat16)
    hb = h.view(torch.int16).numpy().view(np.uint16)
    g = h[:, :F].float().numpy()
    u = h[:, F:].float().numpy()
    a = O.swiglu_f32(g, u)
    q_ref, s_ref = O.swiglu_quant(hb)
    q, s = O.quant_rowwise(a, 128)
    assert np.array_equal(q, q_ref) and np.array_equal(s, s_ref)
    hq, hs, da = _dswiglu_inputs(63, M, F)
    dab = da.view(torch.int16).numpy().view(np.uint16)
    hd = O.dequant(hq, hs, O.ROW1x128).astype(np.float32)
    du, dg = O.dswiglu_f32(hd[:, :F], hd[:, F:], da.float().numpy())
    dq_ref, ds_ref = O.dswiglu_quant(hq, hs, dab)
    dq, ds = O.quant_rowwise(np.concatenate([dg, du], axis=1), 128)
    assert np.array_equal(dq, dq_ref) and np.array_equal(ds, ds_ref)
    # special values: silu(0) = 0 with the sign of 0 * u, the clamps of exp
    gz = np.array([0.0, -0.0, 100.0, -100.0, 89.0, -89.0, 1e-30, -1e-30], np.float32)
    az = O.swiglu_f32(gz, np.ones_like(gz))
    assert az[0] == 0 and az[2] == 100.0 and az[3] == 0.0 and az[4] == 89.0
    assert np.signbit(az[1]) and np.signbit(az[3])  # -0/(1+e) and -100/inf are -0


# --------------------------------------------------------------------------
# MOSS two-level
# --------------------------------------------------------------------------
def test_mx2_level1_and_bounds():
    rng = np.random.default_rng(61)
    R, Cc, g1 = 6, 1024 + 384, 1024
    x = (rng.standard_normal((R, Cc)) * 0.02 * 10.0 ** rng.uniform(-2, 1, (R, 1))).astype(np.float32)
    x[2, :g1] = 0.0
    xb_t = torch.from_numpy(x).to(torch.bfloat16)
    xb = xb_t.view(torch.int16).numpy().view(np.uint16)
    xf = xb_t.float().numpy()
    q, s2, s1 = O.mx2_quant(xb, g1)
    assert s1.shape == (R, 2) and s2.shape == (R, Cc // 32)
    for r in range(R):
        for g in range(2):
            seg = xf[r, g * g1:min((g + 1) * g1, Cc)]
            amax = np.abs(seg).max()
            want = np.float32(amax) / np.float32(448.0) if amax > 0 else np.float32(1.0)
            assert s1[r, g] == want
    xh = O.mx2_dequant(q, s2, s1, g1)
    # level-2 scale rule on y = x / alpha1
    alpha = np.repeat(s1, g1, axis=1)[:, :Cc]
    y = (xf / alpha).astype(np.float32)
    e2 = np.maximum(scale_exp_bits(np.abs(y.reshape(R, -1, 32)).max(-1)), -127)
    e2[np.abs(y.reshape(R, -1, 32)).max(-1) == 0] = -127
    assert np.array_equal(s2.astype(np.int64) - 127, e2)
    # error bound: half an E4M3 ulp relative (2^-4) plus fp32 roundings, for elements
    # in the E4M3 normal range; absolute 2^-10 * 2^e2 * alpha below it
    sc = np.ldexp(1.0, np.repeat(e2, 32, axis=1)) * alpha
    normal = np.abs(y) * np.ldexp(1.0, -np.repeat(e2, 32, axis=1)) >= 2.0 ** -6
    err = np.abs(xh.astype(np.float64) - xf)
    assert np.all(err[normal] <= np.abs(xf[normal]) * (2.0 ** -4 + 4 * 2.0 ** -24))
    assert np.all(err[~normal] <= 2.0 ** -10 * sc[~normal] * (1 + 2.0 ** -20))
    # dequant is exactly (decode * 2^e2) * alpha in fp32
    tab = torch_decode_table()
    v = (tab[q] * np.ldexp(1.0, np.repeat(s2.astype(np.int64) - 127, 32, axis=1))).astype(np.float32)
    assert np.array_equal(xh, (v * alpha).astype(np.float32))


def test_mx2_two_level_snr_not_below_single_level():
    """MOSS review §3: two-level microscaling gives higher SNR than single-level."""
    W, _ = __import__("synth").moss(seed=0, R=64, C=28672, M=1)
    wb = W.view(torch.int16).numpy().view(np.uint16)
    wf = W.float().numpy()
    q, s2, s1 = O.mx2_quant(wb, 10240)
    snr2 = O.snr_db(wf, O.mx2_dequant(q, s2, s1, 10240))
    q1, s = O.quant_rowwise(wb, 32)
    snr1 = O.snr_db(wf, O.dequant(q1, s, O.ROW1x32).astype(np.float32))
    assert snr2 >= snr1 - 1e-9
    assert 25.0 < snr2 < 40.0  # E4M3 with per-32 scales: about 30 dB


def test_snr_closed_form():
    x = np.array([3.0, 4.0], np.float32)
    xh = np.array([3.0, 3.0], np.float32)
    assert abs(O.snr_db(x, xh) - 10 * math.log10(25.0)) < 1e-12
