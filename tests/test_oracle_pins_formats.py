"""Pins for the oracle's format variants: E5M2 elements (gradients), the OCP
floor rule for MX scales, and the format-aware quantizer, direct transpose and
GEMM.  Each test checks the oracle against something other than itself: a
library codec, brute-force search, integer-field arithmetic, closed forms on
the fp32 bits, exact rationals or the already-pinned E4M3 functions.  CPU only."""
from fractions import Fraction

import numpy as np
import torch

import oracle as O
from test_oracle_pins import golden_values


def torch_e5m2_table():
    """E5M2 decode by torch's float8_e5m2 dtype (a library implementation)."""
    c = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    return c.view(torch.float8_e5m2).to(torch.float64).numpy()


def brute_encode_e5m2(x):
    """Nearest finite E5M2 value by search over the sorted magnitudes; ties to
    the even code; >= 57344 clips to 57344; sign kept."""
    tab = torch_e5m2_table()
    codes = np.arange(0x7C)  # 0x00..0x7B: non-negative finite magnitudes, increasing
    mags = tab[codes]
    assert np.all(np.diff(mags) > 0)
    a = np.abs(x)
    i = np.clip(np.searchsorted(mags, a, side="left"), 1, len(mags) - 1)
    lo, hi = mags[i - 1], mags[i]
    pick_hi = ((hi - a) < (a - lo)) | (((hi - a) == (a - lo)) & (codes[i] % 2 == 0))
    code = np.where(pick_hi, codes[i], codes[i - 1])
    code = np.where(a == 0, 0, code)
    code = np.where(a >= 57344.0, 0x7B, code)
    return (code | (np.signbit(x).astype(np.int64) << 7)).astype(np.uint8)


def e_bits(amax_f32):
    b = np.asarray(amax_f32, np.float32).view(np.uint32).astype(np.int64)
    return ((b >> 23) & 255) - 127, b & 0x7FFFFF


# --------------------------------------------------------------------------
# E5M2 codec
# --------------------------------------------------------------------------
def test_e5m2_decode_matches_library_codec_and_printed_range():
    g = golden_values()
    t = O.fp8_decode_all(O.E5M2)
    ref = torch_e5m2_table()
    assert np.array_equal(np.isnan(t), np.isnan(ref))
    fin = ~np.isnan(ref)
    assert np.array_equal(t[fin], ref[fin]) and np.array_equal(np.signbit(t[fin]), np.signbit(ref[fin]))
    assert np.max(t[np.isfinite(t)]) == float(g["e5m2_max"]) == t[0x7B]
    assert int(g["e5m2_has_inf"]) == 1 and t[0x7C] == np.inf and t[0xFC] == -np.inf
    assert t[0x04] == 2.0 ** -14 and t[0x01] == 2.0 ** -16 and t[0x3C] == 1.0
    # the E4M3 table of the generic entry is the pinned E4M3 decoder
    assert np.array_equal(O.fp8_decode_all(O.E4M3), O.e4m3_decode_table(), equal_nan=True)


def test_e5m2_encode_exhaustive_bf16():
    f = (np.arange(65536, dtype=np.uint32) << 16).view(np.float32)
    f = f[np.isfinite(f)]
    assert np.array_equal(O.fp8_encode(f, O.E5M2), brute_encode_e5m2(f.astype(np.float64)))


def test_e5m2_encode_fp32_range():
    """Every fp32 in [2^-19, 2^16] on a stride that hits every mantissa pattern of
    the low bits, plus all values around every tie, against brute force."""
    lo = int(np.float32(2.0 ** -19).view(np.uint32))
    hi = int(np.float32(2.0 ** 16).view(np.uint32))
    b = np.arange(lo, hi + 1, 61, dtype=np.uint32)
    f = b.view(np.float32)
    assert np.array_equal(O.fp8_encode(f, O.E5M2), brute_encode_e5m2(f.astype(np.float64)))
    mags = torch_e5m2_table()[:0x7C]
    mid = ((mags[1:] + mags[:-1]) / 2).astype(np.float32)
    around = np.concatenate([np.nextafter(mid, -np.inf), mid, np.nextafter(mid, np.inf)]).astype(np.float32)
    around = np.concatenate([around, -around])
    assert np.array_equal(O.fp8_encode(around, O.E5M2), brute_encode_e5m2(around.astype(np.float64)))


def test_e5m2_encode_matches_library_cast_below_clip():
    rng = np.random.default_rng(11)
    x = (rng.standard_normal(1 << 20) * rng.choice([1e-6, 1e-3, 1, 300, 3e4], 1 << 20)).astype(np.float32)
    x = x[np.abs(x) < 57344]
    ref = torch.from_numpy(x).to(torch.float8_e5m2).view(torch.uint8).numpy()
    assert np.array_equal(O.fp8_encode(x, O.E5M2), ref)


# --------------------------------------------------------------------------
# scale rules
# --------------------------------------------------------------------------
def test_ceil_rule_for_e5m2_closed_form_and_cases():
    """57344 = 1.75 * 2^15: for a normal amax, e = Ea - 15 + (f > 0x600000)."""
    a = (np.arange(0x0080, 0x7F80, dtype=np.uint32) << 16).view(np.float32)  # every positive normal bf16
    Ea, f = e_bits(a)
    want = np.maximum(Ea - 15 + (f > 0x600000), -29)
    assert np.array_equal(O.scale_exp_fmt(a, O.E5M2, O.SCALE_CEIL, -29), want)
    cases = {57344.0: 0, 57345.0: 1, 28672.0: -1, 28673.0: 0, 1.0: -15, 1e-4: -29, 1e-12: -29, 0.0: -29}
    for amax, e in cases.items():
        assert O.scale_exp_fmt(np.array([amax], np.float32), O.E5M2, O.SCALE_CEIL, -29)[0] == e, amax
    # the 1e-4 amax clamp of the 1x128 rule gives exactly this floor
    g = golden_values()
    clamp = float(g["amax_clamp"])
    assert 57344 * 2.0 ** -30 < clamp <= 57344 * 2.0 ** -29
    # the E4M3 branch is the pinned E4M3 rule
    b = (np.arange(0x0080, 0x7F80, 7, dtype=np.uint32) << 16).view(np.float32)
    assert np.array_equal(O.scale_exp_fmt(b, O.E4M3, O.SCALE_CEIL, -22), O.scale_exp(b, -22))


def test_ocp_floor_rule_bits_and_cases():
    """OCP MX shared exponent: floor(log2 amax) - emax_elem, i.e. the fp32
    exponent field minus 8 (E4M3) or 15 (E5M2); amax * 2^-e lies in
    [2^emax, 2^(emax+1)), so values above the largest finite element clip."""
    a = (np.arange(0x0080, 0x7F80, dtype=np.uint32) << 16).view(np.float32)
    Ea, _ = e_bits(a)
    for fmt, emax in ((O.E4M3, 8), (O.E5M2, 15)):
        e = O.scale_exp_fmt(a, fmt, O.SCALE_OCP_FLOOR, -127)
        assert np.array_equal(e, np.maximum(Ea - emax, -127))
        ok = e > -127
        r = a[ok].astype(np.float64) * np.exp2(-e[ok].astype(np.float64))
        assert np.all((r >= 2.0 ** emax) & (r < 2.0 ** (emax + 1)))
    cases = {448.0: 0, 500.0: 0, 511.9: 0, 512.0: 1, 256.0: 0, 255.9: -1, 1.0: -8}
    for amax, e in cases.items():
        assert O.scale_exp_fmt(np.array([amax], np.float32), O.E4M3, O.SCALE_OCP_FLOOR, -127)[0] == e, amax
    # where both rules exist, the floor rule's exponent never exceeds the ceil rule's
    c = O.scale_exp_fmt(a, O.E4M3, O.SCALE_CEIL, -127)
    fl = O.scale_exp_fmt(a, O.E4M3, O.SCALE_OCP_FLOOR, -127)
    assert np.all((c - fl >= 0) & (c - fl <= 1))


# --------------------------------------------------------------------------
# quantizer, dequantizer, direct transpose and GEMM in either format
# --------------------------------------------------------------------------
def _rows(seed, rows=6, cols=256):
    g = torch.Generator().manual_seed(seed)
    x = torch.randn(rows, cols, generator=g) * torch.exp2(torch.randint(-12, 12, (rows, 1), generator=g).float())
    x[0, :32] = 0.0
    x[1, 5] = 3e4
    return x.to(torch.bfloat16)


def test_quant_rowwise_fmt_brute_force():
    x = _rows(1)
    xb = x.view(torch.int16).numpy().view(np.uint16)
    xv = x.double().numpy()
    for group in (32, 128):
        for fmt in (O.E4M3, O.E5M2):
            for rule in (O.SCALE_CEIL, O.SCALE_OCP_FLOOR):
                q, s = O.quant_rowwise_fmt(xb, group, fmt, rule)
                amax = np.abs(xv).reshape(xv.shape[0], -1, group).max(axis=2).astype(np.float32)
                e = O.scale_exp_fmt(amax, fmt, rule, O.emin_for(group, fmt))
                assert np.array_equal(s, (e + 127).astype(np.uint8))
                scaled = xv * np.exp2(-np.repeat(e, group, axis=1).astype(np.float64))
                want = brute_encode_e5m2(scaled) if fmt == O.E5M2 else __import__("test_oracle_pins").brute_encode(scaled)
                assert np.array_equal(q, want), (group, fmt, rule)
    # E4M3 with the ceil rule is the pinned quantizer
    for group in (32, 128):
        q0, s0 = O.quant_rowwise(xb, group)
        q1, s1 = O.quant_rowwise_fmt(xb, group, O.E4M3, O.SCALE_CEIL)
        assert np.array_equal(q0, q1) and np.array_equal(s0, s1)


def test_floor_rule_saturation_is_the_only_extra_error():
    """With the floor rule the group's largest elements may clip at the element
    maximum; everywhere else the dequantized value is within half a code step
    of x, like the ceil rule."""
    x = _rows(2, rows=16)
    xb = x.view(torch.int16).numpy().view(np.uint16)
    xv = x.double().numpy()
    q, s = O.quant_rowwise_fmt(xb, 32, O.E4M3, O.SCALE_OCP_FLOOR)
    d = O.dequant_fmt(q, s, 32, O.E4M3)
    sc = np.exp2(np.repeat(s.astype(np.int64) - 127, 32, axis=1).astype(np.float64))
    clipped = np.abs(xv) / sc > 448
    assert np.all(np.abs(d[clipped]) == 448 * sc[clipped])
    ok = ~clipped
    rel = np.abs(d[ok] - xv[ok]) <= np.maximum(np.abs(xv[ok]) * 2.0 ** -4, 2.0 ** -10 * sc[ok])
    assert rel.all()


def shift_code_e5m2(c, k):
    """The pages' exponent-shift rule on E5M2 integer fields: exponent field
    minus k while it stays >= 1, else the integer magnitude (units of 2^-16)
    shifted right by k with round-to-nearest-even."""
    s, E, m = c & 0x80, (c >> 2) & 31, c & 3
    if k == 0:
        return c
    if E - k >= 1:
        return s | ((E - k) << 2) | m
    mag = m if E == 0 else (4 + m) << (E - 1)
    q, r = mag >> k, mag & ((1 << k) - 1)
    half = 1 << (k - 1)
    if r > half or (r == half and (q & 1)):
        q += 1
    return s | q


def test_direct_transpose_e5m2_is_the_exponent_shift():
    """All finite E5M2 codes x shifts k in [0, 40]: the oracle's requantization
    at the block-max scale equals the integer-field exponent shift."""
    codes = np.array([c for c in range(256) if ((c >> 2) & 31) != 31], np.uint8)
    for k in range(0, 41):
        # one 128x128 block: row 0 holds the block maximum scale, row 1 the shifted codes
        q = np.zeros((128, 128), np.uint8)
        s = np.full((128, 1), 127 - k, np.uint8)
        s[0] = 127
        n = len(codes)
        for i0 in range(0, n, 128):
            blk = codes[i0:i0 + 128]
            q[1, :len(blk)] = blk
            qt, st = O.direct_transpose_fmt(q, s, O.E5M2)
            assert np.all(st == 127)
            want = np.array([shift_code_e5m2(int(c), k) for c in blk], np.uint8)
            assert np.array_equal(qt[:len(blk), 1], want), k
    # E4M3 codes through the generic entry match the pinned direct transpose
    rng = np.random.default_rng(3)
    q = rng.integers(0, 256, (256, 256), dtype=np.uint8)
    q[(q & 0x7F) == 0x7F] = 0
    s = rng.integers(110, 140, (256, 2), dtype=np.uint8)
    a = O.direct_transpose(q, s)
    b = O.direct_transpose_fmt(q, s, O.E4M3)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


def test_gemm_fmt_exact_rationals():
    """E5M2 A x E4M3 B (a gradient times an activation or weight): every
    product and sum in exact rationals on a tiny shape; the oracle's fp64
    sums stay within the fp64 summation bound K * 2^-53 * sum |p|."""
    rng = np.random.default_rng(5)
    M, N, K = 3, 4, 256
    a = rng.integers(0, 256, (M, K), dtype=np.uint8)
    a[((a >> 2) & 31) == 31] = 0x3C
    b = rng.integers(0, 256, (N, K), dtype=np.uint8)
    b[(b & 0x7F) == 0x7F] = 0x38
    sa = rng.integers(120, 134, (M, K // 128), dtype=np.uint8)
    sb = rng.integers(120, 134, (N, K // 128), dtype=np.uint8)
    t5 = torch_e5m2_table()
    t4 = O.e4m3_decode_table()
    mi, ni = np.repeat(np.arange(M), N), np.tile(np.arange(N), M)
    got = O.block_gemm_fmt_sampled(a, sa, O.ROW1x128, O.E5M2, b, sb, O.ROW1x128, O.E4M3, mi, ni)
    for i, (m, n) in enumerate(zip(mi, ni)):
        tot, mag = Fraction(0), Fraction(0)
        for k in range(K):
            p = Fraction(t5[a[m, k]]) * Fraction(t4[b[n, k]]) * Fraction(2) ** (int(sa[m, k // 128]) + int(sb[n, k // 128]) - 254)
            tot += p
            mag += abs(p)
        assert abs(Fraction(got[i]) - tot) <= K * Fraction(1, 2 ** 53) * mag
    # both operands E4M3: the pinned GEMM
    a4 = a.copy()
    a4[(a4 & 0x7F) == 0x7F] = 0x38
    ref = O.block_gemm(a4, sa, O.ROW1x128, b, sb, O.ROW1x128)
    assert np.array_equal(O.block_gemm_fmt_sampled(a4, sa, O.ROW1x128, O.E4M3, b, sb, O.ROW1x128, O.E4M3, mi, ni),
                          ref[mi, ni])


def test_mx2_floor_rule_is_level1_then_floor_rule_quant():
    """Two-level quantization with the MX standard's level-2 rule: level 1 is
    the pinned fp32 alpha1 = amax/448 and y = fp32(x / alpha1) (numpy fp32
    division here), level 2 the floor-rule quantization of y in 32-groups
    (the pinned quantizer above); the ceil variant is the pinned orc_mx2_quant."""
    g = torch.Generator().manual_seed(9)
    R, Cc, g1 = 5, 1024 + 96, 512
    w = (torch.randn(R, Cc, generator=g) * 0.02 * torch.exp2(torch.randint(-6, 6, (R, 1), generator=g).float()))
    w = w.to(torch.bfloat16)
    wb = w.view(torch.int16).numpy().view(np.uint16)
    wf = w.float().numpy()
    q, s2, s1 = O.mx2_quant(wb, g1, O.SCALE_OCP_FLOOR)
    q0, s20, s10 = O.mx2_quant(wb, g1)
    assert np.array_equal(s1, s10)
    ng = s1.shape[1]
    for r in range(R):
        for gi in range(ng):
            c0, c1 = gi * g1, min((gi + 1) * g1, Cc)
            amax = np.float32(np.abs(wf[r, c0:c1]).max())
            alpha = np.float32(amax / np.float32(448)) if amax > 0 else np.float32(1)
            assert s1[r, gi] == alpha
            y = (wf[r, c0:c1] / alpha).astype(np.float32)[None, :]
            qy, sy = O.quant_rowwise_fmt(y, 32, O.E4M3, O.SCALE_OCP_FLOOR)
            assert np.array_equal(q[r, c0:c1], qy[0]) and np.array_equal(s2[r, c0 // 32:c1 // 32], sy[0])
            qc, sc = O.quant_rowwise_fmt(y, 32, O.E4M3, O.SCALE_CEIL)
            assert np.array_equal(q0[r, c0:c1], qc[0]) and np.array_equal(s20[r, c0 // 32:c1 // 32], sc[0])
