"""Pins of the oracle's grouped-GEMM, run-bound and dequantization helpers,
each against a reference built here from something other than the oracle:
torch's float8 codecs (a library decoder) and numpy fp64 matrix products of
the dequantized operands.

- orc_grouped_gemm_sampled: the M-grouped contiguous layout of
  llm-infra-atlas "01 · DeepSeek FP8 and DeepGEMM: Hopper software recipe"
  §5.6 (experts concatenated along M, each segment multiplied by its own
  expert's weights and 128x128 scales, §3 scale shapes).  A wrong segment
  lookup, a wrong per-expert B or SB offset, or a missed partial 128-row B
  block (N = 2112, the §5.7 shape) changes sampled values and fails here.
- orc_gemm_run_bounds(_fmt)_sampled: the plain definitions of its two sums
  (per-run maximum of |scaled product| summed over runs of 8 K, and the sum
  of |scaled product|), evaluated with numpy.
- orc_dequant's BLOCK128 and ROW1x32 index paths: decode times 2^(s - 127)
  with the scale broadcast by numpy.
"""
import numpy as np
import pytest
import torch

import oracle as O


def decode_table(fmt=0):
    """Code -> value by torch's float8 dtypes (a library implementation)."""
    c = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    dt = torch.float8_e5m2 if fmt == 1 else torch.float8_e4m3fn
    return c.view(dt).to(torch.float64).numpy()


def rand_codes(rng, shape, fmt=0):
    q = rng.integers(0, 256, shape).astype(np.uint8)
    if fmt == 1:
        q[(q & 0x7C) == 0x7C] &= 0x83  # no Inf/NaN codes in E5M2
    else:
        q[(q & 0x7F) == 0x7F] ^= 0x01  # no NaN codes in E4M3
    return q


def deq_row(q, s, g, tab):
    """Row-wise 1 x g scales broadcast along K."""
    return tab[q] * np.ldexp(1.0, np.repeat(s.astype(np.int64) - 127, g, axis=1))


def deq_block(q, s, tab):
    """128 x 128 block scales broadcast over rows (partial last block) and K."""
    rows = q.shape[0]
    e = np.repeat(np.repeat(s.astype(np.int64) - 127, 128, axis=0)[:rows], 128, axis=1)
    return tab[q] * np.ldexp(1.0, e)


def test_grouped_gemm_sampled_against_per_expert_dequantized_matmul():
    rng = np.random.default_rng(71)
    G, N, K = 5, 2112, 384
    lens = [48, 0, 144, 16, 96]  # segments as permute_pad lays them out, with an empty expert
    off = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    M_cap = int(off[-1]) + 32  # rows past off[G]: padding bound, outside every segment
    a = rand_codes(rng, (M_cap, K))
    sa = rng.integers(112, 142, (M_cap, K // 128)).astype(np.uint8)
    b = rand_codes(rng, (G, N, K))
    sb = rng.integers(112, 142, (G, (N + 127) // 128, K // 128)).astype(np.uint8)
    tab = decode_table()
    A = deq_row(a, sa, 128, tab)
    ref_rows = {}
    for g in range(G):
        if lens[g] == 0:
            continue
        Bg = deq_block(b[g], sb[g], tab)
        ref_rows[g] = A[off[g]:off[g + 1]] @ Bg.T
    cols = np.array([0, 1, 127, 128, 255, 1024, 2047, 2048, 2100, 2111], np.int64)
    mi = np.repeat(np.arange(M_cap, dtype=np.int64), cols.size)
    ni = np.tile(cols, M_cap)
    got = O.grouped_gemm_sampled(a, sa, b, sb, off, mi, ni)
    scale = max(np.max(np.abs(r)) for r in ref_rows.values())
    for i, (m, n) in enumerate(zip(mi, ni)):
        g = int(np.searchsorted(off, m, side="right")) - 1
        if m >= off[-1]:
            assert np.isnan(got[i]), (m, n)
            continue
        assert lens[g] > 0
        want = ref_rows[g][m - off[g], n]
        assert abs(got[i] - want) <= 1e-12 * scale, (m, n, got[i], want)
    # another expert's weights give other values at the segment edges
    for g in (0, 2, 3):
        m = int(off[g + 1]) - 1
        other = (g + 2) % G
        if lens[other] == 0:
            continue
        alt = (A[m] @ deq_block(b[other], sb[other], tab).T)[cols]
        assert not np.allclose(alt, got[(mi == m)]), g


def _run_bounds_ref(A, B, run=8, l1=None):
    M, K = A.shape
    N = B.shape[0]
    rm = np.zeros((M, N))
    asum = np.zeros((M, N))
    for m in range(M):
        P = np.abs(A[m][None, :] * B)  # [N, K]
        asum[m] = P.sum(axis=1)
        rm[m] = P.reshape(N, K // run, run).max(axis=2).sum(axis=1)
    if l1 is not None:
        rm *= np.abs(l1.astype(np.float64))[None, :]
        asum *= np.abs(l1.astype(np.float64))[None, :]
    return rm, asum


@pytest.mark.parametrize("layout", ["1d2d", "1d1d", "mx32_l1"])
def test_run_bounds_against_numpy_definition(layout):
    rng = np.random.default_rng(72)
    M, N, K = 3, 200, 256
    a = rand_codes(rng, (M, K))
    b = rand_codes(rng, (N, K))
    tab = decode_table()
    l1 = None
    if layout == "1d2d":
        sa = rng.integers(118, 136, (M, K // 128)).astype(np.uint8)
        sb = rng.integers(118, 136, ((N + 127) // 128, K // 128)).astype(np.uint8)
        A, B, ag, bg = deq_row(a, sa, 128, tab), deq_block(b, sb, tab), O.ROW1x128, O.BLOCK128
    elif layout == "1d1d":
        sa = rng.integers(118, 136, (M, K // 128)).astype(np.uint8)
        sb = rng.integers(118, 136, (N, K // 128)).astype(np.uint8)
        A, B, ag, bg = deq_row(a, sa, 128, tab), deq_row(b, sb, 128, tab), O.ROW1x128, O.ROW1x128
    else:
        sa = rng.integers(118, 136, (M, K // 32)).astype(np.uint8)
        sb = rng.integers(118, 136, (N, K // 32)).astype(np.uint8)
        A, B, ag, bg = deq_row(a, sa, 32, tab), deq_row(b, sb, 32, tab), O.ROW1x32, O.ROW1x32
        l1 = (rng.standard_normal(N) * 3).astype(np.float32)
    rm_ref, as_ref = _run_bounds_ref(A, B, 8, l1)
    mi = np.repeat(np.arange(M, dtype=np.int64), N)
    ni = np.tile(np.arange(N, dtype=np.int64), M)
    rm, asum = O.gemm_run_bounds_sampled(a, sa, ag, b, sb, bg, mi, ni, run=8, b_l1=l1)
    np.testing.assert_allclose(rm, rm_ref[mi, ni], rtol=1e-13, atol=0)
    np.testing.assert_allclose(asum, as_ref[mi, ni], rtol=1e-13, atol=0)
    # the run maximum lies between the mean and the sum of a run's products
    assert np.all(rm <= asum * (1 + 1e-15)) and np.all(rm * 8 >= asum * (1 - 1e-15))
    # runs of 16 give a different (smaller or equal) first sum, same second sum
    rm16, as16 = O.gemm_run_bounds_sampled(a, sa, ag, b, sb, bg, mi, ni, run=16, b_l1=l1)
    rm16_ref, _ = _run_bounds_ref(A, B, 16, l1)
    np.testing.assert_allclose(rm16, rm16_ref[mi, ni], rtol=1e-13, atol=0)
    np.testing.assert_allclose(as16, asum, rtol=1e-13, atol=0)


def test_run_bounds_fmt_e5m2_against_numpy_definition():
    rng = np.random.default_rng(73)
    M, N, K = 2, 130, 256
    a = rand_codes(rng, (M, K), fmt=1)
    b = rand_codes(rng, (N, K))
    sa = rng.integers(110, 130, (M, K // 128)).astype(np.uint8)
    sb = rng.integers(118, 136, ((N + 127) // 128, K // 128)).astype(np.uint8)
    A = deq_row(a, sa, 128, decode_table(1))
    B = deq_block(b, sb, decode_table(0))
    rm_ref, as_ref = _run_bounds_ref(A, B, 8)
    mi = np.repeat(np.arange(M, dtype=np.int64), N)
    ni = np.tile(np.arange(N, dtype=np.int64), M)
    rm, asum = O.gemm_run_bounds_fmt_sampled(a, sa, O.ROW1x128, 1, b, sb, O.BLOCK128, 0, mi, ni)
    np.testing.assert_allclose(rm, rm_ref[mi, ni], rtol=1e-13, atol=0)
    np.testing.assert_allclose(asum, as_ref[mi, ni], rtol=1e-13, atol=0)


def test_dequant_block128_and_row1x32_index_paths():
    rng = np.random.default_rng(74)
    tab = decode_table()
    # 128x128 blocks with a partial last row block (200 = 128 + 72)
    q = rand_codes(rng, (200, 384))
    s = rng.integers(0, 256, (2, 3)).astype(np.uint8)  # includes byte 0 (2^-127) and large bytes
    s[0, 0], s[1, 2] = 0, 254
    out = O.dequant(q, s, O.BLOCK128)
    assert np.array_equal(out, deq_block(q, s, tab))
    # block (1, 2) owns rows 128..199 and columns 256..383
    assert np.array_equal(out[150, 300], tab[q[150, 300]] * 2.0 ** (254 - 127))
    assert np.array_equal(out[5, 5], tab[q[5, 5]] * 2.0 ** -127)
    # 1 x 32 groups
    q = rand_codes(rng, (7, 256))
    s = rng.integers(0, 256, (7, 8)).astype(np.uint8)
    out = O.dequant(q, s, O.ROW1x32)
    assert np.array_equal(out, deq_row(q, s, 32, tab))
    assert np.array_equal(out[3, 33], tab[q[3, 33]] * np.ldexp(1.0, int(s[3, 1]) - 127))
