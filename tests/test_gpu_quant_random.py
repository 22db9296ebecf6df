"""Seeded random sweep of the quantizers, the scaling-aware transposes and
MOSS against the oracle, bit for bit: random shapes (ragged row counts,
partial 128-row weight blocks, one group up to many per row), bf16 and fp32
inputs whose rows span 2^-30..2^30 in magnitude, with all-zero rows and
32-element groups 2^-60 below the rest of their row; both element formats
and both scale rules of the row-wise quantizer; row-wise and 128x128-block
scales in the transposes; random level-1 group sizes in MOSS."""
import numpy as np
import pytest
import torch

import oracle as O
from test_gpu_parity import DEV, bits, np_, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def fgb():
    import fine_grained_blockwise_amd as m
    return m


def _values(rng, rows, cols, seed):
    """N(0,1) rows times 2^u, u uniform in [-30, 30]; an all-zero row and a
    32-element group scaled down by 2^-60."""
    g = torch.Generator().manual_seed(seed)
    x = torch.randn(rows, cols, generator=g, dtype=torch.float64)
    x *= torch.from_numpy(np.exp2(rng.uniform(-30, 30, (rows, 1))))
    if rows > 2:
        x[int(rng.integers(0, rows))] = 0.0
        r = int(rng.integers(0, rows))
        c = 32 * int(rng.integers(0, cols // 32))
        x[r, c:c + 32] *= 2.0 ** -60
    return x


def _as(x, dtype):
    """The tensor in dtype and its oracle input (bf16 bits or fp32)."""
    t = x.to(dtype)
    return t, (bits(t) if dtype == torch.bfloat16 else t.numpy())


def test_random_rowwise_and_block_quant(fgb):
    rng = np.random.default_rng(99)
    for case in range(20):
        group = (32, 128)[int(rng.integers(0, 2))]
        rows, cols = int(rng.integers(1, 601)), group * int(rng.integers(1, 25))
        dtype = (torch.bfloat16, torch.float32)[int(rng.integers(0, 2))]
        fmt, rule = int(rng.integers(0, 2)), int(rng.integers(0, 2))
        say(f"random quant {case}: rows={rows} cols={cols} group={group} {dtype} fmt={fmt} rule={rule}")
        t, ox = _as(_values(rng, rows, cols, 100 + case), dtype)
        q, s = fgb.fp8_quant_rowwise_fmt(t.to(DEV), group, fmt, rule)
        oq, os_ = O.quant_rowwise_fmt(ox, group, fmt, rule)
        assert np.array_equal(np_(s), os_) and np.array_equal(np_(q), oq), case
        if fmt == 0 and rule == 0:  # the plain entry point is the same quantizer
            q2, s2 = fgb.fp8_quant_rowwise(t.to(DEV), group)
            assert np.array_equal(np_(s2), os_) and np.array_equal(np_(q2), oq), case
        if cols % 128 == 0:  # 128x128 weight blocks, the last one possibly partial
            wq, ws = fgb.fp8_quant_blockwise(t.to(DEV))
            owq, ows = O.quant_blockwise(ox)
            assert np.array_equal(np_(ws), ows) and np.array_equal(np_(wq), owq), case


def test_random_direct_transposes(fgb):
    rng = np.random.default_rng(7)
    for case in range(12):
        T, C = 128 * int(rng.integers(1, 9)), 128 * int(rng.integers(1, 9))
        say(f"random direct transpose {case}: T={T} C={C}")
        t, ox = _as(_values(rng, T, C, 300 + case), torch.bfloat16)
        # row-wise E4M3 codes -> column-wise copy by exponent shifts
        xq, xs = O.quant_rowwise(ox, 128)
        qt, st = fgb.fp8_direct_transpose(torch.from_numpy(xq).to(DEV), torch.from_numpy(xs).to(DEV))
        oqt, ost = O.direct_transpose(xq, xs)
        assert np.array_equal(np_(st), ost) and np.array_equal(np_(qt), oqt), case
        # E5M2 codes
        eq, es = O.quant_rowwise_fmt(ox, 128, 1, 0)
        qt, st = fgb.fp8_direct_transpose_fmt(torch.from_numpy(eq).to(DEV), torch.from_numpy(es).to(DEV), fgb.E5M2)
        oqt, ost = O.direct_transpose_fmt(eq, es, 1)
        assert np.array_equal(np_(st), ost) and np.array_equal(np_(qt), oqt), case
        # 128x128 weight blocks: the exact byte transpose
        wq, ws = O.quant_blockwise(ox)
        qt, st = fgb.fp8_direct_transpose(torch.from_numpy(wq).to(DEV), torch.from_numpy(ws).to(DEV), fgb.BLOCK128)
        oqt, ost = O.block_transpose(wq, ws)
        assert np.array_equal(np_(st), ost) and np.array_equal(np_(qt), oqt), case


def test_random_moss(fgb):
    rng = np.random.default_rng(5)
    for case in range(12):
        R, C = int(rng.integers(1, 301)), 32 * int(rng.integers(1, 97))
        g1 = 32 * int(rng.integers(1, 65)) if rng.random() < 0.7 else 10240
        rule = int(rng.integers(0, 2))
        say(f"random moss {case}: R={R} C={C} g1={g1} rule={rule}")
        t, ox = _as(_values(rng, R, C, 500 + case), torch.bfloat16)
        q, s2, s1 = fgb.mx2_quant_rule(t.to(DEV), g1, rule)
        oq, os2, os1 = O.mx2_quant(ox, g1, rule)
        assert np.array_equal(np_(s1).view(np.uint32), os1.view(np.uint32)), case
        assert np.array_equal(np_(s2), os2) and np.array_equal(np_(q), oq), case
        x = fgb.mx2_dequant(q, s2, s1, g1)
        assert np.array_equal(np_(x).view(np.uint32), O.mx2_dequant(oq, os2, os1, g1).view(np.uint32)), case
