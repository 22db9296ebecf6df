"""Seeded random sweep of the GEMM entry points against the oracle (exact
mode): random M, N, K (K = 0 included) over every scale layout (1x128 A with
128x128 or 1x128 B, 1x32 on both sides with and without level-1 factors),
FP32 or BF16 output, accumulation into D, row-padded D (ldd > N; the columns
past N must stay untouched), and the M-grouped form with random, possibly
empty or ragged, expert segments (rows past the last segment untouched).
Every output element is checked, to the tolerance of the parity tests."""
import numpy as np
import pytest
import torch

import oracle as O
from test_gpu_parity import DEV, check_gemm, np_, rand_codes, rand_scales, say

pytestmark = pytest.mark.gpu

FILL = 5.0  # the value D holds where the GEMM must not write
FILL_BF16 = np.uint16(0x40A0)  # 5.0 as a bf16 bit pattern


@pytest.fixture(scope="module")
def fgb():
    import fine_grained_blockwise_amd as m
    return m


def _dense_case(fgb, rng, case):
    M, N = int(rng.integers(1, 521)), int(rng.integers(1, 521))
    K = 128 * int(rng.integers(0, 7))
    layout = ("1d2d", "1d1d", "mx", "mx_l1")[int(rng.integers(0, 4))]
    bf16 = bool(rng.integers(0, 2))
    acc = (not bf16) and bool(rng.random() < 0.4)
    pad = (0, 8, 40)[int(rng.integers(0, 3))]
    say(f"random dense gemm {case}: M={M} N={N} K={K} {layout} {'bf16' if bf16 else 'f32'} acc={acc} pad={pad}")
    seed = 1000 + 10 * case
    a, b = rand_codes((M, K), seed), rand_codes((N, K), seed + 1)
    l1 = None
    if layout in ("mx", "mx_l1"):
        ag = bg = fgb.ROW1x32
        oag = obg = O.ROW1x32
        sa, sb = rand_scales((M, K // 32), -10, 10, seed + 2), rand_scales((N, K // 32), -10, 10, seed + 3)
        if layout == "mx_l1":
            l1 = torch.rand(N, generator=torch.Generator().manual_seed(seed + 4)) * 2 + 0.1
    else:
        ag, oag = fgb.ROW1x128, O.ROW1x128
        sa = rand_scales((M, K // 128), -10, 10, seed + 2)
        if layout == "1d2d":
            bg, obg = fgb.BLOCK128, O.BLOCK128
            sb = rand_scales(((N + 127) // 128, K // 128), -10, 10, seed + 3)
        else:
            bg, obg = fgb.ROW1x128, O.ROW1x128
            sb = rand_scales((N, K // 128), -10, 10, seed + 3)
    dt = torch.bfloat16 if bf16 else torch.float32
    if acc:
        base = torch.randn((M, N + pad), generator=torch.Generator().manual_seed(seed + 5)) + 3.0  # no -0.0
        full = base.clone().to(DEV)
    else:
        full = torch.full((M, N + pad), FILL, dtype=dt, device=DEV)
    fgb.fp8_block_gemm(a.to(DEV), sa.to(DEV), ag, b.to(DEV), sb.to(DEV), bg,
                       b_l1=None if l1 is None else l1.to(DEV), g1=10240 if l1 is not None else 0,
                       d=full[:, :N], accumulate=acc, mode=fgb.GEMM_EXACT)
    got = np_(full)
    # columns past N untouched
    if acc:
        assert np.array_equal(got[:, N:], base.numpy()[:, N:]), case
    else:
        assert np.all(got[:, N:] == (FILL_BF16 if bf16 else np.float32(FILL))), case
    got = got[:, :N]
    if K == 0:  # the empty sum
        if acc:
            assert np.array_equal(got, base.numpy()[:, :N]), case
        else:
            assert np.all(got == 0), case
        return
    ref = O.block_gemm(a.numpy(), sa.numpy(), oag, b.numpy(), sb.numpy(), obg,
                       None if l1 is None else l1.numpy().reshape(N, 1), 10240 if l1 is not None else 0)
    if acc:
        # D = fl32(base + acc): the accumulator within the tolerance, then one fp32 rounding of the sum
        want = base.numpy()[:, :N].astype(np.float64) + ref
        err = np.abs(got.astype(np.float64) - want)
        bound = 1e-5 * np.max(np.abs(ref)) + np.spacing(np.abs(want).astype(np.float32)).astype(np.float64)
        assert np.all(err <= bound), (case, float(np.max(err - bound)))
    else:
        check_gemm(got, ref, "exact", bf16, None, K)


def _grouped_case(fgb, rng, case):
    G = int(rng.integers(1, 7))
    lens = rng.integers(0, 301, G)
    lens[rng.random(G) < 0.25] = 0  # some experts empty
    off = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    used = int(off[-1])
    M_cap = used + int(rng.integers(0, 51))
    N, K = int(rng.integers(1, 521)), 128 * int(rng.integers(1, 7))
    bf16 = bool(rng.integers(0, 2))
    say(f"random grouped gemm {case}: G={G} segments={lens.tolist()} M_cap={M_cap} N={N} K={K} "
        f"{'bf16' if bf16 else 'f32'}")
    seed = 5000 + 10 * case
    a = rand_codes((M_cap, K), seed)
    sa = rand_scales((M_cap, K // 128), -8, 8, seed + 1)
    b = rand_codes((G, N, K), seed + 2)
    sb = rand_scales((G, (N + 127) // 128, K // 128), -8, 8, seed + 3)
    dt = torch.bfloat16 if bf16 else torch.float32
    d = torch.full((M_cap, N), FILL, dtype=dt, device=DEV)
    fgb.fp8_grouped_gemm(a.to(DEV), sa.to(DEV), b.to(DEV), sb.to(DEV), torch.from_numpy(off).to(DEV), d=d,
                         mode=fgb.GEMM_EXACT)
    got = np_(d)
    assert np.all(got[used:] == (FILL_BF16 if bf16 else np.float32(FILL))), case
    if used == 0:
        return
    mi, ni = np.repeat(np.arange(used), N), np.tile(np.arange(N), used)
    ref = O.grouped_gemm_sampled(a.numpy(), sa.numpy(), b.numpy(), sb.numpy(), off, mi, ni).reshape(used, N)
    check_gemm(got[:used], ref, "exact", bf16, None, K)


def test_random_dense_gemms(fgb):
    rng = np.random.default_rng(20261203)
    for case in range(24):
        _dense_case(fgb, rng, case)


def test_random_grouped_gemms(fgb):
    rng = np.random.default_rng(31)
    for case in range(10):
        _grouped_case(fgb, rng, case)
