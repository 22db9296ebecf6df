"""The row-parallel oracle runner (oracle/parallel.py) gives bit for bit the
single-threaded oracle's results, on inputs whose row counts are not
multiples of the slicing (ragged last slices) and with more threads than
slices."""
import numpy as np
import torch

import oracle as O
import oracle.parallel as P
import synth


def _bits(t):
    return synth.bf16_bits(t)


def test_parallel_quantizers_and_transpose_match_one_thread():
    X, W, _ = synth.linear_dsv3(0, T=1000, Cin=1024, Cout=300)
    xb, wb = _bits(X), _bits(W)
    for threads in (1, 3, 16):
        for g in (128, 32):
            q1, s1 = O.quant_rowwise(xb, g)
            qp, sp = P.quant_rowwise_par(xb, g, threads)
            assert np.array_equal(q1, qp) and np.array_equal(s1, sp), (threads, g)
        q1, s1 = O.quant_blockwise(wb)
        qp, sp = P.quant_blockwise_par(wb, threads)
        assert np.array_equal(q1, qp) and np.array_equal(s1, sp), threads
    q, s = synth.wgrad_codes(1152, 512, 0, 41)
    t1, st1 = O.direct_transpose(q.numpy(), s.numpy())
    for threads in (2, 5, 16):
        tp, stp = P.direct_transpose_par(q.numpy(), s.numpy(), threads)
        assert np.array_equal(t1, tp) and np.array_equal(st1, stp), threads


def test_parallel_gemm_and_moe_ops_match_one_thread():
    rng = np.random.default_rng(5)
    X, W, _ = synth.linear_dsv3(0, T=300, Cin=512, Cout=260)
    xq, xs = O.quant_rowwise(_bits(X))
    wq, ws = O.quant_blockwise(_bits(W))
    mi, ni = rng.integers(0, 300, 1001), rng.integers(0, 260, 1001)
    r1 = O.block_gemm_sampled(xq, xs, O.ROW1x128, wq, ws, O.BLOCK128, mi, ni)
    rp = P.block_gemm_sampled_par(xq, xs, O.ROW1x128, wq, ws, O.BLOCK128, mi, ni, threads=7)
    assert np.array_equal(r1.view(np.uint64), rp.view(np.uint64))
    Xm, idx, probs, _, _ = synth.moe(0, T=257, H=256, E=8, weights=False)
    xmq, xms = O.quant_rowwise(_bits(Xm))
    _, _, rm, _, used = O.permute_pad(xmq, xms, idx, 8, 16)
    y = _bits(torch.randn(used, 256).to(torch.bfloat16))
    assert np.array_equal(O.unpermute_unpad(y, rm, probs), P.unpermute_unpad_par(y, rm, probs, 6))
    h = _bits((torch.randn(333, 512) * 3).to(torch.bfloat16))
    for a, b in zip(O.swiglu_quant(h), P.swiglu_quant_par(h, 4)):
        assert np.array_equal(a, b)
    hq, hs = O.quant_rowwise(h)
    da = _bits(torch.randn(333, 256).to(torch.bfloat16))
    for a, b in zip(O.dswiglu_quant(hq, hs, da), P.dswiglu_quant_par(hq, hs, da, 5)):
        assert np.array_equal(a, b)
    Wm, _ = synth.moss(0, R=37, C=20480 + 512, M=1)
    for a, b in zip(O.mx2_quant(_bits(Wm), 10240), P.mx2_quant_par(_bits(Wm), 10240, 4)):
        assert np.array_equal(a.view(np.uint8), b.view(np.uint8))
