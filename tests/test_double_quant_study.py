"""Double quantization: the three-pass conversion (dequantize, transpose,
requantize) against the scaling-aware direct transpose, with power-of-two
scales and with the fp32 sf = amax/448 scales.  CPU only, on the oracle.

awesome-system-papers, "FP8-Flow-MoE: A Casting-Free FP8 Recipe without Double
Quantization Error (MLSys 2026)": the row-wise and column-wise copies of a
tensor carry different scales, and converting one into the other through
dequantize -> transpose -> requantize rounds every value twice; with
power-of-two scales the conversion is an exponent shift inside each 128x128
block ("Core method").  Error is measured against the bf16 input as SNR (dB).
"""
import numpy as np
import torch

import oracle as O
import synth


def _snr(ref, approx):
    ref = ref.astype(np.float64)
    return 10 * np.log10((ref ** 2).sum() / ((ref - approx.astype(np.float64)) ** 2).sum())


def test_double_quantization_study():
    X, _, _ = synth.linear_dsv3(0, T=512, Cin=1024, Cout=128)  # 1% Student-t channels
    x = X.float().numpy()
    xt = np.ascontiguousarray(x.T)
    # power-of-two scales
    q, s = O.quant_rowwise(x)
    single_p2 = O.dequant(*O.quant_rowwise(xt), O.ROW1x128)   # quantize the transposed input once
    direct = O.dequant(*O.direct_transpose(q, s), O.ROW1x128)
    naive_p2 = O.dequant(*O.naive_transpose(q, s), O.ROW1x128)
    # sf = amax / 448
    qf, sf = O.quant_rowwise_sf(x)
    single_sf = O.dequant_sf(*O.quant_rowwise_sf(xt))
    naive_sf = O.dequant_sf(*O.naive_transpose_sf(qf, sf))
    res = {
        "single quantization, pow2": _snr(xt, single_p2),
        "direct transpose, pow2": _snr(xt, direct),
        "three passes, pow2": _snr(xt, naive_p2),
        "single quantization, sf": _snr(xt, single_sf),
        "three passes, sf": _snr(xt, naive_sf),
    }
    for k, v in res.items():
        print(f"  {k:32s} {v:9.5f} dB")
    # with sf scales the second rounding costs accuracy against one rounding
    assert res["three passes, sf"] < res["single quantization, sf"]
    # with pow2 scales the three-pass scales never exceed the direct block scales
    assert res["three passes, pow2"] >= res["direct transpose, pow2"]
