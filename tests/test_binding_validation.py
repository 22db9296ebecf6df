"""The Python binding rejects malformed tensors before any device check or
launch: wrong shapes, dtypes or layouts of codes, scales and outputs raise
ValueError, so a bad call can never reach a kernel that would index past a
buffer.  CPU tensors are enough: the shape checks run first."""
import pytest
import torch

fgb = pytest.importorskip("fine_grained_blockwise_amd")

u8 = torch.uint8


def z(*shape, dtype=u8):
    return torch.zeros(shape, dtype=dtype)


def raises(fn, match):
    with pytest.raises(ValueError, match=match):
        fn()


def test_block_gemm_scale_shapes_and_output():
    M, N, K = 256, 384, 512
    a, b = z(M, K), z(N, K)
    sa, sb = z(M, K // 128), z((N + 127) // 128, K // 128)
    raises(lambda: fgb.fp8_block_gemm(a, z(M, K // 128 - 1), fgb.ROW1x128, b, sb, fgb.BLOCK128), "sa must have shape")
    raises(lambda: fgb.fp8_block_gemm(a, sa, fgb.ROW1x128, b, z(N, K // 128), fgb.BLOCK128), "sb must have shape")
    raises(lambda: fgb.fp8_block_gemm(a, sa, fgb.ROW1x128, b, sb, fgb.ROW1x128), "sb must have shape")
    raises(lambda: fgb.fp8_block_gemm(a, z(M, K // 32), fgb.ROW1x128, b, sb, fgb.BLOCK128), "sa must have shape")
    raises(lambda: fgb.fp8_block_gemm(a, sa.float(), fgb.ROW1x128, b, sb, fgb.BLOCK128), "dtype")
    raises(lambda: fgb.fp8_block_gemm(a.float(), sa, fgb.ROW1x128, b, sb, fgb.BLOCK128), "dtype")
    raises(lambda: fgb.fp8_block_gemm(a, sa, fgb.ROW1x128, z(N, K + 128), sb, fgb.BLOCK128), "same K")
    raises(lambda: fgb.fp8_block_gemm(a, sa, fgb.ROW1x128, b, sb, fgb.BLOCK128, d=z(M, N - 1, dtype=torch.float32)),
           "d must have shape")
    raises(lambda: fgb.fp8_block_gemm(a, sa, fgb.ROW1x128, b, sb, fgb.BLOCK128, d=z(M, N, dtype=torch.float16)),
           "output dtype")
    raises(lambda: fgb.fp8_block_gemm(a, sa, fgb.ROW1x128, b, sb, fgb.BLOCK128, out_dtype=torch.int32),
           "output dtype")
    raises(lambda: fgb.fp8_block_gemm(a, sa, fgb.ROW1x128, b, sb, fgb.BLOCK128, b_l1=z(N - 1, dtype=torch.float32)),
           "b_l1 must have shape")
    raises(lambda: fgb.fp8_block_gemm(a, sa, fgb.ROW1x128, b, sb, fgb.BLOCK128, b_l1=z(N, dtype=torch.float32)),
           "1x32 B scales")
    # well-formed CPU tensors get as far as the device check
    raises(lambda: fgb.fp8_block_gemm(a, sa, fgb.ROW1x128, b, sb, fgb.BLOCK128), "on the GPU")


def test_block_gemm_fmt_checks():
    M, N, K = 128, 128, 256
    raises(lambda: fgb.fp8_block_gemm_fmt(z(M, K), z(M, K // 128), fgb.ROW1x128, fgb.E5M2, z(N, K),
                                          z(N, K // 128), fgb.BLOCK128), "sb must have shape")


def test_grouped_gemm_checks():
    G, M_cap, N, K = 4, 1024, 384, 256
    a, sa = z(M_cap, K), z(M_cap, K // 128)
    b, sb = z(G, N, K), z(G, (N + 127) // 128, K // 128)
    off = z(G + 1, dtype=torch.int32)
    ok = dict(a=a, sa=sa, b=b, sb=sb, group_offsets=off)

    def call(**kw):
        args = dict(ok)
        args.update(kw)
        return lambda: fgb.fp8_grouped_gemm(**args)

    raises(call(b=z(G, N, K + 128)), "b must have shape")
    raises(call(sb=z(G, N, K // 128)), "sb must have shape")
    raises(call(sa=z(M_cap - 16, K // 128)), "sa must have shape")
    raises(call(group_offsets=z(G, dtype=torch.int32)), "group_offsets must have shape")
    raises(call(group_offsets=z(G + 1, dtype=torch.int64)), "group_offsets must have dtype")
    raises(call(d=z(M_cap - 1, N, dtype=torch.bfloat16)), "d must have shape")
    raises(call(d=z(N, M_cap, dtype=torch.bfloat16).t()), "d must be contiguous")
    raises(call(d=z(M_cap, N, dtype=torch.int32)), "output dtype")
    raises(call(), "on the GPU")


def test_masked_and_kgrouped_checks():
    G, M_max, N, K = 3, 256, 256, 256
    a, sa = z(G, M_max, K), z(G, M_max, K // 128)
    b, sb = z(G, N, K), z(G, N // 128, K // 128)
    mm = z(G, dtype=torch.int32)
    raises(lambda: fgb.fp8_grouped_gemm_masked(a, sa, b, z(G, N, K // 128), mm), "sb must have shape")
    raises(lambda: fgb.fp8_grouped_gemm_masked(a, sa, b, sb, z(G + 1, dtype=torch.int32)), "masked_m must have shape")
    raises(lambda: fgb.fp8_grouped_gemm_masked(a, sa, z(G, N, K + 128), sb, mm), "b must have shape")
    Kc = 1024
    ka, kb = z(256, Kc), z(384, Kc)
    koff = z(G + 1, dtype=torch.int32)
    raises(lambda: fgb.fp8_kgrouped_gemm(ka, z(256, Kc // 128 - 1), kb, z(384, Kc // 128), koff), "sa must have shape")
    raises(lambda: fgb.fp8_kgrouped_gemm(ka, z(256, Kc // 128), kb, z(384, Kc // 128), koff,
                                         d=z(G, 256, 383, dtype=torch.float32)), "d must have shape")
    raises(lambda: fgb.fp8_kgrouped_gemm(ka, z(256, Kc // 128), z(384, Kc - 128), z(384, Kc // 128), koff),
           "same K capacity")


def test_data_movement_checks():
    T, C = 256, 512
    q = z(T, C)
    raises(lambda: fgb.fp8_direct_transpose(q, z(T, C // 128 + 1)), "s must have shape")
    raises(lambda: fgb.fp8_direct_transpose(q, z(T, C // 128), fgb.BLOCK128), "s must have shape")
    raises(lambda: fgb.fp8_dequant(q, z(T // 128, C // 128), fgb.ROW1x128), "s must have shape")
    raises(lambda: fgb.fp8_quant_rowwise(z(T, C, dtype=torch.float32), s=z(T, C // 32)), "s must have shape")
    raises(lambda: fgb.fp8_quant_rowwise(z(T, 100, dtype=torch.float32)), "multiple of the group")
    raises(lambda: fgb.fp8_quant_blockwise(z(T, C, dtype=torch.float32), s=z(T, C // 128)), "s must have shape")
    idx = z(T, 8, dtype=torch.int32)
    raises(lambda: fgb.permute_pad(q, z(T, C // 128 - 1), idx, 32), "xs must have shape")
    raises(lambda: fgb.permute_pad(q, z(T, C // 128), idx.long(), 32), "topk_idx must have dtype")
    raises(lambda: fgb.unpermute_unpad(z(T, C, dtype=torch.bfloat16), idx, probs=z(T, 4, dtype=torch.float32)),
           "probs must have shape")
    raises(lambda: fgb.dswiglu_quant(z(T, 2 * C), z(T, 2 * C // 128), z(T, 2 * C, dtype=torch.bfloat16)),
           "da must have shape")
    raises(lambda: fgb.mx2_dequant(q, z(T, C // 32), z(T, 2, dtype=torch.float32), g1=10240), "s1 must have shape")
    raises(lambda: fgb.swiglu_quant(z(T, 2 * C, dtype=torch.float32)), "h must have dtype")
