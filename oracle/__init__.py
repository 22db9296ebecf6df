"""CPU oracle for the fine-grained blockwise FP8 path (TEST INFRASTRUCTURE).

Only the tests, ``__graft_entry__.smoke()`` and the bench's ``cpu_baseline``
leg may import this package.  It wraps ``fgb_oracle.c`` (plain C, fp64 unless
an operation is defined in fp32) through ctypes with numpy arrays, and shares
no code with the HIP library.  Each wrapper's docstring names the C function;
the C source cites the page section each one follows.
"""
import ctypes as C
import os

import numpy as np

from . import build as _build

_lib = None


def lib():
    global _lib
    if _lib is None:
        path = _build.LIB
        if not os.path.exists(path) or os.path.getmtime(path) < os.path.getmtime(_build.SRC):
            _build.build()
        L = C.CDLL(path)
        p = C.c_void_p
        i64 = C.c_int64
        i32 = C.c_int
        L.orc_e4m3_decode.restype = C.c_double
        L.orc_e4m3_decode.argtypes = [C.c_uint8]
        L.orc_e4m3_encode.restype = C.c_uint8
        L.orc_e4m3_encode.argtypes = [C.c_double]
        L.orc_scale_exp.restype = C.c_int
        L.orc_scale_exp.argtypes = [C.c_double, C.c_int]
        L.orc_e4m3_encode_f32.argtypes = [p, i64, p]
        L.orc_e4m3_decode_all.argtypes = [p]
        L.orc_scale_exp_f32.argtypes = [p, i64, i32, p]
        L.orc_quant_rowwise.argtypes = [p, i32, i64, i64, i64, i32, i32, p, i64, p, i64]
        L.orc_quant_blockwise.argtypes = [p, i32, i64, i64, i64, p, i64, p, i64]
        L.orc_dequant.argtypes = [p, p, i32, i64, i64, p]
        L.orc_direct_transpose.argtypes = [p, p, i64, i64, p, p]
        L.orc_block_transpose.argtypes = [p, p, i64, i64, p, p]
        L.orc_naive_transpose.argtypes = [p, p, i64, i64, p, p]
        L.orc_grouped_direct_transpose.argtypes = [p, p, i64, p, i32, p, p, i64, p]
        L.orc_kgrouped_gemm_sampled.argtypes = [p, p, p, p, p, i64, p, p, p, i64, p]
        L.orc_e5m2_decode.restype = C.c_double
        L.orc_e5m2_decode.argtypes = [C.c_uint8]
        L.orc_e5m2_encode.restype = C.c_uint8
        L.orc_e5m2_encode.argtypes = [C.c_double]
        L.orc_fp8_encode_f32.argtypes = [p, i64, i32, p]
        L.orc_fp8_decode_all.argtypes = [i32, p]
        L.orc_scale_exp_fmt.restype = C.c_int
        L.orc_scale_exp_fmt.argtypes = [C.c_double, i32, i32, i32]
        L.orc_scale_exp_fmt_f32.argtypes = [p, i64, i32, i32, i32, p]
        L.orc_quant_rowwise_fmt.argtypes = [p, i32, i64, i64, i64, i32, i32, i32, i32, p, i64, p, i64]
        L.orc_dequant_fmt.argtypes = [p, p, i32, i32, i64, i64, p]
        L.orc_direct_transpose_fmt.argtypes = [p, p, i64, i64, i32, p, p]
        L.orc_block_gemm_fmt_sampled.argtypes = [p, p, i32, i32, p, p, i32, i32, i64, i64, p, p, i64, p]
        L.orc_gemm_run_bounds_fmt_sampled.argtypes = [p, p, i32, i32, p, p, i32, i32, i64, i64, p, p, i64,
                                                      i32, p, p]
        L.orc_quant_rowwise_sf.argtypes = [p, i64, i64, p, p]
        L.orc_dequant_sf.argtypes = [p, p, i64, i64, p]
        L.orc_naive_transpose_sf.argtypes = [p, p, i64, i64, p, p]
        L.orc_block_gemm.argtypes = [p, p, i32, p, p, i32, p, i64, i64, i64, i64, i64, i64, p]
        L.orc_block_gemm_sampled.argtypes = [p, p, i32, p, p, i32, p, i64, i64, i64, i64, i64,
                                             p, p, i64, p]
        L.orc_gemm_run_bounds_sampled.argtypes = [p, p, i32, p, p, i32, p, i64, i64, i64, i64, p, p,
                                                  i64, i32, p, p]
        L.orc_grouped_gemm_sampled.argtypes = [p, p, p, p, p, i32, i64, i64, p, p, i64, p]
        L.orc_permute_pad.restype = C.c_int64
        L.orc_permute_pad.argtypes = [p, p, p, i64, i32, i32, i64, i32, p, p, p, p, i64]
        L.orc_unpermute_unpad.argtypes = [p, p, p, i64, i32, i64, p]
        L.orc_unpermute_backward.argtypes = [p, p, p, i64, i32, i64, i64, p]
        L.orc_expf.restype = C.c_float
        L.orc_expf.argtypes = [C.c_float]
        L.orc_expf_bulk.argtypes = [p, i64, p]
        L.orc_swiglu_quant.argtypes = [p, i64, i64, i64, p, i32, p, p]
        L.orc_dswiglu_quant.argtypes = [p, p, p, i64, i64, p, i32, p, p]
        L.orc_swiglu_f32.argtypes = [p, p, i64, p]
        L.orc_dswiglu_f32.argtypes = [p, p, p, i64, p, p]
        L.orc_mx2_quant.argtypes = [p, i64, i64, i64, p, p, p]
        L.orc_mx2_quant_rule.argtypes = [p, i64, i64, i64, i32, p, p, p]
        L.orc_mx2_dequant.argtypes = [p, p, p, i64, i64, i64, p]
        L.orc_snr_db.restype = C.c_double
        L.orc_snr_db.argtypes = [p, p, i64]
        L.orc_bf16_to_f32.argtypes = [p, i64, p]
        _lib = L
    return _lib


F32, BF16 = 0, 1
ROW1x128, ROW1x32, BLOCK128 = 0, 1, 2
E4M3, E5M2 = 0, 1
SCALE_CEIL, SCALE_OCP_FLOOR = 0, 1


def emin_for(group, fmt=0):
    """Scale floor: the 1e-4 amax clamp for 128-element groups (-22 for E4M3,
    -29 for E5M2), the E8M0 range (-127) for 32-element groups."""
    if group == 32:
        return -127
    return -29 if fmt == E5M2 else -22


def _p(a):
    return None if a is None else a.ctypes.data_as(C.c_void_p)


def _c(a, dtype):
    a = np.ascontiguousarray(a)
    assert a.dtype == dtype, (a.dtype, dtype)
    return a


def _xdtype(x):
    if x.dtype == np.float32:
        return F32
    if x.dtype == np.uint16:  # bf16 bit patterns
        return BF16
    raise TypeError("oracle inputs are float32 or bf16 bit patterns (uint16)")


# ---- formats -------------------------------------------------------------
def e4m3_decode_table():
    """orc_e4m3_decode over all 256 codes (fp64; NaN for 0x7F/0xFF)."""
    out = np.empty(256, np.float64)
    lib().orc_e4m3_decode_all(_p(out))
    return out


def e4m3_encode(x):
    """orc_e4m3_encode applied to float32 values."""
    x = _c(x, np.float32)
    q = np.empty(x.shape, np.uint8)
    lib().orc_e4m3_encode_f32(_p(x), x.size, _p(q))
    return q


def scale_exp(amax, emin=-22):
    """orc_scale_exp applied to float32 amax values."""
    a = _c(amax, np.float32)
    e = np.empty(a.shape, np.int32)
    lib().orc_scale_exp_f32(_p(a), a.size, emin, _p(e))
    return e


def fp8_encode(x, fmt):
    """orc_fp8_encode applied to float32 values (E4M3 or E5M2)."""
    x = _c(x, np.float32)
    q = np.empty(x.shape, np.uint8)
    lib().orc_fp8_encode_f32(_p(x), x.size, fmt, _p(q))
    return q


def fp8_decode_all(fmt):
    """orc_fp8_decode_all: the values of all 256 codes of a format."""
    out = np.empty(256, np.float64)
    lib().orc_fp8_decode_all(fmt, _p(out))
    return out


def scale_exp_fmt(amax, fmt, rule, emin):
    """orc_scale_exp_fmt applied to float32 amax values."""
    a = _c(amax, np.float32)
    e = np.empty(a.shape, np.int32)
    lib().orc_scale_exp_fmt_f32(_p(a), a.size, fmt, rule, emin, _p(e))
    return e


def quant_rowwise_fmt(x, group=128, fmt=0, rule=0):
    """orc_quant_rowwise_fmt: x [rows, cols] fp32 or bf16 bits -> (q, s)."""
    x = np.ascontiguousarray(x)
    rows, cols = x.shape
    q = np.empty((rows, cols), np.uint8)
    s = np.empty((rows, cols // group), np.uint8)
    lib().orc_quant_rowwise_fmt(_p(x), _xdtype(x), rows, cols, cols, group, fmt, rule, emin_for(group, fmt), _p(q),
                                cols, _p(s), cols // group)
    return q, s


def dequant_fmt(q, s, group, fmt):
    """orc_dequant_fmt -> fp64 [rows, cols] (row-wise 1 x group scales)."""
    q = _c(q, np.uint8)
    s = _c(s, np.uint8)
    out = np.empty(q.shape, np.float64)
    lib().orc_dequant_fmt(_p(q), _p(s), group, fmt, q.shape[0], q.shape[1], _p(out))
    return out


def direct_transpose_fmt(q, s, fmt):
    """orc_direct_transpose_fmt: as direct_transpose for codes of format fmt."""
    q = _c(q, np.uint8)
    s = _c(s, np.uint8)
    T, Cc = q.shape
    qt = np.empty((Cc, T), np.uint8)
    st = np.empty((Cc, T // 128), np.uint8)
    lib().orc_direct_transpose_fmt(_p(q), _p(s), T, Cc, fmt, _p(qt), _p(st))
    return qt, st


def block_gemm_fmt_sampled(a, sa, a_gran, a_fmt, b, sb, b_gran, b_fmt, mi, ni):
    """orc_block_gemm_fmt_sampled: D = A B^T at (mi, ni), operand formats chosen."""
    a, b, sa, sb = (_c(v, np.uint8) for v in (a, b, sa, sb))
    mi = _c(np.asarray(mi, np.int64), np.int64)
    ni = _c(np.asarray(ni, np.int64), np.int64)
    out = np.empty(mi.shape, np.float64)
    lib().orc_block_gemm_fmt_sampled(_p(a), _p(sa), a_gran, a_fmt, _p(b), _p(sb), b_gran, b_fmt, b.shape[0],
                                     a.shape[1], _p(mi), _p(ni), mi.size, _p(out))
    return out


def gemm_run_bounds_fmt_sampled(a, sa, a_gran, a_fmt, b, sb, b_gran, b_fmt, mi, ni, run=8):
    """orc_gemm_run_bounds_fmt_sampled -> (runmax, abssum) at (mi, ni)."""
    a, b, sa, sb = (_c(v, np.uint8) for v in (a, b, sa, sb))
    mi = _c(np.asarray(mi, np.int64), np.int64)
    ni = _c(np.asarray(ni, np.int64), np.int64)
    rm = np.empty(mi.shape, np.float64)
    asum = np.empty(mi.shape, np.float64)
    lib().orc_gemm_run_bounds_fmt_sampled(_p(a), _p(sa), a_gran, a_fmt, _p(b), _p(sb), b_gran, b_fmt, b.shape[0],
                                          a.shape[1], _p(mi), _p(ni), mi.size, run, _p(rm), _p(asum))
    return rm, asum


def expf(x):
    """orc_expf (the SwiGLU exponential) applied elementwise."""
    x = _c(x, np.float32)
    y = np.empty_like(x)
    lib().orc_expf_bulk(_p(x), x.size, _p(y))
    return y


def bf16_to_f32(h):
    h = _c(h, np.uint16)
    out = np.empty(h.shape, np.float32)
    lib().orc_bf16_to_f32(_p(h), h.size, _p(out))
    return out


# ---- quantization --------------------------------------------------------
def quant_rowwise(x, group=128):
    """orc_quant_rowwise: x [rows, cols] fp32 or bf16 bits -> (q, s)."""
    x = np.ascontiguousarray(x)
    rows, cols = x.shape
    emin = -22 if group == 128 else -127
    q = np.empty((rows, cols), np.uint8)
    s = np.empty((rows, cols // group), np.uint8)
    lib().orc_quant_rowwise(_p(x), _xdtype(x), rows, cols, cols, group, emin, _p(q), cols,
                            _p(s), cols // group)
    return q, s


def quant_blockwise(w):
    """orc_quant_blockwise: w [rows, cols] -> (q, s[ceil(rows/128), cols/128])."""
    w = np.ascontiguousarray(w)
    rows, cols = w.shape
    q = np.empty((rows, cols), np.uint8)
    s = np.empty(((rows + 127) // 128, cols // 128), np.uint8)
    lib().orc_quant_blockwise(_p(w), _xdtype(w), rows, cols, cols, _p(q), cols, _p(s),
                              cols // 128)
    return q, s


def dequant(q, s, gran):
    """orc_dequant -> fp64 [rows, cols]."""
    q = _c(q, np.uint8)
    s = _c(s, np.uint8)
    out = np.empty(q.shape, np.float64)
    lib().orc_dequant(_p(q), _p(s), gran, q.shape[0], q.shape[1], _p(out))
    return out


def direct_transpose(q, s):
    """orc_direct_transpose: row-wise (q[T,C], s[T,C/128]) -> (qt[C,T], st[C,T/128])."""
    q = _c(q, np.uint8)
    s = _c(s, np.uint8)
    T, Cc = q.shape
    qt = np.empty((Cc, T), np.uint8)
    st = np.empty((Cc, T // 128), np.uint8)
    lib().orc_direct_transpose(_p(q), _p(s), T, Cc, _p(qt), _p(st))
    return qt, st


def block_transpose(q, s):
    """orc_block_transpose: (W[rows,cols], s[rows/128, cols/128]) -> transposed pair."""
    q = _c(q, np.uint8)
    s = _c(s, np.uint8)
    rows, cols = q.shape
    qt = np.empty((cols, rows), np.uint8)
    st = np.empty((cols // 128, rows // 128), np.uint8)
    lib().orc_block_transpose(_p(q), _p(s), rows, cols, _p(qt), _p(st))
    return qt, st


def naive_transpose(q, s):
    """orc_naive_transpose: dequantize, transpose, requantize 1x128 (power-of-two scales)."""
    q = _c(q, np.uint8)
    s = _c(s, np.uint8)
    T, Cc = q.shape
    qt = np.empty((Cc, T), np.uint8)
    st = np.empty((Cc, T // 128), np.uint8)
    lib().orc_naive_transpose(_p(q), _p(s), T, Cc, _p(qt), _p(st))
    return qt, st


def quant_rowwise_sf(x):
    """orc_quant_rowwise_sf: 1x128 with fp32 scales sf = amax/448 (study only) -> (q, sf)."""
    x = _c(x, np.float32)
    rows, cols = x.shape
    q = np.empty((rows, cols), np.uint8)
    sf = np.empty((rows, cols // 128), np.float32)
    lib().orc_quant_rowwise_sf(_p(x), rows, cols, _p(q), _p(sf))
    return q, sf


def dequant_sf(q, sf):
    q = _c(q, np.uint8)
    sf = _c(sf, np.float32)
    rows, cols = q.shape
    out = np.empty((rows, cols), np.float32)
    lib().orc_dequant_sf(_p(q), _p(sf), rows, cols, _p(out))
    return out


def naive_transpose_sf(q, sf):
    """orc_naive_transpose_sf: the three passes with sf = amax/448 scaling (study only)."""
    q = _c(q, np.uint8)
    sf = _c(sf, np.float32)
    T, Cc = q.shape
    qt = np.empty((Cc, T), np.uint8)
    sft = np.empty((Cc, T // 128), np.float32)
    lib().orc_naive_transpose_sf(_p(q), _p(sf), T, Cc, _p(qt), _p(sft))
    return qt, sft


def block_transpose_batched(q, s):
    """Per-expert weight-block transposes: q [G, rows, cols], s [G, rows/128, cols/128]."""
    outs = [block_transpose(q[e], s[e]) for e in range(q.shape[0])]
    return np.stack([o[0] for o in outs]), np.stack([o[1] for o in outs])


def grouped_direct_transpose(q, s, off, Kc):
    """orc_grouped_direct_transpose: segments of q [M, C] -> (qt [C, Kc], st [C, Kc/128], koff [G+1])."""
    q = _c(q, np.uint8)
    s = _c(s, np.uint8)
    off = _c(off, np.int32)
    M, Cc = q.shape
    G = len(off) - 1
    qt = np.zeros((Cc, Kc), np.uint8)
    st = np.zeros((Cc, Kc // 128), np.uint8)
    koff = np.zeros(G + 1, np.int32)
    lib().orc_grouped_direct_transpose(_p(q), _p(s), Cc, _p(off), G, _p(qt), _p(st), Kc, _p(koff))
    return qt, st, koff


def kgrouped_gemm_sampled(a, sa, b, sb, koff, ei, mi, ni):
    a = _c(a, np.uint8)
    sa = _c(sa, np.uint8)
    b = _c(b, np.uint8)
    sb = _c(sb, np.uint8)
    koff = _c(koff, np.int32)
    ei, mi, ni = (_c(v, np.int64) for v in (ei, mi, ni))
    out = np.empty(len(mi), np.float64)
    lib().orc_kgrouped_gemm_sampled(_p(a), _p(sa), _p(b), _p(sb), _p(koff), a.shape[1], _p(ei), _p(mi), _p(ni),
                                   len(mi), _p(out))
    return out


# ---- GEMMs ---------------------------------------------------------------
def block_gemm(a, sa, a_gran, b, sb, b_gran, b_l1=None, g1=0):
    """orc_block_gemm: D[M,N] = A[M,K] * B[N,K]^T with block scales, fp64."""
    a = _c(a, np.uint8)
    b = _c(b, np.uint8)
    sa = _c(sa, np.uint8)
    sb = _c(sb, np.uint8)
    if b_l1 is not None:
        b_l1 = _c(b_l1, np.float32)
    M, K = a.shape
    N = b.shape[0]
    d = np.empty((M, N), np.float64)
    lib().orc_block_gemm(_p(a), _p(sa), a_gran, _p(b), _p(sb), b_gran, _p(b_l1), g1, M, N, K,
                         K, K, _p(d))
    return d


def block_gemm_sampled(a, sa, a_gran, b, sb, b_gran, mi, ni, b_l1=None, g1=0):
    """orc_block_gemm_sampled: the same result at coordinates (mi[i], ni[i])."""
    a = _c(a, np.uint8)
    b = _c(b, np.uint8)
    sa = _c(sa, np.uint8)
    sb = _c(sb, np.uint8)
    if b_l1 is not None:
        b_l1 = _c(b_l1, np.float32)
    mi = _c(np.asarray(mi, np.int64), np.int64)
    ni = _c(np.asarray(ni, np.int64), np.int64)
    K = a.shape[1]
    N = b.shape[0]
    out = np.empty(mi.shape, np.float64)
    lib().orc_block_gemm_sampled(_p(a), _p(sa), a_gran, _p(b), _p(sb), b_gran, _p(b_l1), g1, N,
                                 K, K, K, _p(mi), _p(ni), mi.size, _p(out))
    return out


def gemm_run_bounds_sampled(a, sa, a_gran, b, sb, b_gran, mi, ni, run=8, b_l1=None):
    """orc_gemm_run_bounds_sampled -> (sum of per-run max |p|, sum |p|) at (mi, ni).

    Test tolerance helper for a matrix unit that sums runs of `run`
    consecutive K products with limited precision."""
    a = _c(a, np.uint8)
    b = _c(b, np.uint8)
    sa = _c(sa, np.uint8)
    sb = _c(sb, np.uint8)
    if b_l1 is not None:
        b_l1 = _c(b_l1, np.float32)
    mi = _c(np.asarray(mi, np.int64), np.int64)
    ni = _c(np.asarray(ni, np.int64), np.int64)
    K = a.shape[1]
    N = b.shape[0]
    rm = np.empty(mi.shape, np.float64)
    asum = np.empty(mi.shape, np.float64)
    lib().orc_gemm_run_bounds_sampled(_p(a), _p(sa), a_gran, _p(b), _p(sb), b_gran, _p(b_l1), N,
                                      K, K, K, _p(mi), _p(ni), mi.size, run, _p(rm), _p(asum))
    return rm, asum


def grouped_gemm_sampled(a, sa, b, sb, off, mi, ni):
    """orc_grouped_gemm_sampled: M-grouped contiguous GEMM at (mi, ni); NaN outside segments."""
    a = _c(a, np.uint8)
    sa = _c(sa, np.uint8)
    b = _c(b, np.uint8)
    sb = _c(sb, np.uint8)
    off = _c(np.asarray(off, np.int32), np.int32)
    G, N, K = b.shape
    mi = _c(np.asarray(mi, np.int64), np.int64)
    ni = _c(np.asarray(ni, np.int64), np.int64)
    out = np.empty(mi.shape, np.float64)
    lib().orc_grouped_gemm_sampled(_p(a), _p(sa), _p(b), _p(sb), _p(off), G, N, K, _p(mi),
                                   _p(ni), mi.size, _p(out))
    return out


# ---- MoE data movement ---------------------------------------------------
def permute_pad(xq, xs, topk_idx, G, pad_multiple=16, M_cap=None):
    """orc_permute_pad -> (out_q, out_s, row_map, offsets, rows_used)."""
    xq = _c(xq, np.uint8)
    xs = _c(xs, np.uint8)
    topk_idx = _c(np.asarray(topk_idx, np.int32), np.int32)
    T, H = xq.shape
    topk = topk_idx.shape[1]
    if M_cap is None:
        M_cap = T * topk + (pad_multiple - 1) * G
    out_q = np.full((M_cap, H), 0xCD, np.uint8)
    out_s = np.full((M_cap, H // 128), 0xCD, np.uint8)
    row_map = np.empty((T, topk), np.int32)
    off = np.empty(G + 1, np.int32)
    used = lib().orc_permute_pad(_p(xq), _p(xs), _p(topk_idx), T, topk, G, H, pad_multiple,
                                 _p(out_q), _p(out_s), _p(row_map), _p(off), M_cap)
    if used < 0:
        raise ValueError("M_cap too small")
    return out_q, out_s, row_map, off, int(used)


def unpermute_unpad(y, row_map, probs=None):
    """orc_unpermute_unpad: y bf16 bits [M, H] -> out bf16 bits [T, H]."""
    y = _c(y, np.uint16)
    row_map = _c(np.asarray(row_map, np.int32), np.int32)
    if probs is not None:
        probs = _c(probs, np.float32)
    T, topk = row_map.shape
    H = y.shape[1]
    out = np.empty((T, H), np.uint16)
    lib().orc_unpermute_unpad(_p(y), _p(row_map), _p(probs), T, topk, H, _p(out))
    return out


def unpermute_backward(dout, row_map, probs, M_cap):
    """orc_unpermute_backward: dout bf16 bits [T,H] -> dy bf16 bits [M_cap, H]."""
    dout = _c(dout, np.uint16)
    row_map = _c(row_map, np.int32)
    T, H = dout.shape
    topk = row_map.shape[1]
    dy = np.empty((M_cap, H), np.uint16)
    pp = None
    if probs is not None:
        probs = _c(probs, np.float32)
        pp = _p(probs)
    lib().orc_unpermute_backward(_p(dout), _p(row_map), pp, T, topk, H, M_cap, _p(dy))
    return dy


def swiglu_f32(g, u):
    """orc_swiglu_f32: a = silu(g) * u in fp32, elementwise (no quantization)."""
    g = _c(g, np.float32)
    u = _c(u, np.float32)
    a = np.empty_like(g)
    lib().orc_swiglu_f32(_p(g), _p(u), g.size, _p(a))
    return a


def dswiglu_f32(g, u, da):
    """orc_dswiglu_f32: (du, dg) of the SwiGLU backward in fp32, elementwise (no quantization)."""
    g = _c(g, np.float32)
    u = _c(u, np.float32)
    da = _c(da, np.float32)
    du = np.empty_like(g)
    dg = np.empty_like(g)
    lib().orc_dswiglu_f32(_p(g), _p(u), _p(da), g.size, _p(du), _p(dg))
    return du, dg


def swiglu_quant(h, off=None):
    """orc_swiglu_quant: h bf16 bits [M, 2F] (gate|up) -> (q [M,F], s [M,F/128]).

    Rows at or past off[G] (when off is given) are left as zeros here."""
    h = _c(h, np.uint16)
    M, F2 = h.shape
    F = F2 // 2
    q = np.zeros((M, F), np.uint8)
    s = np.zeros((M, F // 128), np.uint8)
    G = 0
    if off is not None:
        off = _c(np.asarray(off, np.int32), np.int32)
        G = off.size - 1
    lib().orc_swiglu_quant(_p(h), M, F, F2, _p(off), G, _p(q), _p(s))
    return q, s


# ---- MOSS two-level ------------------------------------------------------
def dswiglu_quant(hq, hs, da, off=None):
    """orc_dswiglu_quant: FP8-cached SwiGLU input (hq [M,2F], hs [M,2F/128]) and bf16 bits
    da [M,F] -> 1x128 codes and scales of [dg | du] (dq [M,2F], ds [M,2F/128])."""
    hq = _c(hq, np.uint8)
    hs = _c(hs, np.uint8)
    da = _c(da, np.uint16)
    M, F2 = hq.shape
    F = F2 // 2
    dq = np.zeros((M, F2), np.uint8)
    ds = np.zeros((M, F2 // 128), np.uint8)
    offp = None
    G = 0
    if off is not None:
        off = _c(off, np.int32)
        offp = _p(off)
        G = len(off) - 1
    lib().orc_dswiglu_quant(_p(hq), _p(hs), _p(da), M, F, offp, G, _p(dq), _p(ds))
    return dq, ds


def mx2_quant(x, g1=10240, rule=0):
    """orc_mx2_quant_rule: x bf16 bits [R, C] -> (q, s2 [R, C/32], s1 [R, ceil(C/g1)]).
    rule: SCALE_CEIL (orc_mx2_quant) or SCALE_OCP_FLOOR for the level-2 exponent."""
    x = _c(x, np.uint16)
    R, Cc = x.shape
    ng = (Cc + g1 - 1) // g1
    q = np.empty((R, Cc), np.uint8)
    s2 = np.empty((R, Cc // 32), np.uint8)
    s1 = np.empty((R, ng), np.float32)
    if rule == SCALE_CEIL:
        lib().orc_mx2_quant(_p(x), R, Cc, g1, _p(q), _p(s2), _p(s1))
    else:
        lib().orc_mx2_quant_rule(_p(x), R, Cc, g1, rule, _p(q), _p(s2), _p(s1))
    return q, s2, s1


def mx2_dequant(q, s2, s1, g1=10240):
    """orc_mx2_dequant -> float32 [R, C]."""
    q = _c(q, np.uint8)
    s2 = _c(s2, np.uint8)
    s1 = _c(s1, np.float32)
    R, Cc = q.shape
    out = np.empty((R, Cc), np.float32)
    lib().orc_mx2_dequant(_p(q), _p(s2), _p(s1), R, Cc, g1, _p(out))
    return out


def snr_db(x, xhat):
    """orc_snr_db: 10 log10(sum x^2 / sum (x - xhat)^2) in fp64."""
    x = _c(x, np.float32)
    xhat = _c(xhat, np.float32)
    return lib().orc_snr_db(_p(x), _p(xhat), x.size)
