"""fine_grained_blockwise_amd -- fine-grained blockwise FP8 for AMD MI355X (gfx950).

A thin Python binding over libfgb.so (include/fgb.h).  Every function here
only marshals arguments: it checks shapes, allocates outputs with
``torch.empty`` on the input's device and calls the C entry point of the same
name on torch's current HIP stream.  All arithmetic runs in the HIP kernels.

There is no fallback: if libfgb.so is missing, importing this package raises.
"""
import ctypes as C
import os

import torch

__all__ = [
    "lib", "symbols", "FgbError",
    "fp8_quant_rowwise", "fp8_quant_blockwise", "fp8_dequant", "fgb_e4m3_encode",
    "fp8_direct_transpose", "fp8_naive_transpose", "fp8_naive_transpose_workspace_size",
    "fp8_block_gemm", "fp8_grouped_gemm", "permute_pad",
    "permute_pad_workspace_size", "unpermute_unpad", "swiglu_quant", "dswiglu_quant", "mx2_quant",
    "mx2_dequant", "unpermute_backward", "unpermute_backward_workspace_size",
    "fp8_block_transpose_batched", "fp8_grouped_direct_transpose", "fp8_kgrouped_gemm", "swiglu_quant_cache",
    "unpermute_backward_quant", "fp8_quant_rowwise_fmt", "fp8_dequant_fmt", "fgb_fp8_encode",
    "fp8_direct_transpose_fmt", "mx2_quant_rule", "fp8_block_gemm_fmt", "fp8_grouped_gemm_masked",
    "permute_pad_noalloc", "PERMUTE_PAD_NOALLOC_SCRATCH_BYTES", "fgb_hbm_probe",
    "PROBE_COPY", "PROBE_READ", "PROBE_FILL", "PROBE_STRIDED_READ", "PROBE_STRIDED_WRITE",
    "E4M3", "E5M2", "SCALE_CEIL", "SCALE_OCP_FLOOR", "F32", "BF16", "ROW1x128", "ROW1x32", "BLOCK128", "GEMM_EXACT", "GEMM_FAST",
]

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libfgb.so")

F32, BF16 = 0, 1
ROW1x128, ROW1x32, BLOCK128 = 0, 1, 2
GEMM_EXACT, GEMM_FAST = 0, 1
E4M3, E5M2 = 0, 1
SCALE_CEIL, SCALE_OCP_FLOOR = 0, 1
PROBE_COPY, PROBE_READ, PROBE_FILL, PROBE_STRIDED_READ, PROBE_STRIDED_WRITE = 0, 1, 2, 3, 4

SYMBOLS = [
    "fgb_last_error", "fgb_version", "fp8_quant_rowwise", "fp8_quant_blockwise", "fp8_dequant",
    "fgb_e4m3_encode", "fp8_direct_transpose", "fp8_block_gemm", "fp8_grouped_gemm",
    "permute_pad", "permute_pad_workspace_size", "unpermute_unpad", "swiglu_quant", "mx2_quant",
    "mx2_dequant", "fp8_naive_transpose", "fp8_naive_transpose_workspace_size", "dswiglu_quant",
    "unpermute_backward", "unpermute_backward_workspace_size", "fp8_block_transpose_batched",
    "fp8_grouped_direct_transpose", "fp8_kgrouped_gemm", "swiglu_quant_cache", "unpermute_backward_quant",
    "fp8_quant_rowwise_fmt", "fp8_dequant_fmt", "fgb_fp8_encode", "fp8_direct_transpose_fmt", "mx2_quant_rule",
    "fp8_block_gemm_fmt", "fp8_grouped_gemm_masked", "fp8_quant_blockwise_t", "swiglu_f32", "dswiglu_f32",
    "permute_pad_noalloc", "fgb_hbm_probe",
]


class FgbError(RuntimeError):
    def __init__(self, fn, code, msg):
        super().__init__(f"{fn} failed with status {code}: {msg}")
        self.code = code


if not os.path.exists(LIB_PATH):
    raise ImportError(f"libfgb.so not found at {LIB_PATH}; build it with "
                      "`python -c 'import __graft_entry__ as g; g.build()'`")

_lib = C.CDLL(LIB_PATH)
_p, _i64, _i32, _sz = C.c_void_p, C.c_int64, C.c_int, C.c_size_t
_SIG = {
    "fgb_last_error": (C.c_char_p, []),
    "fgb_version": (C.c_char_p, []),
    "fp8_quant_rowwise": (_i32, [_p, _i32, _i64, _i64, _i64, _i32, _p, _i64, _p, _i64, _p]),
    "fp8_quant_blockwise": (_i32, [_p, _i32, _i64, _i64, _i64, _p, _i64, _p, _i64, _p]),
    "fp8_dequant": (_i32, [_p, _p, _i32, _i64, _i64, _p, _i32, _p]),
    "fgb_e4m3_encode": (_i32, [_p, _i64, _p, _p]),
    "fgb_hbm_probe": (_i32, [_p, _p, _i64, _i64, _i32, _p]),
    "fp8_direct_transpose": (_i32, [_p, _p, _i32, _i64, _i64, _p, _p, _p]),
    "fp8_naive_transpose": (_i32, [_p, _p, _i64, _i64, _p, _p, _p, _sz, _p]),
    "fp8_block_transpose_batched": (_i32, [_p, _p, _i32, _i64, _i64, _p, _p, _p]),
    "fp8_grouped_direct_transpose": (_i32, [_p, _p, _i64, _i64, _p, _i32, _p, _p, _i64, _p, _p]),
    "fp8_naive_transpose_workspace_size": (_sz, [_i64, _i64]),
    "fp8_block_gemm": (_i32, [_p, _p, _i32, _p, _p, _i32, _p, _i64, _i64, _i64, _i64, _i64, _i64,
                              _p, _i32, _i64, _i32, _i32, _p, _sz, _p]),
    "fp8_grouped_gemm": (_i32, [_p, _p, _p, _p, _p, _i32, _i64, _i64, _i64, _p, _i32, _i32, _p]),
    "fp8_kgrouped_gemm": (_i32, [_p, _p, _p, _p, _p, _i32, _i64, _i64, _i64, _p, _i32, _i32, _i32,
                                 _p]),
    "permute_pad": (_i32, [_p, _p, _p, _i64, _i32, _i32, _i64, _i32, _p, _p, _p, _p, _i64, _p,
                           _sz, _p]),
    "permute_pad_workspace_size": (_sz, [_i64, _i32, _i32]),
    "permute_pad_noalloc": (_i32, [_p, _p, _p, _i64, _i32, _i32, _i64, _i32, _p, _p, _p, _p, _i64, _p]),
    "unpermute_unpad": (_i32, [_p, _p, _p, _i64, _i32, _i64, _p, _p]),
    "unpermute_backward": (_i32, [_p, _p, _p, _i64, _i32, _i64, _i64, _p, _p, _sz, _p]),
    "unpermute_backward_workspace_size": (_sz, [_i64]),
    "swiglu_quant": (_i32, [_p, _i64, _i64, _i64, _p, _i32, _p, _p, _p]),
    "swiglu_quant_cache": (_i32, [_p, _i64, _i64, _i64, _p, _i32, _p, _p, _p, _p, _p]),
    "unpermute_backward_quant": (_i32, [_p, _p, _p, _i64, _i32, _i64, _i64, _p, _p, _p, _sz, _p]),
    "dswiglu_quant": (_i32, [_p, _p, _p, _i64, _i64, _p, _i32, _p, _p, _p]),
    "mx2_quant": (_i32, [_p, _i64, _i64, _i64, _p, _p, _p, _p]),
    "mx2_quant_rule": (_i32, [_p, _i64, _i64, _i64, _i32, _p, _p, _p, _p]),
    "fp8_quant_rowwise_fmt": (_i32, [_p, _i32, _i64, _i64, _i64, _i32, _i32, _i32, _p, _i64, _p, _i64, _p]),
    "fp8_dequant_fmt": (_i32, [_p, _p, _i32, _i32, _i64, _i64, _p, _i32, _p]),
    "fgb_fp8_encode": (_i32, [_p, _i64, _i32, _p, _p]),
    "fp8_direct_transpose_fmt": (_i32, [_p, _p, _i32, _i64, _i64, _p, _p, _p]),
    "fp8_block_gemm_fmt": (_i32, [_p, _p, _i32, _i32, _p, _p, _i32, _i32, _p, _i64, _i64, _i64, _i64, _i64, _i64,
                                  _p, _i32, _i64, _i32, _i32, _p]),
    "fp8_grouped_gemm_masked": (_i32, [_p, _p, _p, _p, _p, _i32, _i64, _i64, _i64, _p, _i32, _i32, _p]),
    "fp8_quant_blockwise_t": (_i32, [_p, _i32, _i32, _i64, _i64, _p, _p, _p, _p, _p]),
    "mx2_dequant": (_i32, [_p, _p, _p, _i64, _i64, _i64, _p, _p]),
    "swiglu_f32": (_i32, [_p, _p, _i64, _p, _p]),
    "dswiglu_f32": (_i32, [_p, _p, _p, _i64, _p, _p, _p]),
}
for _name, (_res, _args) in _SIG.items():
    _f = getattr(_lib, _name)
    _f.restype = _res
    _f.argtypes = _args


def lib():
    """The loaded ctypes library (C ABI of include/fgb.h)."""
    return _lib


def symbols():
    return list(SYMBOLS)


def _call(name, *args):
    rc = getattr(_lib, name)(*args)
    if rc != 0:
        raise FgbError(name, rc, _lib.fgb_last_error().decode())


def _ptr(t):
    # A temporary passed here (e.g. x.contiguous()) may be freed as soon as the
    # call returns: every kernel is enqueued on torch's current stream, the
    # stream the temporary was allocated on, and torch's caching allocator only
    # hands a freed block to later work on that same stream, so the kernel
    # always reads it before anything can overwrite it.
    return None if t is None else C.c_void_p(t.data_ptr())


def _stream(t):
    return C.c_void_p(torch.cuda.current_stream(t.device).cuda_stream)


def _dtype_code(t):
    if t.dtype == torch.float32:
        return F32
    if t.dtype == torch.bfloat16:
        return BF16
    raise TypeError(f"expected float32 or bfloat16, got {t.dtype}")


def _check_dev(*ts):
    dev = None
    for t in ts:
        if t is None:
            continue
        if not t.is_cuda:
            raise ValueError("all tensors must be on the GPU")
        if dev is None:
            dev = t.device
        elif t.device != dev:
            raise ValueError("all tensors must be on the same GPU")
    return dev


def _row_ld(t):
    if t.dim() != 2 or t.stride(1) != 1:
        raise ValueError("expected a 2-D tensor with unit column stride")
    return t.stride(0)


def _need(t, name, shape=None, dtype=None, contiguous=False):
    """Raise ValueError unless t has the given shape, dtype and layout."""
    if t is None:
        raise ValueError(f"{name} is required")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name} must have dtype {dtype}, got {t.dtype}")
    if shape is not None and tuple(t.shape) != tuple(int(v) for v in shape):
        raise ValueError(f"{name} must have shape {tuple(int(v) for v in shape)}, got {tuple(t.shape)}")
    if contiguous and not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t


def _scale_shape(rows, K, gran):
    """Shape of the scale tensor of a [rows, K] code tensor with granularity gran."""
    if gran == ROW1x128:
        return (rows, K // 128)
    if gran == ROW1x32:
        return (rows, K // 32)
    if gran == BLOCK128:
        return ((rows + 127) // 128, K // 128)
    raise ValueError(f"unknown scale granularity {gran}")


def _out_dtype(dtype, name):
    if dtype not in (torch.float32, torch.bfloat16):
        raise ValueError(f"{name}: the output dtype must be float32 or bfloat16, got {dtype}")
    return dtype


def _check_2d_codes(t, name):
    if t.dim() != 2:
        raise ValueError(f"{name} must be 2-D")
    return _need(t, name, dtype=torch.uint8)


def _gemm_out(d, M, N, out_dtype, name, contiguous=False):
    """The output tensor of a GEMM: validated when given (shape [M, N], float32 or bfloat16, unit column
    stride or contiguous), else None (the caller allocates)."""
    if d is None:
        _out_dtype(out_dtype, name)
        return None
    _out_dtype(d.dtype, name)
    _need(d, f"{name}: d", shape=(M, N), contiguous=contiguous)
    if d.dim() == 2 and d.stride(1) != 1:
        raise ValueError(f"{name}: d must have unit column stride")
    return d


def _quant_io_check(name, x, group, q, s, block=False):
    """Shape checks of a quantizer's input and optional outputs; returns (rows, cols)."""
    if x.dim() != 2:
        raise ValueError(f"{name}: the input must be 2-D")
    _dtype_code(x)
    rows, cols = x.shape
    if group not in (32, 128) or cols % group:
        raise ValueError(f"{name}: cols ({cols}) must be a multiple of the group (32 or 128, got {group})")
    if q is not None:
        _need(q, f"{name}: q", shape=(rows, cols), dtype=torch.uint8)
    if s is not None:
        shp = ((rows + 127) // 128, cols // 128) if block else (rows, cols // group)
        _need(s, f"{name}: s", shape=shp, dtype=torch.uint8)
    return rows, cols


# ---------------------------------------------------------------------------
def fp8_quant_rowwise(x, group=128, q=None, s=None):
    """1 x group quantization of x [rows, cols] (fp32/bf16) -> (q uint8, s uint8 [rows, cols/group])."""
    rows, cols = _quant_io_check("fp8_quant_rowwise", x, group, q, s)
    _check_dev(x, q, s)
    if q is None:
        q = torch.empty((rows, cols), dtype=torch.uint8, device=x.device)
    if s is None:
        s = torch.empty((rows, cols // group), dtype=torch.uint8, device=x.device)
    _call("fp8_quant_rowwise", _ptr(x), _dtype_code(x), rows, cols, _row_ld(x), group, _ptr(q),
          _row_ld(q), _ptr(s), _row_ld(s), _stream(x))
    return q, s


def fp8_quant_rowwise_fmt(x, group=128, fmt=E4M3, rule=SCALE_CEIL, q=None, s=None):
    """fp8_quant_rowwise in element format fmt (E4M3/E5M2) with scale rule (SCALE_CEIL/SCALE_OCP_FLOOR)."""
    rows, cols = _quant_io_check("fp8_quant_rowwise_fmt", x, group, q, s)
    _check_dev(x, q, s)
    if q is None:
        q = torch.empty((rows, cols), dtype=torch.uint8, device=x.device)
    if s is None:
        s = torch.empty((rows, cols // group), dtype=torch.uint8, device=x.device)
    _call("fp8_quant_rowwise_fmt", _ptr(x), _dtype_code(x), rows, cols, _row_ld(x), group, fmt, rule, _ptr(q),
          _row_ld(q), _ptr(s), _row_ld(s), _stream(x))
    return q, s


def fp8_quant_blockwise(w, q=None, s=None):
    """128 x 128 quantization of w [rows, cols] -> (q, s [ceil(rows/128), cols/128])."""
    rows, cols = _quant_io_check("fp8_quant_blockwise", w, 128, q, s, block=True)
    _check_dev(w, q, s)
    if q is None:
        q = torch.empty((rows, cols), dtype=torch.uint8, device=w.device)
    if s is None:
        s = torch.empty(((rows + 127) // 128, cols // 128), dtype=torch.uint8, device=w.device)
    _call("fp8_quant_blockwise", _ptr(w), _dtype_code(w), rows, cols, _row_ld(w), _ptr(q),
          _row_ld(q), _ptr(s), _row_ld(s), _stream(w))
    return q, s


def fp8_quant_blockwise_t(w):
    """128x128 quantization of bf16 w [G, rows, cols] (or [rows, cols]) with the transposed copy:
    -> (q, s [G, rows/128, cols/128], qt [G, cols, rows], st [G, cols/128, rows/128])."""
    if w.dim() not in (2, 3):
        raise ValueError("fp8_quant_blockwise_t: w must be [rows, cols] or [G, rows, cols]")
    _need(w, "fp8_quant_blockwise_t: w", dtype=torch.bfloat16, contiguous=True)
    _check_dev(w)
    w3 = w if w.dim() == 3 else w.unsqueeze(0)
    G, rows, cols = w3.shape
    dev = w.device
    q = torch.empty((G, rows, cols), dtype=torch.uint8, device=dev)
    s = torch.empty((G, rows // 128, cols // 128), dtype=torch.uint8, device=dev)
    qt = torch.empty((G, cols, rows), dtype=torch.uint8, device=dev)
    st = torch.empty((G, cols // 128, rows // 128), dtype=torch.uint8, device=dev)
    _call("fp8_quant_blockwise_t", _ptr(w3), _dtype_code(w3), G, rows, cols, _ptr(q), _ptr(s), _ptr(qt), _ptr(st),
          _stream(w))
    if w.dim() == 2:
        return q[0], s[0], qt[0], st[0]
    return q, s, qt, st


def fp8_dequant(q, s, gran, out_dtype=torch.float32):
    """decode(q) * 2^(s-127) -> out [rows, cols] (fp32 or bf16); q, s dense."""
    _check_2d_codes(q, "fp8_dequant: q")
    rows, cols = q.shape
    _need(s, "fp8_dequant: s", shape=_scale_shape(rows, cols, gran), dtype=torch.uint8)
    _out_dtype(out_dtype, "fp8_dequant")
    _check_dev(q, s)
    out = torch.empty((rows, cols), dtype=out_dtype, device=q.device)
    _call("fp8_dequant", _ptr(q.contiguous()), _ptr(s.contiguous()), gran, rows, cols, _ptr(out),
          _dtype_code(out), _stream(q))
    return out


def fp8_dequant_fmt(q, s, gran, fmt, out_dtype=torch.float32):
    """fp8_dequant for codes of format fmt."""
    _check_2d_codes(q, "fp8_dequant_fmt: q")
    rows, cols = q.shape
    _need(q, "fp8_dequant_fmt: q", contiguous=True)
    _need(s, "fp8_dequant_fmt: s", shape=_scale_shape(rows, cols, gran), dtype=torch.uint8, contiguous=True)
    _out_dtype(out_dtype, "fp8_dequant_fmt")
    _check_dev(q, s)
    out = torch.empty((rows, cols), dtype=out_dtype, device=q.device)
    _call("fp8_dequant_fmt", _ptr(q), _ptr(s), gran, fmt, rows, cols, _ptr(out), _dtype_code(out), _stream(q))
    return out


def fgb_fp8_encode(x, fmt):
    """Device encoding of a contiguous float32 tensor in format fmt (nearest even, clipped)."""
    _check_dev(x)
    if not x.is_contiguous():
        raise ValueError("fgb_fp8_encode: x must be contiguous")
    q = torch.empty(x.shape, dtype=torch.uint8, device=x.device)
    _call("fgb_fp8_encode", _ptr(x), x.numel(), fmt, _ptr(q), _stream(x))
    return q


def fgb_e4m3_encode(x):
    """Device E4M3 encoding of a float32 tensor (nearest even, saturating)."""
    _check_dev(x)
    x = x.contiguous()
    q = torch.empty(x.shape, dtype=torch.uint8, device=x.device)
    _call("fgb_e4m3_encode", _ptr(x), x.numel(), _ptr(q), _stream(x))
    return q


def fgb_hbm_probe(src, dst, pattern):
    """Diagnostic byte movement in one access pattern (PROBE_*); src and dst are
    contiguous uint8 [rows, cols] tensors (rows, cols multiples of 128), except
    that PROBE_READ's dst holds rows*cols/256 bytes and PROBE_FILL takes no src.
    Returns dst."""
    if pattern not in (PROBE_COPY, PROBE_READ, PROBE_FILL, PROBE_STRIDED_READ, PROBE_STRIDED_WRITE):
        raise ValueError(f"fgb_hbm_probe: unknown pattern {pattern}")
    ref = dst if src is None else src
    _check_2d_codes(ref, "fgb_hbm_probe: src")
    rows, cols = ref.shape
    if rows % 128 or cols % 128:
        raise ValueError("fgb_hbm_probe: rows and cols must be multiples of 128")
    if pattern == PROBE_FILL:
        if src is not None:
            _need(src, "fgb_hbm_probe: src", shape=(rows, cols), dtype=torch.uint8, contiguous=True)
    else:
        _need(src, "fgb_hbm_probe: src", shape=(rows, cols), dtype=torch.uint8, contiguous=True)
    _need(dst, "fgb_hbm_probe: dst", dtype=torch.uint8, contiguous=True)
    need = rows * cols // 256 if pattern == PROBE_READ else rows * cols
    if dst.numel() != need:
        raise ValueError(f"fgb_hbm_probe: dst must hold {need} bytes, got {dst.numel()}")
    _check_dev(src, dst)
    _call("fgb_hbm_probe", _ptr(src), _ptr(dst), rows, cols, pattern, _stream(dst))
    return dst


def fp8_direct_transpose(q, s, s_gran=ROW1x128):
    """Scaling-aware transpose: (q [T, C], s) -> (qt [C, T], st)."""
    _check_2d_codes(q, "fp8_direct_transpose: q")
    T, Cc = q.shape
    if s_gran not in (ROW1x128, BLOCK128):
        raise ValueError("fp8_direct_transpose: s_gran must be ROW1x128 or BLOCK128")
    _need(s, "fp8_direct_transpose: s", shape=_scale_shape(T, Cc, s_gran), dtype=torch.uint8)
    _check_dev(q, s)
    qt = torch.empty((Cc, T), dtype=torch.uint8, device=q.device)
    if s_gran == ROW1x128:
        st = torch.empty((Cc, T // 128), dtype=torch.uint8, device=q.device)
    else:
        st = torch.empty((Cc // 128, T // 128), dtype=torch.uint8, device=q.device)
    _call("fp8_direct_transpose", _ptr(q.contiguous()), _ptr(s.contiguous()), s_gran, T, Cc,
          _ptr(qt), _ptr(st), _stream(q))
    return qt, st


def fp8_direct_transpose_fmt(q, s, fmt):
    """fp8_direct_transpose (1x128 scales) of codes in format fmt: (q [T, C], s) -> (qt [C, T], st)."""
    _check_2d_codes(q, "fp8_direct_transpose_fmt: q")
    T, Cc = q.shape
    _need(q, "fp8_direct_transpose_fmt: q", contiguous=True)
    _need(s, "fp8_direct_transpose_fmt: s", shape=(T, Cc // 128), dtype=torch.uint8, contiguous=True)
    _check_dev(q, s)
    qt = torch.empty((Cc, T), dtype=torch.uint8, device=q.device)
    st = torch.empty((Cc, T // 128), dtype=torch.uint8, device=q.device)
    _call("fp8_direct_transpose_fmt", _ptr(q), _ptr(s), fmt, T, Cc, _ptr(qt), _ptr(st), _stream(q))
    return qt, st


def fp8_block_transpose_batched(q, s):
    """Per-matrix 128x128-block transposes: q [G, rows, cols] -> qt [G, cols, rows]."""
    if q.dim() != 3:
        raise ValueError("fp8_block_transpose_batched: q must be [G, rows, cols]")
    G, rows, cols = q.shape
    _need(q, "fp8_block_transpose_batched: q", dtype=torch.uint8)
    _need(s, "fp8_block_transpose_batched: s", shape=(G, rows // 128, cols // 128), dtype=torch.uint8)
    _check_dev(q, s)
    qt = torch.empty((G, cols, rows), dtype=torch.uint8, device=q.device)
    st = torch.empty((G, cols // 128, rows // 128), dtype=torch.uint8, device=q.device)
    _call("fp8_block_transpose_batched", _ptr(q.contiguous()), _ptr(s.contiguous()), G, rows, cols, _ptr(qt),
          _ptr(st), _stream(q))
    return qt, st


def grouped_k_cap(M_cap, G):
    """Host bound on the columns of the per-expert transposed copy."""
    return (M_cap + 127 * G + 127) // 128 * 128


def fp8_grouped_direct_transpose(q, s, group_offsets, K_cap=None):
    """Direct transpose of expert segments: q [M_cap, C] -> (qt [C, K_cap], st, k_offsets [G+1])."""
    _check_2d_codes(q, "fp8_grouped_direct_transpose: q")
    M_cap, Cc = q.shape
    _need(s, "fp8_grouped_direct_transpose: s", shape=(M_cap, Cc // 128), dtype=torch.uint8)
    if group_offsets.dim() != 1 or group_offsets.numel() < 2:
        raise ValueError("fp8_grouped_direct_transpose: group_offsets must be [G+1] with G >= 1")
    _need(group_offsets, "fp8_grouped_direct_transpose: group_offsets", dtype=torch.int32, contiguous=True)
    _check_dev(q, s, group_offsets)
    G = group_offsets.numel() - 1
    if K_cap is None:
        K_cap = grouped_k_cap(M_cap, G)
    qt = torch.empty((Cc, K_cap), dtype=torch.uint8, device=q.device)
    st = torch.empty((Cc, K_cap // 128), dtype=torch.uint8, device=q.device)
    koff = torch.empty(G + 1, dtype=torch.int32, device=q.device)
    _call("fp8_grouped_direct_transpose", _ptr(q.contiguous()), _ptr(s.contiguous()), M_cap, Cc,
          _ptr(group_offsets), G, _ptr(qt), _ptr(st), K_cap, _ptr(koff), _stream(q))
    return qt, st, koff


def fp8_naive_transpose_workspace_size(rows, cols):
    return int(_lib.fp8_naive_transpose_workspace_size(rows, cols))


def fp8_naive_transpose(q, s, workspace=None):
    """Three-pass baseline (dequantize, transpose, requantize): (q [T, C], s) -> (qt [C, T], st)."""
    _check_2d_codes(q, "fp8_naive_transpose: q")
    T, Cc = q.shape
    _need(s, "fp8_naive_transpose: s", shape=(T, Cc // 128), dtype=torch.uint8)
    if workspace is not None:
        _need(workspace, "fp8_naive_transpose: workspace", dtype=torch.uint8, contiguous=True)
    _check_dev(q, s, workspace)
    qt = torch.empty((Cc, T), dtype=torch.uint8, device=q.device)
    st = torch.empty((Cc, T // 128), dtype=torch.uint8, device=q.device)
    if workspace is None:
        workspace = torch.empty(fp8_naive_transpose_workspace_size(T, Cc), dtype=torch.uint8,
                                device=q.device)
    _call("fp8_naive_transpose", _ptr(q.contiguous()), _ptr(s.contiguous()), T, Cc, _ptr(qt), _ptr(st),
          _ptr(workspace), workspace.numel(), _stream(q))
    return qt, st


def fp8_block_gemm(a, sa, a_gran, b, sb, b_gran, b_l1=None, g1=0, out_dtype=torch.bfloat16,
                   d=None, accumulate=False, mode=GEMM_EXACT):
    """D = A * B^T with blockwise scales (A [M,K], B [N,K] codes) -> D [M, N]."""
    _check_2d_codes(a, "fp8_block_gemm: a")
    _check_2d_codes(b, "fp8_block_gemm: b")
    M, K = a.shape
    N = b.shape[0]
    if b.shape[1] != K:
        raise ValueError("fp8_block_gemm: a and b must have the same K")
    _need(sa, "fp8_block_gemm: sa", shape=_scale_shape(M, K, a_gran), dtype=torch.uint8)
    _need(sb, "fp8_block_gemm: sb", shape=_scale_shape(N, K, b_gran), dtype=torch.uint8)
    if b_l1 is not None:
        _need(b_l1, "fp8_block_gemm: b_l1", shape=(N,), dtype=torch.float32, contiguous=True)
        if b_gran != ROW1x32:
            raise ValueError("fp8_block_gemm: b_l1 needs 1x32 B scales (b_gran ROW1x32)")
    d = _gemm_out(d, M, N, out_dtype, "fp8_block_gemm")
    _check_dev(a, sa, b, sb, b_l1, d)
    if d is None:
        d = torch.empty((M, N), dtype=out_dtype, device=a.device)
    _call("fp8_block_gemm", _ptr(a), _ptr(sa.contiguous()), a_gran, _ptr(b), _ptr(sb.contiguous()),
          b_gran, _ptr(b_l1), g1, M, N, K, _row_ld(a), _row_ld(b), _ptr(d), _dtype_code(d),
          _row_ld(d), int(bool(accumulate)), mode, None, 0, _stream(a))
    return d


def fp8_block_gemm_fmt(a, sa, a_gran, a_fmt, b, sb, b_gran, b_fmt=E4M3, out_dtype=torch.bfloat16, d=None,
                       accumulate=False, mode=GEMM_EXACT):
    """fp8_block_gemm with the operands' element formats (A: E4M3 or E5M2; B: E4M3)."""
    _check_2d_codes(a, "fp8_block_gemm_fmt: a")
    _check_2d_codes(b, "fp8_block_gemm_fmt: b")
    M, K = a.shape
    N = b.shape[0]
    if b.shape[1] != K:
        raise ValueError("fp8_block_gemm_fmt: a and b must have the same K")
    _need(sa, "fp8_block_gemm_fmt: sa", shape=_scale_shape(M, K, a_gran), dtype=torch.uint8, contiguous=True)
    _need(sb, "fp8_block_gemm_fmt: sb", shape=_scale_shape(N, K, b_gran), dtype=torch.uint8, contiguous=True)
    d = _gemm_out(d, M, N, out_dtype, "fp8_block_gemm_fmt")
    _check_dev(a, sa, b, sb, d)
    if d is None:
        d = torch.empty((M, N), dtype=out_dtype, device=a.device)
    _call("fp8_block_gemm_fmt", _ptr(a), _ptr(sa), a_gran, a_fmt, _ptr(b), _ptr(sb), b_gran, b_fmt, None, 0, M, N, K,
          _row_ld(a), _row_ld(b), _ptr(d), _dtype_code(d), _row_ld(d), int(bool(accumulate)), mode, _stream(a))
    return d


def fp8_grouped_gemm_masked(a, sa, b, sb, masked_m, out_dtype=torch.bfloat16, d=None, mode=GEMM_EXACT):
    """Masked grouped GEMM: a [G, M_max, K], b [G, N, K], masked_m int32 [G] (device) -> d [G, M_max, N];
    rows m >= masked_m[g] of d are not written."""
    name = "fp8_grouped_gemm_masked"
    if a.dim() != 3 or b.dim() != 3:
        raise ValueError(f"{name}: a must be [G, M_max, K] and b [G, N, K]")
    G, M_max, K = a.shape
    N = b.shape[1]
    _need(a, f"{name}: a", dtype=torch.uint8, contiguous=True)
    _need(b, f"{name}: b", shape=(G, N, K), dtype=torch.uint8, contiguous=True)
    _need(sa, f"{name}: sa", shape=(G, M_max, K // 128), dtype=torch.uint8, contiguous=True)
    _need(sb, f"{name}: sb", shape=(G, (N + 127) // 128, K // 128), dtype=torch.uint8, contiguous=True)
    _need(masked_m, f"{name}: masked_m", shape=(G,), dtype=torch.int32, contiguous=True)
    if d is None:
        _out_dtype(out_dtype, name)
    else:
        _out_dtype(d.dtype, name)
        _need(d, f"{name}: d", shape=(G, M_max, N), contiguous=True)
    _check_dev(a, sa, b, sb, masked_m, d)
    if d is None:
        d = torch.empty((G, M_max, N), dtype=out_dtype, device=a.device)
    _call("fp8_grouped_gemm_masked", _ptr(a), _ptr(sa), _ptr(b), _ptr(sb), _ptr(masked_m), G, M_max, N, K, _ptr(d),
          _dtype_code(d), mode, _stream(a))
    return d


def fp8_grouped_gemm(a, sa, b, sb, group_offsets, out_dtype=torch.bfloat16, d=None,
                     mode=GEMM_EXACT):
    """M-grouped contiguous GEMM: a [M_cap, K], b [G, N, K], offsets [G+1] (device) -> d [M_cap, N]."""
    name = "fp8_grouped_gemm"
    _check_2d_codes(a, f"{name}: a")
    M_cap, K = a.shape
    if b.dim() != 3:
        raise ValueError(f"{name}: b must be [G, N, K]")
    G, N = b.shape[0], b.shape[1]
    _need(b, f"{name}: b", shape=(G, N, K), dtype=torch.uint8)
    _need(sa, f"{name}: sa", shape=(M_cap, K // 128), dtype=torch.uint8)
    _need(sb, f"{name}: sb", shape=(G, (N + 127) // 128, K // 128), dtype=torch.uint8)
    _need(group_offsets, f"{name}: group_offsets", shape=(G + 1,), dtype=torch.int32, contiguous=True)
    d = _gemm_out(d, M_cap, N, out_dtype, name, contiguous=True)
    _check_dev(a, sa, b, sb, group_offsets, d)
    if d is None:
        d = torch.empty((M_cap, N), dtype=out_dtype, device=a.device)
    _call("fp8_grouped_gemm", _ptr(a.contiguous()), _ptr(sa.contiguous()), _ptr(b.contiguous()),
          _ptr(sb.contiguous()), _ptr(group_offsets), G, M_cap, N, K, _ptr(d), _dtype_code(d),
          mode, _stream(a))
    return d


def fp8_kgrouped_gemm(a, sa, b, sb, k_offsets, out_dtype=torch.float32, d=None, accumulate=False,
                      mode=GEMM_EXACT):
    """K-grouped GEMM (expert Wgrad): a [M, K_cap], b [N, K_cap], k_offsets [G+1] (device) -> d [G, M, N]."""
    name = "fp8_kgrouped_gemm"
    _check_2d_codes(a, f"{name}: a")
    _check_2d_codes(b, f"{name}: b")
    M, K_cap = a.shape
    N = b.shape[0]
    if b.shape[1] != K_cap:
        raise ValueError("fp8_kgrouped_gemm: a and b must have the same K capacity")
    if k_offsets.dim() != 1 or k_offsets.numel() < 2:
        raise ValueError(f"{name}: k_offsets must be [G+1] with G >= 1")
    G = k_offsets.numel() - 1
    for t, nm in ((a, "a"), (b, "b")):
        _need(t, f"{name}: {nm}", contiguous=True)
    _need(sa, f"{name}: sa", shape=(M, K_cap // 128), dtype=torch.uint8, contiguous=True)
    _need(sb, f"{name}: sb", shape=(N, K_cap // 128), dtype=torch.uint8, contiguous=True)
    _need(k_offsets, f"{name}: k_offsets", dtype=torch.int32, contiguous=True)
    if d is None:
        _out_dtype(out_dtype, name)
    else:
        _out_dtype(d.dtype, name)
        _need(d, f"{name}: d", shape=(G, M, N), contiguous=True)
    _check_dev(a, sa, b, sb, k_offsets, d)
    if d is None:
        d = torch.empty((G, M, N), dtype=out_dtype, device=a.device)
    _call("fp8_kgrouped_gemm", _ptr(a), _ptr(sa), _ptr(b), _ptr(sb), _ptr(k_offsets), G, M, N, K_cap,
          _ptr(d), _dtype_code(d), int(bool(accumulate)), mode, _stream(a))
    return d


def permute_pad_workspace_size(T, topk, G):
    return int(_lib.permute_pad_workspace_size(T, topk, G))


def permute_pad(xq, xs, topk_idx, G, pad_multiple=16, M_cap=None, workspace=None, out=None):
    """Fused permute + pad -> (out_q [M_cap, H], out_s, row_map [T, topk], group_offsets [G+1])."""
    name = "permute_pad"
    _check_2d_codes(xq, f"{name}: xq")
    T, H = xq.shape
    _need(xs, f"{name}: xs", shape=(T, H // 128), dtype=torch.uint8)
    if topk_idx.dim() != 2 or topk_idx.shape[0] != T:
        raise ValueError(f"{name}: topk_idx must be [T, topk]")
    _need(topk_idx, f"{name}: topk_idx", dtype=torch.int32)
    topk = topk_idx.shape[1]
    if M_cap is None:
        M_cap = T * topk + (pad_multiple - 1) * G
    if out is not None:
        out_q, out_s, row_map, offs = out
        _need(out_q, f"{name}: out_q", shape=(M_cap, H), dtype=torch.uint8, contiguous=True)
        _need(out_s, f"{name}: out_s", shape=(M_cap, H // 128), dtype=torch.uint8, contiguous=True)
        _need(row_map, f"{name}: row_map", shape=(T, topk), dtype=torch.int32, contiguous=True)
        _need(offs, f"{name}: group_offsets", shape=(G + 1,), dtype=torch.int32, contiguous=True)
    if workspace is not None:
        _need(workspace, f"{name}: workspace", dtype=torch.uint8, contiguous=True)
    _check_dev(xq, xs, topk_idx, workspace, *(out or ()))
    dev = xq.device
    if out is None:
        out_q = torch.empty((M_cap, H), dtype=torch.uint8, device=dev)
        out_s = torch.empty((M_cap, H // 128), dtype=torch.uint8, device=dev)
        row_map = torch.empty((T, topk), dtype=torch.int32, device=dev)
        offs = torch.empty((G + 1,), dtype=torch.int32, device=dev)
    else:
        out_q, out_s, row_map, offs = out
    ws_need = permute_pad_workspace_size(T, topk, G)
    if workspace is None:
        workspace = torch.empty((max(ws_need, 1),), dtype=torch.uint8, device=dev)
    _call("permute_pad", _ptr(xq.contiguous()), _ptr(xs.contiguous()), _ptr(topk_idx.contiguous()),
          T, topk, G, H, pad_multiple, _ptr(out_q), _ptr(out_s), _ptr(row_map), _ptr(offs), M_cap,
          _ptr(workspace), workspace.numel(), _stream(xq))
    return out_q, out_s, row_map, offs


PERMUTE_PAD_NOALLOC_SCRATCH_BYTES = 1 << 20


def permute_pad_noalloc(xq, xs, topk_idx, G, out, pad_multiple=16):
    """permute_pad without any allocation: the caller passes the outputs
    out = (out_q [M_cap, H], out_s [M_cap, H/128], row_map [T, topk], group_offsets [G+1]); the workspace
    is the library's per-GPU scratch array (see include/fgb.h for the size limit and the concurrency rule)."""
    name = "permute_pad_noalloc"
    _check_2d_codes(xq, f"{name}: xq")
    T, H = xq.shape
    _need(xs, f"{name}: xs", shape=(T, H // 128), dtype=torch.uint8, contiguous=True)
    _need(xq, f"{name}: xq", contiguous=True)
    if topk_idx.dim() != 2 or topk_idx.shape[0] != T:
        raise ValueError(f"{name}: topk_idx must be [T, topk]")
    _need(topk_idx, f"{name}: topk_idx", dtype=torch.int32, contiguous=True)
    topk = topk_idx.shape[1]
    if out is None or len(out) != 4:
        raise ValueError(f"{name}: out must be (out_q, out_s, row_map, group_offsets)")
    out_q, out_s, row_map, offs = out
    if out_q.dim() != 2:
        raise ValueError(f"{name}: out_q must be [M_cap, H]")
    M_cap = out_q.shape[0]
    _need(out_q, f"{name}: out_q", shape=(M_cap, H), dtype=torch.uint8, contiguous=True)
    _need(out_s, f"{name}: out_s", shape=(M_cap, H // 128), dtype=torch.uint8, contiguous=True)
    _need(row_map, f"{name}: row_map", shape=(T, topk), dtype=torch.int32, contiguous=True)
    _need(offs, f"{name}: group_offsets", shape=(G + 1,), dtype=torch.int32, contiguous=True)
    _check_dev(xq, xs, topk_idx, out_q, out_s, row_map, offs)
    _call(name, _ptr(xq), _ptr(xs), _ptr(topk_idx), T, topk, G, H, pad_multiple, _ptr(out_q), _ptr(out_s),
          _ptr(row_map), _ptr(offs), M_cap, _stream(xq))
    return out_q, out_s, row_map, offs


def unpermute_unpad(y, row_map, probs=None, out=None):
    """out [T, H] bf16 = sum over slots of probs * y[row_map] (fmaf fold, RNE to bf16)."""
    name = "unpermute_unpad"
    if y.dim() != 2 or row_map.dim() != 2:
        raise ValueError(f"{name}: y must be [rows, H] and row_map [T, topk]")
    _need(y, f"{name}: y", dtype=torch.bfloat16)
    _need(row_map, f"{name}: row_map", dtype=torch.int32)
    T, topk = row_map.shape
    H = y.shape[1]
    if probs is not None:
        _need(probs, f"{name}: probs", shape=(T, topk), dtype=torch.float32)
    if out is not None:
        _need(out, f"{name}: out", shape=(T, H), dtype=torch.bfloat16, contiguous=True)
    _check_dev(y, row_map, probs, out)
    if out is None:
        out = torch.empty((T, H), dtype=torch.bfloat16, device=y.device)
    _call("unpermute_unpad", _ptr(y.contiguous()), _ptr(row_map.contiguous()),
          _ptr(None if probs is None else probs.contiguous()), T, topk, H, _ptr(out), _stream(y))
    return out


def unpermute_backward_workspace_size(M_cap):
    return int(_lib.unpermute_backward_workspace_size(M_cap))


def unpermute_backward(dout, row_map, probs, M_cap, dy=None, workspace=None):
    """Gradient of unpermute_unpad: dout bf16 [T, H] -> dy bf16 [M_cap, H] (padding rows zero)."""
    name = "unpermute_backward"
    if dout.dim() != 2 or row_map.dim() != 2 or row_map.shape[0] != dout.shape[0]:
        raise ValueError(f"{name}: dout must be [T, H] and row_map [T, topk]")
    _need(dout, f"{name}: dout", dtype=torch.bfloat16)
    _need(row_map, f"{name}: row_map", dtype=torch.int32)
    T, H = dout.shape
    topk = row_map.shape[1]
    if probs is not None:
        _need(probs, f"{name}: probs", shape=(T, topk), dtype=torch.float32)
    if dy is not None:
        _need(dy, f"{name}: dy", shape=(M_cap, H), dtype=torch.bfloat16, contiguous=True)
    if workspace is not None:
        _need(workspace, f"{name}: workspace", dtype=torch.uint8, contiguous=True)
    _check_dev(dout, row_map, probs, dy, workspace)
    if dy is None:
        dy = torch.empty((M_cap, H), dtype=torch.bfloat16, device=dout.device)
    if workspace is None:
        workspace = torch.empty(max(unpermute_backward_workspace_size(M_cap), 1), dtype=torch.uint8,
                                device=dout.device)
    _call("unpermute_backward", _ptr(dout.contiguous()), _ptr(row_map.contiguous()),
          _ptr(None if probs is None else probs.contiguous()), T, topk, H, M_cap, _ptr(dy), _ptr(workspace),
          workspace.numel(), _stream(dout))
    return dy


def unpermute_backward_quant(dout, row_map, probs, M_cap, q=None, s=None, workspace=None):
    """unpermute_backward + 1x128 quant in one pass: dout bf16 [T, H] -> (q [M_cap, H], s [M_cap, H/128])."""
    name = "unpermute_backward_quant"
    if dout.dim() != 2 or row_map.dim() != 2 or row_map.shape[0] != dout.shape[0]:
        raise ValueError(f"{name}: dout must be [T, H] and row_map [T, topk]")
    T, H = dout.shape
    topk = row_map.shape[1]
    _need(dout, f"{name}: dout", dtype=torch.bfloat16, contiguous=True)
    _need(row_map, f"{name}: row_map", dtype=torch.int32, contiguous=True)
    if probs is not None:
        _need(probs, f"{name}: probs", shape=(T, topk), dtype=torch.float32, contiguous=True)
    if q is not None:
        _need(q, f"{name}: q", shape=(M_cap, H), dtype=torch.uint8, contiguous=True)
    if s is not None:
        _need(s, f"{name}: s", shape=(M_cap, H // 128), dtype=torch.uint8, contiguous=True)
    if workspace is not None:
        _need(workspace, f"{name}: workspace", dtype=torch.uint8, contiguous=True)
    _check_dev(dout, row_map, probs, q, s, workspace)
    if q is None:
        q = torch.empty((M_cap, H), dtype=torch.uint8, device=dout.device)
    if s is None:
        s = torch.empty((M_cap, H // 128), dtype=torch.uint8, device=dout.device)
    if workspace is None:
        workspace = torch.empty(max(unpermute_backward_workspace_size(M_cap), 1), dtype=torch.uint8,
                                device=dout.device)
    _call("unpermute_backward_quant", _ptr(dout), _ptr(row_map), _ptr(probs), T, topk, H, M_cap, _ptr(q),
          _ptr(s), _ptr(workspace), workspace.numel(), _stream(dout))
    return q, s


def swiglu_quant_cache(h, group_offsets=None, q=None, s=None, hq=None, hs=None):
    """swiglu_quant that also returns the FP8 cache of h: -> (q [M, F], s, hq [M, 2F], hs [M, 2F/128])."""
    name = "swiglu_quant_cache"
    if h.dim() != 2:
        raise ValueError(f"{name}: h must be [M, 2F]")
    _need(h, f"{name}: h", dtype=torch.bfloat16)
    M, F2 = h.shape
    F = F2 // 2
    for t, nm, shp in ((q, "q", (M, F)), (s, "s", (M, F // 128)), (hq, "hq", (M, F2)), (hs, "hs", (M, F2 // 128))):
        if t is not None:
            _need(t, f"{name}: {nm}", shape=shp, dtype=torch.uint8, contiguous=True)
    if group_offsets is not None:
        _need(group_offsets, f"{name}: group_offsets", dtype=torch.int32, contiguous=True)
    _check_dev(h, group_offsets, q, s, hq, hs)
    if q is None:
        q = torch.empty((M, F), dtype=torch.uint8, device=h.device)
    if s is None:
        s = torch.empty((M, F // 128), dtype=torch.uint8, device=h.device)
    if hq is None:
        hq = torch.empty((M, F2), dtype=torch.uint8, device=h.device)
    if hs is None:
        hs = torch.empty((M, F2 // 128), dtype=torch.uint8, device=h.device)
    G = 0 if group_offsets is None else group_offsets.numel() - 1
    _call("swiglu_quant_cache", _ptr(h), M, F, _row_ld(h), _ptr(group_offsets), G, _ptr(q), _ptr(s), _ptr(hq),
          _ptr(hs), _stream(h))
    return q, s, hq, hs


def swiglu_quant(h, group_offsets=None, q=None, s=None):
    """SwiGLU of h [M, 2F] (gate|up, bf16) + 1x128 quant -> (q [M, F], s [M, F/128])."""
    name = "swiglu_quant"
    if h.dim() != 2:
        raise ValueError(f"{name}: h must be [M, 2F]")
    _need(h, f"{name}: h", dtype=torch.bfloat16)
    M, F2 = h.shape
    F = F2 // 2
    for t, nm, shp in ((q, "q", (M, F)), (s, "s", (M, F // 128))):
        if t is not None:
            _need(t, f"{name}: {nm}", shape=shp, dtype=torch.uint8, contiguous=True)
    if group_offsets is not None:
        _need(group_offsets, f"{name}: group_offsets", dtype=torch.int32, contiguous=True)
    _check_dev(h, group_offsets, q, s)
    if q is None:
        q = torch.empty((M, F), dtype=torch.uint8, device=h.device)
    if s is None:
        s = torch.empty((M, F // 128), dtype=torch.uint8, device=h.device)
    G = 0 if group_offsets is None else group_offsets.numel() - 1
    _call("swiglu_quant", _ptr(h), M, F, _row_ld(h), _ptr(group_offsets), G, _ptr(q), _ptr(s),
          _stream(h))
    return q, s


def swiglu_f32(g, u):
    """Diagnostic: a = silu(g) * u in fp32, elementwise, the arithmetic of swiglu_quant."""
    _check_dev(g, u)
    g = g.contiguous().float()
    u = u.contiguous().float()
    if g.shape != u.shape:
        raise ValueError("swiglu_f32: g and u must have the same shape")
    a = torch.empty_like(g)
    _call("swiglu_f32", _ptr(g), _ptr(u), g.numel(), _ptr(a), _stream(g))
    return a


def dswiglu_f32(g, u, da):
    """Diagnostic: (du, dg) of the SwiGLU backward in fp32, elementwise, the arithmetic of dswiglu_quant."""
    _check_dev(g, u, da)
    g, u, da = (t.contiguous().float() for t in (g, u, da))
    if g.shape != u.shape or g.shape != da.shape:
        raise ValueError("dswiglu_f32: g, u and da must have the same shape")
    du = torch.empty_like(g)
    dg = torch.empty_like(g)
    _call("dswiglu_f32", _ptr(g), _ptr(u), _ptr(da), g.numel(), _ptr(du), _ptr(dg), _stream(g))
    return du, dg


def dswiglu_quant(hq, hs, da, group_offsets=None, dq=None, ds=None):
    """SwiGLU backward from the FP8-cached input: (hq [M,2F], hs, da bf16 [M,F]) -> (dq [M,2F], ds)."""
    name = "dswiglu_quant"
    _check_2d_codes(hq, f"{name}: hq")
    M, F2 = hq.shape
    _need(hs, f"{name}: hs", shape=(M, F2 // 128), dtype=torch.uint8)
    _need(da, f"{name}: da", shape=(M, F2 // 2), dtype=torch.bfloat16)
    for t, nm, shp in ((dq, "dq", (M, F2)), (ds, "ds", (M, F2 // 128))):
        if t is not None:
            _need(t, f"{name}: {nm}", shape=shp, dtype=torch.uint8, contiguous=True)
    if group_offsets is not None:
        _need(group_offsets, f"{name}: group_offsets", dtype=torch.int32, contiguous=True)
    _check_dev(hq, hs, da, group_offsets, dq, ds)
    if dq is None:
        dq = torch.empty((M, F2), dtype=torch.uint8, device=hq.device)
    if ds is None:
        ds = torch.empty((M, F2 // 128), dtype=torch.uint8, device=hq.device)
    G = 0 if group_offsets is None else group_offsets.numel() - 1
    _call("dswiglu_quant", _ptr(hq.contiguous()), _ptr(hs.contiguous()), _ptr(da.contiguous()), M, F2 // 2,
          _ptr(group_offsets), G, _ptr(dq), _ptr(ds), _stream(hq))
    return dq, ds


def mx2_quant(x, g1=10240):
    """MOSS two-level quantization of x [R, C] bf16 -> (q, s2 [R, C/32], s1 fp32 [R, ceil(C/g1)])."""
    if x.dim() != 2:
        raise ValueError("mx2_quant: x must be 2-D")
    _need(x, "mx2_quant: x", dtype=torch.bfloat16)
    _check_dev(x)
    R, Cc = x.shape
    ng = (Cc + g1 - 1) // g1
    q = torch.empty((R, Cc), dtype=torch.uint8, device=x.device)
    s2 = torch.empty((R, Cc // 32), dtype=torch.uint8, device=x.device)
    s1 = torch.empty((R, ng), dtype=torch.float32, device=x.device)
    _call("mx2_quant", _ptr(x.contiguous()), R, Cc, g1, _ptr(q), _ptr(s2), _ptr(s1), _stream(x))
    return q, s2, s1


def mx2_quant_rule(x, g1=10240, rule=SCALE_CEIL):
    """mx2_quant with the level-2 exponent rule chosen (SCALE_CEIL or SCALE_OCP_FLOOR)."""
    if x.dim() != 2:
        raise ValueError("mx2_quant_rule: x must be 2-D")
    _need(x, "mx2_quant_rule: x", dtype=torch.bfloat16, contiguous=True)
    _check_dev(x)
    R, Cc = x.shape
    ng = (Cc + g1 - 1) // g1
    q = torch.empty((R, Cc), dtype=torch.uint8, device=x.device)
    s2 = torch.empty((R, Cc // 32), dtype=torch.uint8, device=x.device)
    s1 = torch.empty((R, ng), dtype=torch.float32, device=x.device)
    _call("mx2_quant_rule", _ptr(x), R, Cc, g1, rule, _ptr(q), _ptr(s2), _ptr(s1), _stream(x))
    return q, s2, s1


def mx2_dequant(q, s2, s1, g1=10240):
    """x_hat = (decode(q) * 2^(s2-127)) * s1 -> fp32 [R, C]."""
    _check_2d_codes(q, "mx2_dequant: q")
    R, Cc = q.shape
    _need(s2, "mx2_dequant: s2", shape=(R, Cc // 32), dtype=torch.uint8)
    if g1 <= 0:
        raise ValueError("mx2_dequant: g1 must be positive")
    _need(s1, "mx2_dequant: s1", shape=(R, (Cc + g1 - 1) // g1), dtype=torch.float32)
    _check_dev(q, s2, s1)
    out = torch.empty((R, Cc), dtype=torch.float32, device=q.device)
    _call("mx2_dequant", _ptr(q.contiguous()), _ptr(s2.contiguous()), _ptr(s1.contiguous()), R, Cc,
          g1, _ptr(out), _stream(q))
    return out
