"""Row-parallel runner of the CPU oracle (test infrastructure only, like the
rest of oracle/).

Each function applies the same single-threaded oracle routine to independent
slices of its input -- rows, 128-row blocks, tokens or sampled outputs -- on
a pool of threads (the C routines run without the interpreter lock, called
through ctypes) and assembles the slices.  Every slice is computed by exactly
the code that computes it in a one-thread call, so the results are bit for
bit those of the single-threaded oracle (checked in
tests/test_oracle_parallel.py).  permute_pad and the unpermute backward are
not row-parallel in the oracle (a scan over every token, a scatter into the
padded layout) and run on one thread.
"""
import concurrent.futures as cf

import numpy as np

from . import (block_gemm_sampled, direct_transpose, dswiglu_quant, mx2_quant, quant_blockwise, quant_rowwise,
               swiglu_quant, unpermute_unpad)


def _ranges(n, parts, align=1):
    """Split [0, n) into at most `parts` ranges whose inner bounds are multiples of align."""
    units = (n + align - 1) // align
    parts = max(1, min(parts, units))
    out = []
    for i in range(parts):
        lo = (units * i // parts) * align
        hi = min(n, (units * (i + 1) // parts) * align)
        if hi > lo:
            out.append((lo, hi))
    return out


def _map(fn, ranges, threads):
    if threads <= 1 or len(ranges) <= 1:
        return [fn(lo, hi) for lo, hi in ranges]
    with cf.ThreadPoolExecutor(threads) as ex:
        return list(ex.map(lambda r: fn(*r), ranges))


def quant_rowwise_par(x, group=128, threads=8):
    parts = _map(lambda lo, hi: quant_rowwise(x[lo:hi], group), _ranges(x.shape[0], threads), threads)
    return np.concatenate([p[0] for p in parts]), np.concatenate([p[1] for p in parts])


def quant_blockwise_par(w, threads=8):
    """128 x 128 blocks: slices of whole 128-row blocks (a partial last block stays whole)."""
    parts = _map(lambda lo, hi: quant_blockwise(w[lo:hi]), _ranges(w.shape[0], threads, 128), threads)
    return np.concatenate([p[0] for p in parts]), np.concatenate([p[1] for p in parts])


def direct_transpose_par(q, s, threads=8):
    """Slices of whole 128-row blocks of T; each gives its own columns of the transposed copy."""
    parts = _map(lambda lo, hi: direct_transpose(q[lo:hi], s[lo:hi]), _ranges(q.shape[0], threads, 128), threads)
    return np.concatenate([p[0] for p in parts], axis=1), np.concatenate([p[1] for p in parts], axis=1)


def block_gemm_sampled_par(a, sa, a_gran, b, sb, b_gran, mi, ni, b_l1=None, g1=0, threads=8):
    mi = np.asarray(mi, np.int64)
    ni = np.asarray(ni, np.int64)
    parts = _map(lambda lo, hi: block_gemm_sampled(a, sa, a_gran, b, sb, b_gran, mi[lo:hi], ni[lo:hi], b_l1, g1),
                 _ranges(mi.size, threads), threads)
    return np.concatenate(parts) if parts else np.empty(0)


def unpermute_unpad_par(y, row_map, probs=None, threads=8):
    row_map = np.asarray(row_map, np.int32)
    parts = _map(lambda lo, hi: unpermute_unpad(y, row_map[lo:hi], None if probs is None else probs[lo:hi]),
                 _ranges(row_map.shape[0], threads), threads)
    return np.concatenate(parts)


def swiglu_quant_par(h, threads=8):
    parts = _map(lambda lo, hi: swiglu_quant(h[lo:hi]), _ranges(h.shape[0], threads), threads)
    return np.concatenate([p[0] for p in parts]), np.concatenate([p[1] for p in parts])


def dswiglu_quant_par(hq, hs, da, threads=8):
    parts = _map(lambda lo, hi: dswiglu_quant(hq[lo:hi], hs[lo:hi], da[lo:hi], None), _ranges(hq.shape[0], threads),
                 threads)
    return np.concatenate([p[0] for p in parts]), np.concatenate([p[1] for p in parts])


def mx2_quant_par(x, g1=10240, threads=8):
    parts = _map(lambda lo, hi: mx2_quant(x[lo:hi], g1), _ranges(x.shape[0], threads), threads)
    return tuple(np.concatenate([p[i] for p in parts]) for i in range(3))
