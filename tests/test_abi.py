"""C ABI checks that need no GPU: the library loads, exports every symbol the
header declares, and rejects bad arguments on the host with the documented
status codes before anything is enqueued."""
import ctypes as C
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def header_functions():
    src = open(os.path.join(ROOT, "include", "fgb.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b([a-z0-9_]+)\s*\(", src)) - {"defined"})


def test_header_symbols_exported():
    import fine_grained_blockwise_amd as fgb
    names = header_functions()
    assert len(names) >= 14
    L = fgb.lib()
    for n in names:
        assert hasattr(L, n), n
    assert set(fgb.symbols()) == set(names)
    assert fgb.lib().fgb_version().decode().startswith("fgb")


def test_library_has_gfx950_code_object():
    from fine_grained_blockwise_amd import LIB_PATH
    blob = open(LIB_PATH, "rb").read()
    assert b"gfx950" in blob


P = C.c_void_p


def _fake(addr=0x1000):
    return C.c_void_p(addr)


def test_quant_rowwise_validation():
    import fine_grained_blockwise_amd as fgb
    L = fgb.lib()
    assert L.fp8_quant_rowwise(None, 1, 4, 128, 128, 128, _fake(), 128, _fake(), 1, None) == 1
    assert b"null" in L.fgb_last_error()
    assert L.fp8_quant_rowwise(_fake(), 7, 4, 128, 128, 128, _fake(), 128, _fake(), 1, None) == 2
    assert L.fp8_quant_rowwise(_fake(), 1, 4, 100, 128, 128, _fake(), 128, _fake(), 1, None) == 1
    assert L.fp8_quant_rowwise(_fake(), 1, 4, 128, 128, 64, _fake(), 128, _fake(), 1, None) == 2
    assert L.fp8_quant_rowwise(_fake(), 1, 4, 128, 120, 128, _fake(), 128, _fake(), 1, None) == 1
    assert L.fp8_quant_rowwise(_fake(0x1001), 1, 4, 128, 128, 128, _fake(), 128, _fake(), 1, None) == 1
    assert b"aligned" in L.fgb_last_error()
    # rows == 0 is a no-op that touches nothing
    assert L.fp8_quant_rowwise(_fake(), 1, 0, 128, 128, 128, _fake(), 128, _fake(), 1, None) == 0


def test_gemm_validation():
    import fine_grained_blockwise_amd as fgb
    L = fgb.lib()
    f = _fake()
    args = dict(a=f, sa=f, ag=0, b=f, sb=f, bg=2, l1=None, g1=0, M=256, N=256, K=512, lda=512,
                ldb=512, d=f, dt=1, ldd=256, acc=0)

    def call(**kw):
        a = dict(args, **kw)
        return L.fp8_block_gemm(a["a"], a["sa"], a["ag"], a["b"], a["sb"], a["bg"], a["l1"], a["g1"],
                                a["M"], a["N"], a["K"], a["lda"], a["ldb"], a["d"], a["dt"],
                                a["ldd"], a["acc"], a.get("mode", 0), None, 0, None)
    assert call(K=500) == 1
    assert call(M=-1) == 1
    assert call(M=0) == 0 and call(N=0) == 0  # empty D: nothing to do, nothing launched
    assert call(M=0, a=None, sa=None, b=None, sb=None, d=None) == 0
    assert call(d=None, K=0) == 1  # a non-empty D must exist
    assert call(lda=500, K=256) == 1
    assert call(ag=2) == 2          # BLOCK128 A scales are not a mode
    assert call(ag=1, bg=2) == 2    # 1x32 must pair with 1x32
    assert call(acc=1, dt=1) == 2   # accumulate needs FP32 output
    assert call(l1=f, g1=256, ag=1, bg=1) == 2  # level-1 factor needs K <= g1
    assert call(l1=f, g1=1024) == 2  # level-1 factor needs 1x32 B scales
    assert call(a=None) == 1
    assert call(mode=2) == 2
    assert call(dt=0, ldd=1 << 23) == 2  # FP32 rows of 2^23 elements or more
    assert call(ag=1, bg=1, sa=_fake(0x1001)) == 1  # 1x32 scales need 4-byte alignment
    assert L.fp8_grouped_gemm(f, f, f, f, f, 0, 100, 256, 512, f, 1, 0, None) == 1
    assert L.fp8_grouped_gemm(f, f, f, f, f, 4, 100, 256, 512, f, 1, 5, None) == 2
    kg = lambda G=4, M=256, N=256, Kc=1024, dt=0, acc=0, mode=0, a=f: L.fp8_kgrouped_gemm(
        a, f, f, f, f, G, M, N, Kc, f, dt, acc, mode, None)
    assert kg(G=0) == 1 and kg(G=1025) == 1
    assert kg(Kc=1000) == 1          # K capacity must be a multiple of 128
    assert kg(M=0) == 1
    assert kg(Kc=1 << 24) == 1       # 256 * K_cap must stay below 2^32
    assert kg(a=_fake(0x1008)) == 1  # codes 16-byte aligned
    assert kg(dt=1, acc=1) == 2      # accumulate needs FP32 output
    assert kg(mode=3) == 2
    assert kg(a=None) == 1


def test_transpose_and_moe_validation():
    import fine_grained_blockwise_amd as fgb
    L = fgb.lib()
    f = _fake()
    assert L.fp8_direct_transpose(f, f, 0, 200, 256, f, f, None) == 1
    assert L.fp8_direct_transpose(f, f, 1, 256, 256, f, f, None) == 2
    assert L.fp8_block_transpose_batched(f, f, 0, 256, 256, f, f, None) == 1
    assert L.fp8_block_transpose_batched(f, f, 4, 200, 256, f, f, None) == 1
    assert L.fp8_grouped_direct_transpose(f, f, 1000, 256, f, 8, f, f, 1024, f, None) == 1  # K_cap too small
    assert L.fp8_grouped_direct_transpose(f, f, 1000, 200, f, 8, f, f, 4096, f, None) == 1  # cols % 128
    assert L.swiglu_quant_cache(f, 64, 256, 512, None, 0, f, f, None, f, None) == 1  # null cache
    assert L.swiglu_quant_cache(f, 64, 200, 512, None, 0, f, f, f, f, None) == 1    # F % 128
    assert L.swiglu_quant_cache(f, 64, 256, 512, None, 0, f, f, _fake(0x1008), f, None) == 1  # alignment
    assert L.unpermute_backward_quant(f, f, None, 64, 8, 200, 1000, f, f, f, 1 << 20, None) == 1  # H % 128
    assert L.unpermute_backward_quant(f, f, None, 64, 8, 256, 1000, f, f, f, 100, None) == 3  # workspace
    assert L.unpermute_backward_quant(f, f, None, 64, 0, 256, 1000, f, f, f, 1 << 20, None) == 1  # topk
    # format variants
    assert L.fp8_quant_rowwise_fmt(f, 1, 4, 256, 256, 128, 2, 0, f, 256, f, 2, None) == 2  # unknown format
    assert L.fp8_quant_rowwise_fmt(f, 1, 4, 256, 256, 128, 1, 2, f, 256, f, 2, None) == 2  # unknown rule
    assert L.fp8_quant_rowwise_fmt(f, 1, 4, 200, 256, 128, 1, 1, f, 256, f, 2, None) == 1  # cols % group
    assert L.fp8_dequant_fmt(f, f, 0, 3, 4, 256, f, 0, None) == 2
    assert L.fgb_fp8_encode(f, 16, 5, f, None) == 2
    assert L.fp8_direct_transpose_fmt(f, f, 1, 200, 256, f, f, None) == 1
    assert L.fp8_direct_transpose_fmt(f, f, 4, 256, 256, f, f, None) == 2
    assert L.mx2_quant_rule(f, 4, 1024, 512, 3, f, f, f, None) == 2
    gf = lambda af=1, bf=0, ag=0, bg=2, l1=None: L.fp8_block_gemm_fmt(f, f, ag, af, f, f, bg, bf, l1, 0, 256, 256,
                                                                     512, 512, 512, f, 1, 256, 0, 0, None)
    assert gf(af=2) == 2 and gf(bf=1) == 2   # A E4M3/E5M2 only, B E4M3 only
    assert gf(ag=1, bg=1) == 2               # E5M2 A needs 1x128 scales
    assert gf(l1=f) == 2                     # no level-1 factor with E5M2
    gm = lambda G=4, Mm=256, K=512, m=f: L.fp8_grouped_gemm_masked(f, f, f, f, m, G, Mm, 256, K, f, 1, 0, None)
    assert gm(G=0) == 1 and gm(Mm=0) == 1 and gm(K=500) == 1 and gm(m=None) == 1
    assert L.fp8_quant_blockwise_t(f, 0, 2, 256, 256, f, f, f, f, None) == 2   # bf16 only
    assert L.fp8_quant_blockwise_t(f, 1, 2, 200, 256, f, f, f, f, None) == 1   # rows % 128
    assert L.fp8_quant_blockwise_t(f, 1, 0, 256, 256, f, f, f, f, None) == 1   # G >= 1
    # three-pass baseline: shape and workspace checks
    assert fgb.fp8_naive_transpose_workspace_size(256, 384) == 4 * 256 * 384
    assert L.fp8_naive_transpose(f, f, 200, 256, f, f, f, 1 << 20, None) == 1
    assert L.fp8_naive_transpose(f, f, 256, 256, f, f, f, 1000, None) == 3
    assert L.fp8_naive_transpose(f, f, 256, 256, f, f, None, 1 << 20, None) == 3
    ws = fgb.permute_pad_workspace_size(16384, 8, 32)
    assert ws > 0
    # M_cap below the host-side bound
    assert L.permute_pad(f, f, f, 100, 8, 32, 7168, 16, f, f, f, f, 800, f, ws, None) == 1
    # workspace too small
    assert L.permute_pad(f, f, f, 100, 8, 32, 7168, 16, f, f, f, f, 800 + 15 * 32, f, 4, None) == 3
    assert L.unpermute_unpad(f, f, None, 10, 8, 7, f, None) == 1
    assert fgb.unpermute_backward_workspace_size(1000) == 4000
    assert L.unpermute_backward(f, f, None, 10, 8, 7, 200, f, f, 4096, None) == 1  # H % 8
    assert L.unpermute_backward(f, f, None, 10, 8, 128, 200, f, f, 16, None) == 3  # workspace
    assert L.swiglu_quant(f, 10, 100, 200, None, 0, f, f, None) == 1
    assert L.dswiglu_quant(f, f, f, 10, 100, None, 0, f, f, None) == 1
    assert L.dswiglu_quant(f, f, _fake(0x1008), 10, 128, None, 0, f, f, None) == 1  # da not 16-byte aligned
    assert L.dswiglu_quant(f, f, f, 10, 128, f, 0, f, f, None) == 1  # offsets without G
    assert L.mx2_quant(f, 4, 64, 48, f, f, f, None) == 2
    assert L.mx2_quant(f, 4, 48, 64, f, f, f, None) == 1
    assert L.swiglu_f32(f, f, -1, f, None) == 1
    assert L.swiglu_f32(f, None, 5, f, None) == 1
    assert L.swiglu_f32(None, None, 0, None, None) == 0  # nothing to do
    assert L.dswiglu_f32(f, f, f, 5, f, None, None) == 1


def test_oracle_and_library_share_nothing():
    """The oracle never includes or loads the HIP library, and the library never
    includes, imports or loads the oracle."""
    osrc = open(os.path.join(ROOT, "oracle", "fgb_oracle.c")).read()
    includes = re.findall(r"#include\s*[<\"]([^>\"]+)", osrc)
    assert all(not (i.startswith("hip") or "fgb" in i) for i in includes), includes
    for fn in os.listdir(os.path.join(ROOT, "oracle")):
        if fn.endswith(".py"):
            txt = open(os.path.join(ROOT, "oracle", fn)).read()
            assert "fine_grained_blockwise_amd" not in txt and "libfgb" not in txt
    pkg = os.path.join(ROOT, "fine_grained_blockwise_amd")
    for dp, _, fns in os.walk(pkg):
        for fn in fns:
            if fn.endswith((".py", ".hip", ".h")):
                txt = open(os.path.join(dp, fn)).read()
                assert not re.search(r"import\s+oracle|from\s+oracle|liboracle|fgb_oracle", txt), fn


def test_permute_pad_noalloc_rejects_sizes_beyond_its_scratch():
    import fine_grained_blockwise_amd as fgb
    L = fgb.lib()
    f = _fake()
    T, topk, G = 1 << 20, 8, 1024
    need = L.permute_pad_workspace_size(T, topk, G)
    assert need > fgb.PERMUTE_PAD_NOALLOC_SCRATCH_BYTES
    assert L.permute_pad_noalloc(f, f, f, T, topk, G, 7168, 16, f, f, f, f, T * topk + 15 * G, None) == 3
    assert b"scratch" in L.fgb_last_error()
    # the largest size it takes at G = 32: 2*ceil(T/256)*32 + 32 words fit in 1 MiB
    T = 4095 * 256
    assert L.permute_pad_workspace_size(T, topk, 32) <= fgb.PERMUTE_PAD_NOALLOC_SCRATCH_BYTES
    assert L.permute_pad_workspace_size(T + 256, topk, 32) > fgb.PERMUTE_PAD_NOALLOC_SCRATCH_BYTES
    # argument errors come first, as for permute_pad
    assert L.permute_pad_noalloc(None, f, f, 16, topk, 32, 7168, 16, f, f, f, f, 16 * topk + 15 * 32, None) == 1


def test_hbm_probe_validation():
    import fine_grained_blockwise_amd as fgb
    L = fgb.lib()
    f = _fake()
    assert L.fgb_hbm_probe(f, f, 256, 256, 9, None) == 2             # unknown pattern
    assert L.fgb_hbm_probe(None, f, 256, 256, fgb.PROBE_COPY, None) == 1
    assert b"null" in L.fgb_last_error()
    assert L.fgb_hbm_probe(f, f, 200, 256, fgb.PROBE_STRIDED_READ, None) == 1  # rows % 128
    assert L.fgb_hbm_probe(f, _fake(0x1008), 256, 256, fgb.PROBE_COPY, None) == 1  # alignment
    assert L.fgb_hbm_probe(f, f, 0, 256, fgb.PROBE_COPY, None) == 0  # empty: touches nothing
