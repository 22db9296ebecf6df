// transpose.hip -- scaling-aware direct transpose of row-wise FP8.
//
// awesome-system-papers, "FP8-Flow-MoE: A Casting-Free FP8 Recipe without
// Double Quantization Error", "Core method" and key observation 2: with
// power-of-two scales, converting row-wise (1x128) FP8 into column-wise FP8
// needs only, inside each 128x128 block, the block's largest scale Smax and an
// exponent shift of every code by k = log2(Smax / S_row), recombining the
// mantissa when the result leaves the normal range.  The result equals
// requantizing the dequantized block at Smax -- without a dequantize /
// requantize pass.
//
// gfx950 mapping: one wave per 128x128 block.  Lane (tsub = lane & 7,
// csub = lane >> 3) owns the 16x16 byte sub-tile at rows tsub*16.., columns
// csub*16..: 16 row loads of 16 bytes (8 lanes cover one 128-byte row
// segment), the shift applied in the row domain where k is uniform per row,
// a 16x16 byte transpose in registers with v_perm_b32, and 16 column stores of
// 16 bytes (8 lanes cover one 128-byte output row segment).  The four waves
// of a workgroup take four consecutive row blocks of one column block, so
// each output row gets 512 contiguous bytes at once (measured: 5.0 TB/s on
// [131584, 7168] against 3.5-4.0 TB/s with four column blocks per
// workgroup, whose writes land in four separate 128-byte pieces per row).
// No LDS, no bank conflicts; HBM-bound.
//
// The shift decodes two codes to fp32 (exact), multiplies by 2^-k (exact) and
// converts back with round-to-nearest-even; for E - k >= 1 that is the plain
// exponent decrement, below it the subnormal re-rounding.
#include "fgb_internal.h"

namespace fgb {

// 4x4 byte transpose: rows a,b,c,d (byte i = column i) -> columns.
__device__ __forceinline__ void tr4x4(uint32_t a, uint32_t b, uint32_t c, uint32_t d, uint32_t &o0,
                                      uint32_t &o1, uint32_t &o2, uint32_t &o3)
{
    uint32_t ab_lo = __builtin_amdgcn_perm(b, a, 0x05010400u); // a0 b0 a1 b1
    uint32_t ab_hi = __builtin_amdgcn_perm(b, a, 0x07030602u); // a2 b2 a3 b3
    uint32_t cd_lo = __builtin_amdgcn_perm(d, c, 0x05010400u); // c0 d0 c1 d1
    uint32_t cd_hi = __builtin_amdgcn_perm(d, c, 0x07030602u); // c2 d2 c3 d3
    o0 = __builtin_amdgcn_perm(cd_lo, ab_lo, 0x05040100u);     // a0 b0 c0 d0
    o1 = __builtin_amdgcn_perm(cd_lo, ab_lo, 0x07060302u);     // a1 b1 c1 d1
    o2 = __builtin_amdgcn_perm(cd_hi, ab_hi, 0x05040100u);     // a2 b2 c2 d2
    o3 = __builtin_amdgcn_perm(cd_hi, ab_hi, 0x07060302u);     // a3 b3 c3 d3
}

template <int FMT = FMT_E4M3>
__device__ __forceinline__ uint32_t shift_word(uint32_t w, float f)
{
    if constexpr (FMT == FMT_E5M2) {
        float2 a = dec2_lo_e5m2(w), b = dec2_hi_e5m2(w);
        return cvt4_e5m2(a.x * f, a.y * f, b.x * f, b.y * f);
    } else {
        float2 a = dec2_lo(w), b = dec2_hi(w);
        return cvt4_e4m3(a.x * f, a.y * f, b.x * f, b.y * f);
    }
}

// FMT: element format of the codes (the shift is the same exponent move).
template <bool ROWSCALE, int FMT = FMT_E4M3>
__global__ __launch_bounds__(256) void direct_transpose_kernel(const uint8_t *__restrict__ q,
                                                               const uint8_t *__restrict__ s,
                                                               int64_t T, int64_t C,
                                                               uint8_t *__restrict__ qt,
                                                               uint8_t *__restrict__ st,
                                                               int64_t nblocks)
{
    const int lane = lane_id();
    const int64_t blk = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    if (blk >= nblocks)
        return;
    // consecutive waves take consecutive row blocks of one column block, so
    // each output row receives long runs from one workgroup
    const int64_t ncb = C / 128, ntb = T / 128;
    const int64_t tb = blk % ntb, cb = blk / ntb;
    { // matrix blockIdx.y of a dense batch
        const int64_t e = blockIdx.y;
        q += e * T * C;
        qt += e * T * C;
        s += e * (ROWSCALE ? T * ncb : ntb * ncb);
        st += e * (ROWSCALE ? C * ntb : ntb * ncb);
    }
    const int tsub = lane & 7, csub = lane >> 3;
    const int64_t t0 = tb * 128 + tsub * 16;
    const int64_t c0 = cb * 128 + csub * 16;

    uint32_t w[16][4];
#pragma unroll
    for (int j = 0; j < 16; j++) {
        uint4 v = ld_stream16(q + (t0 + j) * C + c0);
        w[j][0] = v.x;
        w[j][1] = v.y;
        w[j][2] = v.z;
        w[j][3] = v.w;
    }
    int emax = 0;
    if constexpr (ROWSCALE) {
        int e[16];
        uint32_t m = 0;
#pragma unroll
        for (int j = 0; j < 16; j++) {
            e[j] = s[(t0 + j) * ncb + cb];
            m = max(m, (uint32_t)e[j]);
        }
        emax = (int)group_max_u32<8>(m); // lanes with equal csub hold all 128 rows
#pragma unroll
        for (int j = 0; j < 16; j++) {
            int k = min(emax - e[j], 64); // E5M2 codes survive shifts up to 32, E4M3 up to 17
            float f = pow2f(-k);
#pragma unroll
            for (int x = 0; x < 4; x++)
                w[j][x] = shift_word<FMT>(w[j][x], f);
        }
    }
    uint32_t o[16][4]; // o[c][i]: column c0+c, rows t0+4i .. t0+4i+3
#pragma unroll
    for (int i = 0; i < 4; i++)
#pragma unroll
        for (int x = 0; x < 4; x++)
            tr4x4(w[4 * i + 0][x], w[4 * i + 1][x], w[4 * i + 2][x], w[4 * i + 3][x], o[4 * x + 0][i],
                  o[4 * x + 1][i], o[4 * x + 2][i], o[4 * x + 3][i]);
#pragma unroll
    for (int c = 0; c < 16; c++)
        st_stream16(qt + (c0 + c) * T + t0, make_uint4(o[c][0], o[c][1], o[c][2], o[c][3]));
    if constexpr (ROWSCALE) {
        st[(cb * 128 + lane) * ntb + tb] = (uint8_t)emax;
        st[(cb * 128 + 64 + lane) * ntb + tb] = (uint8_t)emax;
    } else {
        if (lane == 0)
            st[cb * ntb + tb] = s[tb * ncb + cb];
    }
}

// ---- expert segments, for the expert backward's Wgrad --------------------------
// koff[e+1] = koff[e] + ceil(len_e / 128) * 128 (one thread; G <= 1024).
__global__ void koff_kernel(const int32_t *__restrict__ off, int G, int32_t *__restrict__ koff)
{
    if (threadIdx.x == 0 && blockIdx.x == 0) {
        int32_t k = 0;
        koff[0] = 0;
        for (int e = 0; e < G; e++) {
            k += ((off[e + 1] - off[e] + 127) / 128) * 128;
            koff[e + 1] = k;
        }
    }
}

// Direct transpose of expert segments: one wave per 128x128 output block
// (column block kb of the transposed copy, row block cb of C), as in
// direct_transpose_kernel, except that the block's source rows are the
// segment's rows present (the last block of a segment may be short: its
// absent rows count as code 0 and take no part in the block maximum).
__global__ __launch_bounds__(256) void grouped_direct_transpose_kernel(
    const uint8_t *__restrict__ q, const uint8_t *__restrict__ s, int64_t C, const int32_t *__restrict__ off,
    const int32_t *__restrict__ koff, int G, uint8_t *__restrict__ qt, uint8_t *__restrict__ st, int64_t Kc,
    int64_t nslots)
{
    const int lane = lane_id();
    const int64_t slot = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    if (slot >= nslots)
        return;
    const int64_t ncb = C / 128, nkb = Kc / 128;
    const int64_t kb = slot / ncb, cb = slot % ncb; // (K-block-major measured faster here)
    int ex = -1;
    for (int g = 0; g < G; g++)
        if (kb * 128 >= koff[g] && kb * 128 < koff[g + 1])
            ex = g;
    if (ex < 0)
        return; // past the last segment (uniform per wave)
    const int64_t r0 = off[ex] + (kb * 128 - koff[ex]);
    const int64_t n = min((int64_t)128, (int64_t)off[ex + 1] - r0);
    const int tsub = lane & 7, csub = lane >> 3;
    const int tl = tsub * 16;
    const int64_t c0 = cb * 128 + csub * 16;

    uint32_t w[16][4];
    int e[16];
    uint32_t m = 0;
    // absent rows (past a short last block) re-read the block's first row
    // and are zeroed after the load: no branches around the loads
#pragma unroll
    for (int j = 0; j < 16; j++) {
        const bool present = tl + j < n;
        const int64_t row = r0 + (present ? tl + j : 0);
        const uint4 v = ld_stream16(q + row * C + c0);
        const int ej = s[row * ncb + cb];
        w[j][0] = present ? v.x : 0u;
        w[j][1] = present ? v.y : 0u;
        w[j][2] = present ? v.z : 0u;
        w[j][3] = present ? v.w : 0u;
        e[j] = present ? ej : 0;
        m = max(m, (uint32_t)e[j]);
    }
    const int emax = (int)group_max_u32<8>(m);
#pragma unroll
    for (int j = 0; j < 16; j++) {
        const int k = min(emax - e[j], 31);
        const float f = pow2f(-k);
#pragma unroll
        for (int x = 0; x < 4; x++)
            w[j][x] = shift_word(w[j][x], f);
    }
    uint32_t o[16][4];
#pragma unroll
    for (int i = 0; i < 4; i++)
#pragma unroll
        for (int x = 0; x < 4; x++)
            tr4x4(w[4 * i + 0][x], w[4 * i + 1][x], w[4 * i + 2][x], w[4 * i + 3][x], o[4 * x + 0][i],
                  o[4 * x + 1][i], o[4 * x + 2][i], o[4 * x + 3][i]);
#pragma unroll
    for (int c = 0; c < 16; c++)
        st_stream16(qt + (c0 + c) * Kc + kb * 128 + tl, make_uint4(o[c][0], o[c][1], o[c][2], o[c][3]));
    st[(cb * 128 + lane) * nkb + kb] = (uint8_t)emax;
    st[(cb * 128 + 64 + lane) * nkb + kb] = (uint8_t)emax;
}

// ---- three-pass baseline ------------------------------------------------------
// The conversion the direct transpose replaces (FP8-Flow-MoE "Core method",
// Fig. 1): dequantize to bf16, transpose, requantize 1x128.  The middle pass
// is this 2-byte transpose: one wave per 64x64 tile; lane (rg = lane / 8,
// cg = lane % 8) loads rows rg*8.. of columns cg*8.. (8 lanes cover one
// 128-byte row segment), swaps 16-bit halves across row pairs with v_perm_b32,
// and stores 8 output rows of 16 bytes (8 lanes cover one 128-byte segment).
__global__ __launch_bounds__(256) void transpose16_kernel(const uint16_t *__restrict__ x, int64_t R,
                                                          int64_t C, uint16_t *__restrict__ xt,
                                                          int64_t ntc, int64_t ntiles)
{
    const int lane = lane_id();
    const int64_t tile = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    if (tile >= ntiles)
        return;
    const int64_t r0 = (tile / ntc) * 64 + (lane >> 3) * 8, c0 = (tile % ntc) * 64 + (lane & 7) * 8;
    uint32_t w[8][4];
#pragma unroll
    for (int j = 0; j < 8; j++) {
        const uint4 v = ld_stream16(x + (r0 + j) * C + c0);
        w[j][0] = v.x;
        w[j][1] = v.y;
        w[j][2] = v.z;
        w[j][3] = v.w;
    }
    // output row c0+i, dword m = input rows r0+2m (low half), r0+2m+1 (high half)
#pragma unroll
    for (int i = 0; i < 8; i++) {
        const uint32_t sel = (i & 1) ? 0x07060302u : 0x05040100u;
        uint32_t o[4];
#pragma unroll
        for (int m = 0; m < 4; m++)
            o[m] = __builtin_amdgcn_perm(w[2 * m + 1][i >> 1], w[2 * m][i >> 1], sel);
        st_stream16(xt + (c0 + i) * R + r0, make_uint4(o[0], o[1], o[2], o[3]));
    }
}

} // namespace fgb

using namespace fgb;

extern "C" int fp8_direct_transpose(const uint8_t *q, const uint8_t *s, int s_gran, int64_t rows,
                                    int64_t cols, uint8_t *qt, uint8_t *st, void *stream)
{
    clear_error();
    FGB_REQUIRE(q && s && qt && st, FGB_EINVAL, "fp8_direct_transpose: null pointer");
    FGB_REQUIRE(s_gran == FGB_ROW1x128 || s_gran == FGB_BLOCK128, FGB_EUNSUPPORTED,
                "fp8_direct_transpose: s_gran must be FGB_ROW1x128 or FGB_BLOCK128");
    FGB_REQUIRE(rows >= 0 && cols >= 0 && rows % 128 == 0 && cols % 128 == 0, FGB_EINVAL,
                "fp8_direct_transpose: rows and cols must be multiples of 128 (rows=%lld cols=%lld)",
                (long long)rows, (long long)cols);
    FGB_REQUIRE(aligned16(q) && aligned16(qt), FGB_EINVAL,
                "fp8_direct_transpose: q and qt must be 16-byte aligned");
    int64_t nb = (rows / 128) * (cols / 128);
    if (nb == 0)
        return FGB_OK;
    int64_t grid = (nb + 3) / 4;
    FGB_REQUIRE(grid < (1ll << 31), FGB_EINVAL, "fp8_direct_transpose: too many blocks");
    hipStream_t stm = (hipStream_t)stream;
    if (s_gran == FGB_ROW1x128)
        direct_transpose_kernel<true><<<(int)grid, 256, 0, stm>>>(q, s, rows, cols, qt, st, nb);
    else
        direct_transpose_kernel<false><<<(int)grid, 256, 0, stm>>>(q, s, rows, cols, qt, st, nb);
    FGB_LAUNCHED("fp8_direct_transpose");
    return FGB_OK;
}

extern "C" int fp8_direct_transpose_fmt(const uint8_t *q, const uint8_t *s, int fmt, int64_t rows, int64_t cols,
                                        uint8_t *qt, uint8_t *st, void *stream)
{
    clear_error();
    FGB_REQUIRE(fmt == FGB_E4M3 || fmt == FGB_E5M2, FGB_EUNSUPPORTED,
                "fp8_direct_transpose_fmt: fmt must be FGB_E4M3 or FGB_E5M2");
    if (fmt == FGB_E4M3)
        return fp8_direct_transpose(q, s, FGB_ROW1x128, rows, cols, qt, st, stream);
    FGB_REQUIRE(q && s && qt && st, FGB_EINVAL, "fp8_direct_transpose_fmt: null pointer");
    FGB_REQUIRE(rows >= 0 && cols >= 0 && rows % 128 == 0 && cols % 128 == 0, FGB_EINVAL,
                "fp8_direct_transpose_fmt: rows and cols must be multiples of 128 (rows=%lld cols=%lld)",
                (long long)rows, (long long)cols);
    FGB_REQUIRE(aligned16(q) && aligned16(qt), FGB_EINVAL,
                "fp8_direct_transpose_fmt: q and qt must be 16-byte aligned");
    int64_t nb = (rows / 128) * (cols / 128);
    if (nb == 0)
        return FGB_OK;
    int64_t grid = (nb + 3) / 4;
    FGB_REQUIRE(grid < (1ll << 31), FGB_EINVAL, "fp8_direct_transpose_fmt: too many blocks");
    direct_transpose_kernel<true, FMT_E5M2><<<(int)grid, 256, 0, (hipStream_t)stream>>>(q, s, rows, cols, qt, st, nb);
    FGB_LAUNCHED("fp8_direct_transpose_fmt");
    return FGB_OK;
}

extern "C" size_t fp8_naive_transpose_workspace_size(int64_t rows, int64_t cols)
{
    return rows > 0 && cols > 0 ? (size_t)(4 * rows * cols) : 0;
}

extern "C" int fp8_naive_transpose(const uint8_t *q, const uint8_t *s, int64_t rows, int64_t cols,
                                   uint8_t *qt, uint8_t *st, void *workspace, size_t ws_bytes,
                                   void *stream)
{
    clear_error();
    FGB_REQUIRE(q && s && qt && st, FGB_EINVAL, "fp8_naive_transpose: null pointer");
    FGB_REQUIRE(rows >= 0 && cols >= 0 && rows % 128 == 0 && cols % 128 == 0, FGB_EINVAL,
                "fp8_naive_transpose: rows and cols must be multiples of 128 (rows=%lld cols=%lld)",
                (long long)rows, (long long)cols);
    FGB_REQUIRE(aligned16(q) && aligned16(qt), FGB_EINVAL,
                "fp8_naive_transpose: q and qt must be 16-byte aligned");
    if (rows == 0 || cols == 0)
        return FGB_OK;
    const size_t need = fp8_naive_transpose_workspace_size(rows, cols);
    FGB_REQUIRE(workspace && ws_bytes >= need && aligned16(workspace), FGB_EWORKSPACE,
                "fp8_naive_transpose: workspace must be 16-byte aligned and >= %zu bytes", need);
    uint16_t *x = (uint16_t *)workspace, *xt = x + rows * cols;
    // pass 1: dequantize to bf16 (exact for power-of-two scales)
    int rc = fp8_dequant(q, s, FGB_ROW1x128, rows, cols, x, FGB_BF16, stream);
    if (rc != FGB_OK)
        return rc;
    // pass 2: transpose
    const int64_t ntc = cols / 64, ntiles = (rows / 64) * ntc;
    transpose16_kernel<<<(unsigned)((ntiles + 3) / 4), 256, 0, (hipStream_t)stream>>>(x, rows, cols, xt, ntc, ntiles);
    FGB_LAUNCHED("fp8_naive_transpose");
    // pass 3: requantize the rows of the transposed copy
    return fp8_quant_rowwise(xt, FGB_BF16, cols, rows, rows, 128, qt, rows, st, rows / 128, stream);
}

extern "C" int fp8_block_transpose_batched(const uint8_t *q, const uint8_t *s, int G, int64_t rows, int64_t cols,
                                           uint8_t *qt, uint8_t *st, void *stream)
{
    clear_error();
    FGB_REQUIRE(q && s && qt && st, FGB_EINVAL, "fp8_block_transpose_batched: null pointer");
    FGB_REQUIRE(G >= 1 && G <= 65535, FGB_EINVAL, "fp8_block_transpose_batched: G must be in [1, 65535]");
    FGB_REQUIRE(rows >= 0 && cols >= 0 && rows % 128 == 0 && cols % 128 == 0, FGB_EINVAL,
                "fp8_block_transpose_batched: rows and cols must be multiples of 128");
    FGB_REQUIRE(aligned16(q) && aligned16(qt), FGB_EINVAL, "fp8_block_transpose_batched: q and qt must be 16-byte aligned");
    const int64_t nb = (rows / 128) * (cols / 128);
    if (nb == 0)
        return FGB_OK;
    const dim3 grid((unsigned)((nb + 3) / 4), (unsigned)G);
    direct_transpose_kernel<false><<<grid, 256, 0, (hipStream_t)stream>>>(q, s, rows, cols, qt, st, nb);
    FGB_LAUNCHED("fp8_block_transpose_batched");
    return FGB_OK;
}

extern "C" int fp8_grouped_direct_transpose(const uint8_t *q, const uint8_t *s, int64_t M_cap, int64_t cols,
                                            const int32_t *group_offsets, int G, uint8_t *qt, uint8_t *st,
                                            int64_t K_cap, int32_t *k_offsets, void *stream)
{
    clear_error();
    FGB_REQUIRE(q && s && qt && st && group_offsets && k_offsets, FGB_EINVAL,
                "fp8_grouped_direct_transpose: null pointer");
    FGB_REQUIRE(G >= 1 && G <= 1024, FGB_EINVAL, "fp8_grouped_direct_transpose: G must be in [1, 1024]");
    FGB_REQUIRE(M_cap >= 0 && cols > 0 && cols % 128 == 0 && K_cap % 128 == 0, FGB_EINVAL,
                "fp8_grouped_direct_transpose: cols and K_cap must be multiples of 128");
    FGB_REQUIRE(K_cap >= ((M_cap + 127 * (int64_t)G + 127) / 128) * 128, FGB_EINVAL,
                "fp8_grouped_direct_transpose: K_cap must be >= M_cap + 127*G rounded up to 128");
    FGB_REQUIRE(aligned16(q) && aligned16(qt), FGB_EINVAL, "fp8_grouped_direct_transpose: q and qt must be 16-byte aligned");
    hipStream_t stm = (hipStream_t)stream;
    koff_kernel<<<1, 64, 0, stm>>>(group_offsets, G, k_offsets);
    FGB_LAUNCHED("fp8_grouped_direct_transpose");
    const int64_t nslots = (K_cap / 128) * (cols / 128);
    if (nslots == 0)
        return FGB_OK;
    grouped_direct_transpose_kernel<<<(unsigned)((nslots + 3) / 4), 256, 0, stm>>>(q, s, cols, group_offsets,
                                                                                   k_offsets, G, qt, st, K_cap, nslots);
    FGB_LAUNCHED("fp8_grouped_direct_transpose");
    return FGB_OK;
}
