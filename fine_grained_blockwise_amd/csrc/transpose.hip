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
// and a 16x16 byte transpose in registers with v_perm_b32.  A workgroup of
// eight waves takes eight consecutive row blocks of one column block and
// stages their transposed blocks in LDS, so that every output row is written
// as one 1 KB run (the staging is described below).  HBM-bound.
//
// The shift decodes two codes to fp32 (exact), multiplies by 2^-k (exact) and
// converts back with round-to-nearest-even; for E - k >= 1 that is the plain
// exponent decrement, below it the subnormal re-rounding.
#include <atomic>

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

// The four codes of w times f = 2^-k, re-encoded with round-to-nearest-even.
// The decode takes the power of two as its scale operand (gfx950's scaled
// conversion multiplies the decoded value by 2^(exponent field of f - 127)):
// one instruction per two codes, and exact, since every decoded code times
// 2^-k for k <= 64 is a normal fp32.
typedef float fgb_v2f __attribute__((ext_vector_type(2)));
template <int FMT = FMT_E4M3>
__device__ __forceinline__ uint32_t shift_word(uint32_t w, float f)
{
    if constexpr (FMT == FMT_E5M2) {
        const fgb_v2f a = __builtin_amdgcn_cvt_scalef32_pk_f32_bf8((int)w, f, false);
        const fgb_v2f b = __builtin_amdgcn_cvt_scalef32_pk_f32_bf8((int)w, f, true);
        return cvt4_e5m2(a.x, a.y, b.x, b.y);
    } else {
        const fgb_v2f a = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8((int)w, f, false);
        const fgb_v2f b = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8((int)w, f, true);
        return cvt4_e4m3(a.x, a.y, b.x, b.y);
    }
}

// Transposed 16x16 byte sub-tile: w[j][x] holds row j, bytes 4x..4x+3 of the
// lane's sub-tile; o[c][i] receives column c, rows 4i..4i+3.
__device__ __forceinline__ void transpose16x16(const uint32_t (&w)[16][4], uint32_t (&o)[16][4])
{
#pragma unroll
    for (int i = 0; i < 4; i++)
#pragma unroll
        for (int x = 0; x < 4; x++)
            tr4x4(w[4 * i + 0][x], w[4 * i + 1][x], w[4 * i + 2][x], w[4 * i + 3][x], o[4 * x + 0][i],
                  o[4 * x + 1][i], o[4 * x + 2][i], o[4 * x + 3][i]);
}

// The 128 row scales of a block: lane l loads those of rows l and l + 64
// (the rows present: n of them, absent rows count as 0), the wave maximum is
// the block's e_max, and each lane reads back the 16 scales of its rows
// tsub*16 .. tsub*16 + 15 (e[j], row tsub*16 + j) through the wave's 128-byte
// LDS slot -- two loads per lane instead of sixteen: 2-3% on the expert
// segments; measured slower in the staged dense kernel (97 against 94 us on
// [32768, 7168]), which keeps the sixteen.  col = the scale of the block's
// first row; ld = the scale row stride.
__device__ __forceinline__ int block_row_scales(const uint8_t *col, int64_t ld, int n, uint8_t *slot, int lane,
                                                int tsub, int (&e)[16])
{
    const uint32_t a = lane < n ? col[lane * ld] : 0u;
    const uint32_t b = lane + 64 < n ? col[(lane + 64) * ld] : 0u;
    slot[lane] = (uint8_t)a;
    slot[lane + 64] = (uint8_t)b;
    __builtin_amdgcn_wave_barrier(); // the wave's LDS accesses complete in order
    const uint4 v = *reinterpret_cast<const uint4 *>(slot + tsub * 16);
    const uint32_t words[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int j = 0; j < 16; j++)
        e[j] = (int)((words[j / 4] >> (8 * (j % 4))) & 0xFFu);
    return (int)group_max_u32<64>(max(a, b));
}

// ---- LDS staging of TB transposed blocks ----------------------------------------
// A workgroup of TB waves takes TB consecutive 128-row blocks (rows of the
// source, columns of the transposed copy) of one 128-column block.  Each wave
// transposes its block in registers and writes it into an LDS tile of 128
// output rows x TB*128 bytes; the workgroup then stores every output row as
// one run of TB*128 contiguous bytes (1 KB at TB = 8).  Measured on the
// MI355X against one wave per block with 512-byte runs per output row
// (four waves): +5% on [32768, 7168] and [32768, 2048] with the Infinity
// Cache flushed, +10% on [8192, 7168].
// Tile row r keeps its 16-byte chunk ch at position ch ^ (((r >> 4) & 1) << 3):
// the 16 lanes of a quarter-wave write rows r and r + 16 at the same chunk
// index, which the swizzle moves to the other half of the 64 banks, and the
// store phase reads 16 consecutive chunks of one row, a permutation within
// an aligned group of 16 -- both free of bank conflicts.
template <int TB> struct Stage {
    static constexpr int RS = TB * 128; // bytes per tile row
    static constexpr int CPR = TB * 8;  // 16-byte chunks per tile row
    static constexpr int TILE = 128 * RS;
    static constexpr int LDS = TILE + 64; // + the per-wave scale bytes
    static_assert(TB >= 2, "the swizzle needs at least 16 chunks per row");
    __device__ static int at(int r, int ch) { return r * RS + 16 * (ch ^ (((r >> 4) & 1) << 3)); }
};

// The lane's 16 columns x 16 bytes of wave `w`'s block into the tile.
template <int TB>
__device__ __forceinline__ void stage_put(uint8_t *lds, int w, int tsub, int csub, const uint32_t (&o)[16][4])
{
#pragma unroll
    for (int c = 0; c < 16; c++)
        *reinterpret_cast<uint4 *>(lds + Stage<TB>::at(csub * 16 + c, w * 8 + tsub)) =
            make_uint4(o[c][0], o[c][1], o[c][2], o[c][3]);
}

// Store the tile: output row r goes to out + r * ld_out, chunks of blocks
// [0, nvalid) only (a last group may hold fewer than TB blocks).
template <int TB>
__device__ __forceinline__ void stage_store(const uint8_t *lds, uint8_t *out, int64_t ld_out, int nvalid)
{
    constexpr int NTH = TB * 64, NCH = 128 * Stage<TB>::CPR;
#pragma unroll
    for (int k = 0; k < NCH / NTH; k++) {
        const int idx = (int)threadIdx.x + k * NTH;
        const int r = idx / Stage<TB>::CPR, ch = idx % Stage<TB>::CPR;
        if (ch / 8 < nvalid)
            st_stream16(out + r * ld_out + ch * 16, *reinterpret_cast<const uint4 *>(lds + Stage<TB>::at(r, ch)));
    }
}

// The TB scale bytes of output row r (blocks [0, nvalid)) at dst: one 8-, 4-
// or 2-byte store when the group is whole and dst aligned, else bytes.
template <int TB>
__device__ __forceinline__ void store_scale_run(uint8_t *dst, const uint8_t *esc, int nvalid)
{
    if (nvalid == TB && ((uintptr_t)dst % TB) == 0) {
        uint32_t v[2] = {0u, 0u};
#pragma unroll
        for (int b = 0; b < TB; b++)
            v[b / 4] |= (uint32_t)esc[b] << (8 * (b % 4));
        if constexpr (TB == 8)
            *reinterpret_cast<uint2 *>(dst) = make_uint2(v[0], v[1]);
        else if constexpr (TB == 4)
            *reinterpret_cast<uint32_t *>(dst) = v[0];
        else
            *reinterpret_cast<uint16_t *>(dst) = (uint16_t)v[0];
    } else {
        for (int b = 0; b < nvalid; b++)
            dst[b] = esc[b];
    }
}

// Direct transpose of dense [T, C] codes.  Workgroup (tg, cb): row blocks
// tg*TB .. tg*TB + TB-1 (those below T/128) of column block cb; consecutive
// workgroups take consecutive row groups of one column block.
// ROWSCALE: 1x128 scales and the exponent shift; else 128x128 block scales,
// k = 0 (an exact byte transpose).  FMT: element format of the codes (the
// shift is the same exponent move).  blockIdx.y: matrix of a dense batch.
template <int TB, bool ROWSCALE, int FMT = FMT_E4M3>
__global__ __launch_bounds__(TB * 64) void direct_transpose_kernel(const uint8_t *__restrict__ q,
                                                                   const uint8_t *__restrict__ s, int64_t T,
                                                                   int64_t C, uint8_t *__restrict__ qt,
                                                                   uint8_t *__restrict__ st)
{
    extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
    uint8_t *esc = lds + Stage<TB>::TILE;
    const int lane = lane_id(), wave = threadIdx.x >> 6;
    const int64_t ncb = C / 128, ntb = T / 128;
    const int64_t ngt = (ntb + TB - 1) / TB;
    const int64_t tg = blockIdx.x % ngt, cb = blockIdx.x / ngt;
    const int nvalid = (int)min((int64_t)TB, ntb - tg * TB);
    {
        const int64_t e = blockIdx.y;
        q += e * T * C;
        qt += e * T * C;
        s += e * (ROWSCALE ? T * ncb : ntb * ncb);
        st += e * (ROWSCALE ? C * ntb : ntb * ncb);
    }
    const int tsub = lane & 7, csub = lane >> 3;
    if (wave < nvalid) { // uniform per wave
        const int64_t tb = tg * TB + wave;
        const int64_t t0 = tb * 128 + tsub * 16;
        const int64_t c0 = cb * 128 + csub * 16;
        uint32_t w[16][4];
#pragma unroll
        for (int j = 0; j < 16; j++) {
            const uint4 v = ld_stream16(q + (t0 + j) * C + c0);
            w[j][0] = v.x;
            w[j][1] = v.y;
            w[j][2] = v.z;
            w[j][3] = v.w;
        }
        int emax;
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
                const int k = min(emax - e[j], 64); // E5M2 codes survive shifts up to 32, E4M3 up to 17
                const float f = pow2f(-k);
#pragma unroll
                for (int x = 0; x < 4; x++)
                    w[j][x] = shift_word<FMT>(w[j][x], f);
            }
        } else {
            emax = s[tb * ncb + cb];
        }
        uint32_t o[16][4];
        transpose16x16(w, o);
        stage_put<TB>(lds, wave, tsub, csub, o);
        if (lane == 0)
            esc[wave] = (uint8_t)emax;
    }
    __syncthreads();
    stage_store<TB>(lds, qt + (cb * 128) * T + tg * TB * 128, T, nvalid);
    if constexpr (ROWSCALE) {
        if (threadIdx.x < 128)
            store_scale_run<TB>(st + (cb * 128 + threadIdx.x) * ntb + tg * TB, esc, nvalid);
    } else {
        if (threadIdx.x == 0)
            store_scale_run<TB>(st + cb * ntb + tg * TB, esc, nvalid);
    }
}

// The register-only form for small transposes (too few row-block groups to
// keep every CU busy with the staged form): one wave per 128x128 block, the
// four waves of a workgroup on consecutive row blocks of one column block (512
// contiguous bytes per output row), each lane storing its 16 columns directly.
// No LDS, so up to five workgroups share a CU.  ROWSCALE and FMT as in
// direct_transpose_kernel.
template <bool ROWSCALE, int FMT = FMT_E4M3>
__global__ __launch_bounds__(256) void direct_transpose_reg_kernel(const uint8_t *__restrict__ q,
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
    transpose16x16(w, o);
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
// koff[e+1] = koff[e] + ceil(len_e / 128) * 128 (G <= 1024): one wave, lane
// l taking expert g0 + l of each pass of 64, an inclusive wave prefix sum of
// the padded lengths plus the carry of the passes before.
__global__ __launch_bounds__(64) void koff_kernel(const int32_t *__restrict__ off, int G, int32_t *__restrict__ koff)
{
    const int lane = lane_id();
    int32_t carry = 0;
    if (lane == 0)
        koff[0] = 0;
    for (int g0 = 0; g0 < G; g0 += 64) {
        const int g = g0 + lane;
        int32_t v = g < G ? ((off[g + 1] - off[g] + 127) / 128) * 128 : 0;
#pragma unroll
        for (int d = 1; d < 64; d <<= 1) {
            const int32_t u = __shfl_up(v, d);
            v += lane >= d ? u : 0;
        }
        if (g < G)
            koff[g + 1] = carry + v;
        carry += __shfl(v, 63);
    }
}

// Direct transpose of expert segments: one wave per 128x128 output block
// (column block kb of the transposed copy, row block cb of C), the lane
// mapping of direct_transpose_kernel without the LDS staging, except that the
// block's source rows are the segment's rows present (the last block of a
// segment may be short: its absent rows count as code 0 and take no part in
// the block maximum).  The four waves of a workgroup take four consecutive
// column blocks of one output block, i.e. 512 contiguous bytes of each source
// row: measured faster here than staging eight output blocks through LDS
// (422 against 441 us on the MoE's [131376, 7168] segments, 130 against 135 us
// on [131376, 2048]; again with the present shift and scale gather: 400
// against 406 us and 118 against 126 us).
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
    // The segment holding K block kb: lane l of each pass reads expert g0 + l's
    // K range (one vector load instead of a dependent walk), a ballot names it.
    int ex = -1;
    for (int g0 = 0; g0 < G; g0 += 64) {
        const int g = g0 + lane;
        const int64_t k = kb * 128;
        const uint64_t hit = __ballot(g < G && k >= koff[g] && k < koff[g + 1]);
        if (hit) { // uniform
            ex = g0 + __builtin_ctzll(hit);
            break;
        }
    }
    if (ex < 0)
        return; // past the last segment (uniform per wave)
    const int64_t r0 = off[ex] + (kb * 128 - koff[ex]);
    const int64_t n = min((int64_t)128, (int64_t)off[ex + 1] - r0);
    const int tsub = lane & 7, csub = lane >> 3;
    const int tl = tsub * 16;
    const int64_t c0 = cb * 128 + csub * 16;

    __shared__ __attribute__((aligned(16))) uint8_t slots[4][128];
    uint32_t w[16][4];
    // absent rows (past a short last block) re-read the block's first row
    // and are zeroed after the load: no branches around the loads
#pragma unroll
    for (int j = 0; j < 16; j++) {
        const bool present = tl + j < n;
        const int64_t row = r0 + (present ? tl + j : 0);
        const uint4 v = ld_stream16(q + row * C + c0);
        w[j][0] = present ? v.x : 0u;
        w[j][1] = present ? v.y : 0u;
        w[j][2] = present ? v.z : 0u;
        w[j][3] = present ? v.w : 0u;
    }
    int e[16];
    const int emax = block_row_scales(s + r0 * ncb + cb, ncb, (int)n, slots[threadIdx.x >> 6], lane, tsub, e);
#pragma unroll
    for (int j = 0; j < 16; j++) {
        const int k = min(emax - e[j], 31);
        const float f = pow2f(-k);
#pragma unroll
        for (int x = 0; x < 4; x++)
            w[j][x] = shift_word(w[j][x], f);
    }
    uint32_t o[16][4];
    transpose16x16(w, o);
#pragma unroll
    for (int c = 0; c < 16; c++)
        st_stream16(qt + (c0 + c) * Kc + kb * 128 + tl, make_uint4(o[c][0], o[c][1], o[c][2], o[c][3]));
    st[(cb * 128 + lane) * nkb + kb] = (uint8_t)emax;
    st[(cb * 128 + 64 + lane) * nkb + kb] = (uint8_t)emax;
}

// The staged kernels use more than 64 KB of LDS at TB = 8: the limit is raised
// once per kernel (the template parameter: one flag table per kernel) and device.
template <auto KERN>
static int raise_lds_limit(int bytes, const char *name)
{
    static std::atomic<bool> done[64] = {}; // threads that launch at once may both set it: harmless
    const auto kern = KERN;
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess)
        dev = -1;
    const bool cached = dev >= 0 && dev < 64;
    if (!cached || !done[dev].load(std::memory_order_acquire)) {
        hipError_t e = hipFuncSetAttribute((const void *)kern, hipFuncAttributeMaxDynamicSharedMemorySize, bytes);
        if (e != hipSuccess)
            return set_error(FGB_EHIP, "%s: hipFuncSetAttribute failed: %s", name, hipGetErrorString(e));
        if (cached)
            done[dev].store(true, std::memory_order_release);
    }
    return FGB_OK;
}

template <int TB, bool ROWSCALE, int FMT>
static int launch_direct(const uint8_t *q, const uint8_t *s, int64_t T, int64_t C, uint8_t *qt, uint8_t *st,
                         int batch, hipStream_t stm, const char *name)
{
    auto kern = direct_transpose_kernel<TB, ROWSCALE, FMT>;
    int rc = raise_lds_limit<direct_transpose_kernel<TB, ROWSCALE, FMT>>(Stage<TB>::LDS, name);
    if (rc != FGB_OK)
        return rc;
    const int64_t ngt = (T / 128 + TB - 1) / TB;
    const int64_t grid = ngt * (C / 128);
    if (grid >= (1ll << 31))
        return set_error(FGB_EINVAL, "%s: too many blocks", name);
    kern<<<dim3((unsigned)grid, (unsigned)batch), TB * 64, Stage<TB>::LDS, stm>>>(q, s, T, C, qt, st);
    FGB_LAUNCHED(name);
    return FGB_OK;
}

// Eight row blocks per workgroup, staged through LDS, where that gives at
// least 384 workgroups (1.5 per CU; the 128 KB tile allows one workgroup per
// CU); else the register-only form.  Measured on the MI355X, cache flushed:
// staged 94.3 / 31.2 / 28.7 us against 97.5 / 32.7 / 31.2 us on [32768, 7168],
// [32768, 2048], [8192, 7168]; on [8192, 2048] (128 staged workgroups) and the
// [2048, 7168] weight, two- and four-block staging lost 4-19% to the
// register-only form.
template <bool ROWSCALE, int FMT = FMT_E4M3>
static int launch_direct_any(const uint8_t *q, const uint8_t *s, int64_t T, int64_t C, uint8_t *qt, uint8_t *st,
                             int batch, hipStream_t stm, const char *name)
{
    const int64_t ntb = T / 128, work = (C / 128) * batch;
    if ((ntb + 7) / 8 * work >= 384)
        return launch_direct<8, ROWSCALE, FMT>(q, s, T, C, qt, st, batch, stm, name);
    const int64_t nb = ntb * (C / 128);
    const int64_t grid = (nb + 3) / 4;
    if (grid >= (1ll << 31))
        return set_error(FGB_EINVAL, "%s: too many blocks", name);
    direct_transpose_reg_kernel<ROWSCALE, FMT><<<dim3((unsigned)grid, (unsigned)batch), 256, 0, stm>>>(
        q, s, T, C, qt, st, nb);
    FGB_LAUNCHED(name);
    return FGB_OK;
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
    if (rows == 0 || cols == 0)
        return FGB_OK;
    hipStream_t stm = (hipStream_t)stream;
    if (s_gran == FGB_ROW1x128)
        return launch_direct_any<true>(q, s, rows, cols, qt, st, 1, stm, "fp8_direct_transpose");
    return launch_direct_any<false>(q, s, rows, cols, qt, st, 1, stm, "fp8_direct_transpose");
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
    if (rows == 0 || cols == 0)
        return FGB_OK;
    return launch_direct_any<true, FMT_E5M2>(q, s, rows, cols, qt, st, 1, (hipStream_t)stream,
                                             "fp8_direct_transpose_fmt");
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
    if (rows == 0 || cols == 0)
        return FGB_OK;
    return launch_direct_any<false>(q, s, rows, cols, qt, st, G, (hipStream_t)stream, "fp8_block_transpose_batched");
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
    FGB_REQUIRE((nslots + 3) / 4 < (1ll << 31), FGB_EINVAL, "fp8_grouped_direct_transpose: too many blocks");
    grouped_direct_transpose_kernel<<<(unsigned)((nslots + 3) / 4), 256, 0, stm>>>(q, s, cols, group_offsets,
                                                                                   k_offsets, G, qt, st, K_cap, nslots);
    FGB_LAUNCHED("fp8_grouped_direct_transpose");
    return FGB_OK;
}
