// gemm.hip -- blockwise-scaled FP8 GEMM (dense and M-grouped) on gfx950 MFMA.
//
// llm-infra-atlas, "01 · DeepSeek FP8 and DeepGEMM: Hopper software recipe":
//   §1 a Linear's Fprop / Dgrad / Wgrad; §0 and §4 the accumulation-precision
//   problem of FP8 matrix units and its fix -- every 128-element K group's
//   scaled partial sum is accumulated in full FP32; §5.2 1D2D (1x128 A,
//   128x128 B scales) vs 1D1D (1x128 scales on both sides, Wgrad); §5.6
//   M-grouped contiguous layout for MoE experts; §5.7 NT, K-major operands.
// xllm-io review "MOSS", §3: 32-element E8M0 scales plus an FP32 level-1
//   factor (the b_l1 epilogue).
//
// Two arithmetic modes share the tiling, the copy pipeline and the epilogue:
//
// FGB_GEMM_EXACT (default).  The gfx950 FP8 matrix unit adds the 8 products of
//   each 8-byte lane group with the smaller ones cut to 13 bits below the
//   group's largest (measured), which is far from FP32 accumulation on
//   data with outliers.  This mode therefore converts each FP8 fragment to
//   bf16 with its power-of-two scale folded in (v_cvt_scalef32_pk_bf16_fp8:
//   an E4M3 value times 2^e is exact in bf16) and multiplies with the bf16
//   MFMA, whose products are exact and whose sums are FP32 with
//   round-to-nearest-even.  The result is the FP32 accumulation of exact
//   products -- the scale per K group is applied exactly, before the sum.
// FGB_GEMM_FAST.  V_MFMA_SCALE_F32_32X32X64_F8F6F4 consumes the FP8 codes and
//   one E8M0 scale byte per lane and 32-element K block directly (the
//   128-element group scale is fed to its four blocks; 1x32 scales as they
//   are).  Twice the MFMA rate, with the matrix unit's own product-sum
//   precision (see above); accumulation across K groups is FP32.
//
// Tiling: a 256x256 output tile per workgroup, K steps of 128.  Four waves,
// one per SIMD, each own a 128x128 quarter (4x4 tiles of 32x32); the exact
// mode's masked layout runs eight waves of 128x64 instead (two per SIMD).  A
// and B tiles go HBM -> LDS with global_load_lds (16 bytes per lane) through
// a ring of two K-step buffers (64 KB each, A then B); one barrier per K step
// waits for step k+1 and frees the buffer of step k, and step k+2's copies
// trickle out over the slots that follow it, between the MFMAs.  The scale
// bytes travel the same way into two K-step tables.  A tile row (128 bytes
// of one K step) keeps its 16-byte chunk c at position c ^ (row % 8), so the
// reads of one chunk by 8 or 16 consecutive rows are free of bank conflicts.
// Tiles run in bands of 4 m-tiles; dense and K-grouped launches give each XCD
// a contiguous range of tiles, M-grouped ones interleave chunks of 32 tiles
// over the XCDs.
//
// Fragment layout, per lane (row r = lane%32 of a 32-row tile, half h =
// lane/32), per K step (chunks 0-7 of each tile row):
//   FAST : half-step hs (64 K) is one 32x32x64 scaled MFMA; lane half h
//          supplies chunks 4hs+h and 4hs+2+h.
//   EXACT: 16-deep sub-step s uses bytes 0-7 (s even) or 8-15 (s odd) of
//          chunk 2(s/2)+h, converted to 8 bf16 values.
#include <atomic>
#include <type_traits>

#include "fgb_internal.h"

namespace fgb {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));

constexpr int BM = 256, BN = 256, BK = 128;
constexpr int NBUF = 2;                              // ring of K-step (K = 128) buffers
constexpr int STEP_BYTES = BM * BK;                  // one operand tile of a K step: 32 KB
constexpr int BUF_BYTES = 2 * STEP_BYTES;            // A and B: 64 KB
constexpr int SC_SLOT = 2 * 256 * 4;                 // A and B scale tables of one K step: 2 KB
constexpr int SC_OFF = 0;                             // LDS: scale tables of two K steps,
constexpr int RING_OFF = 2 * SC_SLOT;                 // then the ring of K-step buffers,
constexpr int EPI_OFF = RING_OFF + BUF_BYTES;         // the epilogue staging from buffer 1 on
constexpr int EPI_CAP = 8 * 64 * (64 * 2 + 16);       // largest staging (8 waves x 64 rows of 64 bf16): 72 KB
constexpr int LDS_BYTES = EPI_OFF + EPI_CAP;          // 140 KB
static_assert(LDS_BYTES >= RING_OFF + NBUF * BUF_BYTES, "the ring fits");

// Word 3 of a raw buffer descriptor on gfx9-family GPUs: 32-bit data format,
// no swizzle, no index stride (range checks on the byte offset).
constexpr int BUF_DWORD3 = 0x00020000;

enum { MODE_EXACT = 0, MODE_FAST = 1 };
enum { AG_ROW128 = 0, AG_ROW32 = 1 };
// dense, M-grouped (experts' rows: contiguous segments, or the masked layout), K-grouped (experts' K ranges)
enum { GK_NONE = 0, GK_M = 1, GK_K = 2, GK_MM = 3 };
// Waves per workgroup: one per SIMD (each 128 x 128 of the tile), except the
// exact mode's masked layout, which runs two per SIMD (each 128 x 64): there
// most tiles have valid rows only in their upper half, and with 128 x 128
// waves the lower half's SIMDs would idle.
template <int MODE, int GK> struct Waves {
    static constexpr int NW = MODE == MODE_EXACT && GK == GK_MM ? 8 : 4;
};
enum { BG_ROW128 = 0, BG_ROW32 = 1, BG_BLOCK = 2 };

struct GemmArgs {
    const uint8_t *a, *sa, *b, *sb;
    const float *l1;
    void *d;
    int64_t M, N, K, lda, ldb, ldd;
    int accumulate;
    int tiles_n;
    const int32_t *offs; // grouped: group offsets [G+1]
    int G;
    int64_t b_stride, sb_stride; // M-grouped: per-expert B / SB strides
    const int32_t *koffs;        // K-grouped: per-expert K offsets [G+1] (multiples of 128)
    int64_t d_stride;            // K-grouped: per-expert output stride (elements)
    const int32_t *masked_m;     // M-grouped, masked layout: valid rows per expert [G] (else NULL)
    int64_t m_max;               // masked layout: rows reserved per expert
};

// Rows [lo, hi) of expert g in the M-grouped layouts: the group offsets, or
// in the masked layout the first masked_m[g] (clamped to [0, m_max]) rows of
// the expert's m_max-row slot.
__device__ __forceinline__ void expert_rows(const GemmArgs &p, int g, int64_t &lo, int64_t &hi)
{
    if (p.masked_m) {
        int64_t v = p.masked_m[g];
        v = v < 0 ? 0 : (v > p.m_max ? p.m_max : v);
        lo = (int64_t)g * p.m_max;
        hi = lo + v;
    } else {
        lo = p.offs[g];
        hi = p.offs[g + 1];
    }
}

// The m-tiles of the M-grouped layouts, found with one lane per expert: lane l
// of each pass over 64 experts reads expert g0 + l's row range (one vector
// load for all experts of the pass instead of one dependent load per expert),
// counts its 256-row tiles and takes a wave prefix sum of the counts.
// Measured on the MI355X over 32 experts: 2-5% off each expert GEMM against a
// loop with one dependent load per expert.
__device__ __forceinline__ int32_t wave_inclusive_sum(int32_t v)
{
    const int lane = (int)(threadIdx.x & 63);
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
        const int32_t u = __shfl_up(v, d);
        if (lane >= d)
            v += u;
    }
    return v;
}

// Rows and m-tile count of expert g0 + lane (0 past the last expert).
__device__ __forceinline__ int32_t expert_tiles_lane(const GemmArgs &p, int g, int64_t &lo, int64_t &hi)
{
    lo = hi = 0;
    if (g >= p.G)
        return 0;
    expert_rows(p, g, lo, hi);
    return hi > lo ? (int32_t)((hi - lo + BM - 1) / BM) : 0;
}

// One pass over 64 experts (lane l: expert g0 + l): row range, tile count
// and the inclusive prefix sum of the counts.  The first pass is loaded once
// and serves both the tile count and the lookup below (one dependent round
// of loads fewer per workgroup for the usual G <= 64).
struct ExpertPass {
    int64_t lo, hi;
    int32_t nt, incl;
};
__device__ __forceinline__ ExpertPass expert_pass(const GemmArgs &p, int g0)
{
    ExpertPass x;
    x.nt = expert_tiles_lane(p, g0 + (int)(threadIdx.x & 63), x.lo, x.hi);
    x.incl = wave_inclusive_sum(x.nt);
    return x;
}

// Total m-tiles over all experts (uniform over the wave); ep0 = expert_pass(p, 0).
__device__ __forceinline__ int64_t count_mtiles(const GemmArgs &p, const ExpertPass &ep0)
{
    int64_t total = __shfl(ep0.incl, 63);
    for (int g0 = 64; g0 < p.G; g0 += 64)
        total += __shfl(expert_pass(p, g0).incl, 63);
    return total;
}

// The expert owning m-tile tm (in expert order, each expert's tiles
// contiguous), its first row of the tile and its row end; e = -1 if none.
__device__ __forceinline__ void find_mtile(const GemmArgs &p, const ExpertPass &ep0, int64_t tm, int &e,
                                           int64_t &m0, int64_t &m_end)
{
    int64_t base = 0;
    e = -1;
    for (int g0 = 0; g0 < p.G; g0 += 64) {
        const ExpertPass x = g0 == 0 ? ep0 : expert_pass(p, g0);
        const int64_t first = base + x.incl - x.nt;
        const uint64_t hit = __ballot(x.nt > 0 && tm >= first && tm < first + x.nt);
        if (hit) { // uniform
            const int l = __builtin_ctzll(hit);
            e = g0 + l;
            const int64_t lo_e = __shfl(x.lo, l), hi_e = __shfl(x.hi, l), first_e = __shfl(first, l);
            m0 = lo_e + (tm - first_e) * BM;
            m_end = hi_e;
            return;
        }
        base += __shfl(x.incl, 63);
    }
}

// Contiguous tile ranges per XCD: workgroup b runs on XCD b % 8.
__device__ __forceinline__ int64_t xcd_remap(int64_t b, int64_t nb)
{
    int64_t x = b & 7, i = b >> 3, q = nb >> 3, r = nb & 7;
    return x < r ? x * (q + 1) + i : r * (q + 1) + (x - r) * q + i;
}

// Chunks of 32 tiles (one per CU of an XCD): XCD x runs chunk x of each group
// of 8 chunks, so at any time the eight XCDs work on 8 neighbouring chunks,
// i.e. on the same expert's weights; a last partial group falls back to
// contiguous ranges.  Workgroup b runs on XCD b % 8.
__device__ __forceinline__ int64_t xcd_chunked(int64_t b, int64_t nb)
{
    constexpr int64_t CH = 32;
    const int64_t full = nb / (8 * CH) * (8 * CH);
    if (b >= full)
        return full + xcd_remap(b - full, nb - full);
    const int64_t x = b & 7, i = b >> 3;
    return (i / CH) * (8 * CH) + x * CH + (i % CH);
}

// LDS chunk swizzle of a 128-byte tile row: chunk c of row r sits at
// position c ^ (r % 8).  For 8 consecutive rows reading one chunk the
// positions are all distinct (every bank once), and 16 consecutive rows touch
// every bank exactly twice, so 16-byte reads of a chunk column are free of
// conflicts whether the LDS serves 8 or 16 lanes per pass.
__device__ __forceinline__ int swz(int r) { return r & 7; }

// 8 E4M3 codes (two words) -> one 8-element bf16 operand, each value times 2^e (sc = 2^e).
__device__ __forceinline__ v8bf cvt8_bf16(uint32_t w0, uint32_t w1, float sc)
{
    uint4 a;
    a.x = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w0, sc, false));
    a.y = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w0, sc, true));
    a.z = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w1, sc, false));
    a.w = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w1, sc, true));
    return __builtin_bit_cast(v8bf, a);
}

// The same for 8 E5M2 codes (an E5M2 value times 2^e is exact in bf16 too).
__device__ __forceinline__ v8bf cvt8_bf16_e5m2(uint32_t w0, uint32_t w1, float sc)
{
    uint4 a;
    a.x = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_bf8(w0, sc, false));
    a.y = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_bf8(w0, sc, true));
    a.z = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_bf8(w1, sc, false));
    a.w = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_bf8(w1, sc, true));
    return __builtin_bit_cast(v8bf, a);
}

// Scale byte -> the fp32 whose exponent field it is.  The scaled conversion
// reads only the exponent field of its scale operand, as an E8M0 value, so
// byte 0 (exponent field 0, the fp32 zero) multiplies by 2^-127 exactly like
// every other byte multiplies by 2^(byte - 127) (measured on gfx950 for every
// code at exponent fields 0, 1 and 127; the result is the nearest bf16, so it
// is exact wherever code * 2^(byte - 127) has a bf16 representation).
__device__ __forceinline__ float scale_f32(uint32_t byte) { return __uint_as_float(byte << 23); }

__device__ __forceinline__ v8i cat(uint4 x, uint4 y)
{
    return (v8i){(int)x.x, (int)x.y, (int)x.z, (int)x.w, (int)y.x, (int)y.y, (int)y.z, (int)y.w};
}

// FA: A's element format for the matrix unit (0 = E4M3, 1 = E5M2); B is E4M3.
template <int OPA, int OPB, int FA = 0>
__device__ __forceinline__ v16f mfma_scaled(v8i a, v8i b, v16f c, uint32_t sa, uint32_t sb)
{
    return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, FA, 0, OPA, (int)sa, OPB, (int)sb);
}

// AF: element format of A's codes (FMT_E4M3, or FMT_E5M2 for gradients).
// ACC: FP32 out, D += the product (dense and K-grouped forms only).
template <int MODE, int AG, int BG, bool OUT_BF16, int GK, int AF = FMT_E4M3, bool ACC = false>
__global__ __launch_bounds__((Waves<MODE, GK>::NW * 64)) __attribute__((amdgpu_waves_per_eu(Waves<MODE, GK>::NW / 4, Waves<MODE, GK>::NW / 4))) void
gemm_fp8_kernel(GemmArgs p)
{
    extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
    // NW waves: a 2 x NW/2 grid of 128 x WNC sub-tiles (TJ column tiles of 32)
    constexpr int NW = Waves<MODE, GK>::NW, WNC = 256 / (NW / 2), TJ = WNC / 32;
    constexpr int RPW = 256 / NW, IPO = RPW / 8; // copy rows and instructions per wave and operand
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wm = wave / (NW / 2), wn = wave % (NW / 2);
    const int l32 = lane & 31, hk = lane >> 5;
    const int64_t K = p.K; // row length of A and B (K-grouped: the whole K capacity)
    int64_t kbeg = 0, nk = K / BK;
    const int64_t N = p.N;

    // ---- tile -> (m0, n0) ------------------------------------------------
    // Tiles run in bands of GM m-tiles: consecutive tiles walk down a band
    // first, so the ~32 tiles an XCD runs at once form a GM x 8 block sharing
    // A rows and B columns in L2.  Dense and K-grouped: each XCD takes a
    // contiguous range of tiles.  M-grouped: chunks of 32 tiles interleave
    // over the XCDs, so all of them work on one expert's weights at a time
    // (with contiguous ranges each XCD held other experts' weights).
    // K-grouped: workgroups run expert by expert, and the remap applies inside
    // each expert's range, so every expert's tiles spread over all XCDs
    // (expert K ranges differ widely; whole experts per XCD would unbalance them).
    int64_t tiles_here = gridDim.x;
    ExpertPass ep0 = {}; // M-grouped: the first 64 experts (see expert_pass)
    int ke = 0; // K-grouped: this workgroup's expert, whose K range is [koffs[ke], koffs[ke+1])
    if constexpr (GK == GK_K)
        tiles_here = gridDim.x / p.G;
    constexpr bool MG = GK == GK_M || GK == GK_MM; // M-grouped (GK_MM: the masked layout)
    if constexpr (MG) {
        // The grid is a host-side bound; the m-tiles that exist are counted
        // from the expert row ranges and the surplus workgroups exit, so the
        // XCD mapping spreads only real tiles.
        ep0 = expert_pass(p, 0);
        const int64_t mt = count_mtiles(p, ep0);
        tiles_here = min(mt, (int64_t)gridDim.x / p.tiles_n) * p.tiles_n;
        if ((int64_t)blockIdx.x >= tiles_here)
            return; // uniform per workgroup
    }
    const int64_t tile = MG ? xcd_chunked(blockIdx.x, tiles_here)
                                    : xcd_remap(blockIdx.x % tiles_here, tiles_here);
    if constexpr (GK == GK_K) {
        ke = (int)(blockIdx.x / tiles_here);
        kbeg = p.koffs[ke];
        nk = (p.koffs[ke + 1] - kbeg) / BK;
    }
    int64_t tm, tn;
    {
        constexpr int64_t GM = 4;
        const int64_t tiles_m = tiles_here / p.tiles_n;
        const int64_t band = tile / (GM * p.tiles_n), in = tile % (GM * p.tiles_n);
        const int64_t bm = min(GM, tiles_m - band * GM); // rows in this (possibly last) band
        tm = band * GM + in % bm;
        tn = in / bm;
    }
    int64_t m0 = 0, m_end = 0;
    const uint8_t *B = p.b, *SB = p.sb;
    if constexpr (!MG) {
        m0 = tm * BM;
        m_end = p.M;
    } else {
        int e;
        find_mtile(p, ep0, tm, e, m0, m_end);
        if (e < 0)
            return; // not reached: tm < the counted m-tiles (uniform per workgroup)
        B += (int64_t)e * p.b_stride;
        SB += (int64_t)e * p.sb_stride;
    }
    const int64_t n0 = tn * BN;

    // ---- LDS layout ----------------------------------------------------------
    // Scale tables (one dword per tile row of A and per tile column of B, the
    // scale byte zero-extended, or the 4 bytes of the step's 32-element
    // blocks) for two K steps at SC_OFF, then a ring of 2 K-step buffers
    // (K = 128 each) at RING_OFF: buffer b holds the A tile (256 rows x 128
    // bytes) at b*64K and the B tile at b*64K + 32K.  Row r's 16-byte chunk c
    // sits at r*128 + 16*(c ^ swz(r)).  Step k uses buffer k % 2 and scale slot k % 2;
    // each wave copies it with 2*IPO tile instructions and one scale
    // instruction, issued over the slots after the barrier that frees buffer
    // k % 2 (every wave has read step k-2).

    // ---- copy plan ---------------------------------------------------------
    // Instruction g (0..IPO-1) of wave w copies tile rows w*RPW + g*8 .. +7,
    // 128 bytes (one K step) of each: lane l lands at LDS
    // (w*RPW + g*8)*128 + 16*l, i.e. row +l/8, position l%8, which holds chunk
    // (l%8) ^ swz(l/8) of that row (the first row is a multiple of 8).  Each
    // instruction thus reads 8 whole 128-byte lines.  Rows past the end
    // re-read the last valid row (those outputs are never stored).
    const uint8_t *a_base = p.a + m0 * p.lda + kbeg;
    const uint8_t *b_base = B + n0 * p.ldb + kbeg;
    uint32_t a_off[IPO], b_off[IPO];
#pragma unroll
    for (int g = 0; g < IPO; g++) {
        const int r = wave * RPW + g * 8 + (lane >> 3);
        const int chunk = (lane & 7) ^ swz(lane >> 3);
        const int64_t ar = m0 + r < m_end ? r : m_end - 1 - m0;
        const int64_t br = n0 + r < N ? r : N - 1 - n0;
        a_off[g] = (uint32_t)(ar * p.lda + chunk * 16);
        b_off[g] = (uint32_t)(br * p.ldb + chunk * 16);
    }
    // Scale copy: lane l of wave w fetches the scale of tile row (A) or tile
    // column (B) sw*64 + l for K step ks into dword sw*64 + l of the step's
    // table, sw = w % 4 (with 8 waves, waves 0-3 copy the A scales and waves
    // 4-7 the B scales; with 4 waves each wave copies both).
    constexpr bool A32 = AG == AG_ROW32, B32 = BG == BG_ROW32;
    const int64_t sa_row = A32 ? K / 32 : K / 128;
    const int64_t sb_row = B32 ? K / 32 : K / 128;
    uint32_t sa_off, sb_off;
    const uint8_t *sa_base = p.sa + m0 * sa_row + kbeg / (A32 ? 32 : 128), *sb_base;
    {
        const int64_t r = (wave & 3) * 64 + lane;
        const int64_t rc = m0 + r < m_end ? r : m_end - 1 - m0;
        sa_off = (uint32_t)(rc * sa_row);
        const int64_t c = n0 + r < N ? r : N - 1 - n0;
        if constexpr (BG == BG_BLOCK) {
            sb_base = SB;
            sb_off = (uint32_t)(((n0 + c) / 128) * (K / 128));
        } else {
            sb_base = SB + n0 * sb_row + kbeg / (B32 ? 32 : 128);
            sb_off = (uint32_t)(c * sb_row);
        }
    }

    // One copy instruction: M0 holds the wave-uniform LDS destination (lane l
    // lands at M0 + 16*l, or M0 + 4*l for the 1- and 4-byte forms); the global
    // address is a uniform 64-bit base (SGPRs) plus the lane's 32-bit offset.
    // Issued as inline asm so that the compiler does not place waits on them
    // in front of unrelated LDS reads; the kernel counts them itself.
    auto uniform = [](const uint8_t *q) {
        const uint64_t v = (uint64_t)(uintptr_t)q;
        const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v);
        const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
        return (const uint8_t *)(uintptr_t)(((uint64_t)hi << 32) | lo);
    };
    auto dma16 = [&](const uint8_t *gbase, uint32_t off, uint32_t lds_addr) {
        asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, %2"
                     :
                     : "s"(lds_addr), "v"(off), "s"(uniform(gbase))
                     : "memory", "m0");
    };
    auto dma4 = [&](const uint8_t *gbase, uint32_t off, uint32_t lds_addr) {
        asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dword %1, %2"
                     :
                     : "s"(lds_addr), "v"(off), "s"(uniform(gbase))
                     : "memory", "m0");
    };
    auto dma1 = [&](const uint8_t *gbase, uint32_t off, uint32_t lds_addr) {
        asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_ubyte %1, %2"
                     :
                     : "s"(lds_addr), "v"(off), "s"(uniform(gbase))
                     : "memory", "m0");
    };
    const uint32_t lds_base = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) uint8_t *)smem;
    const uint32_t wave_u = __builtin_amdgcn_readfirstlane(wave);
    const uint8_t *a_base_u = uniform(a_base), *b_base_u = uniform(b_base);
    const uint8_t *sa_base_u = uniform(sa_base), *sb_base_u = uniform(sb_base);
    const int nk32 = (int)nk; // K steps (K < 2^24)
    // Copy instruction i (0..2*IPO-1: A g=0..IPO-1, then B) of K step k
    // (clamped to the last one: copies past the end rewrite the last step's
    // buffer with the bytes it already holds).
    auto dma_tile = [&](int k, int i) {
        const int kc = k < nk32 ? k : nk32 - 1;
        const uint32_t dst = lds_base + RING_OFF + (uint32_t)(kc & 1) * BUF_BYTES + (i >= IPO ? STEP_BYTES : 0) +
                             (wave_u * RPW + (i % IPO) * 8) * 128;
        if (i < IPO)
            dma16(a_base_u + (uint32_t)kc * 128u, a_off[i % IPO], dst);
        else
            dma16(b_base_u + (uint32_t)kc * 128u, b_off[i % IPO], dst);
    };
    // The scale copies of K step ks (clamped likewise).  Both operands use
    // the same copy size (1x32 scales come on both sides or on neither).
    auto dma_scales = [&](int ks) {
        const int kc = ks < nk32 ? ks : nk32 - 1;
        const uint32_t dst = lds_base + SC_OFF + (uint32_t)(kc & 1) * SC_SLOT + (wave_u & 3) * 256;
        const uint32_t ka = A32 ? (uint32_t)kc * 4u : (uint32_t)kc, kb = B32 ? (uint32_t)kc * 4u : (uint32_t)kc;
        if constexpr (NW == 4) {
            if constexpr (A32)
                dma4(sa_base_u + ka, sa_off, dst);
            else
                dma1(sa_base_u + ka, sa_off, dst);
            if constexpr (B32)
                dma4(sb_base_u + kb, sb_off, dst + 1024);
            else
                dma1(sb_base_u + kb, sb_off, dst + 1024);
        } else {
            // one instruction per wave, no branch: waves 0-3 copy A's, 4-7 B's
            const bool is_a = wave_u < 4;
            const uint8_t *g = is_a ? sa_base_u + ka : sb_base_u + kb;
            const uint32_t off = is_a ? sa_off : sb_off;
            if constexpr (A32)
                dma4(g, off, dst + (is_a ? 0u : 1024u));
            else
                dma1(g, off, dst + (is_a ? 0u : 1024u));
        }
    };
    // Copies of step k: its scale instruction when first == 0, then tile
    // instructions first..last.
    auto dma_step = [&](int k, int first, int last) {
        if (first == 0)
            dma_scales(k);
        for (int i = first; i <= last; i++)
            dma_tile(k, i);
    };
    // Wait until at most n copy instructions are outstanding, then sync.
#define FGB_WAIT_SYNC(n)                                                                                               \
    do {                                                                                                               \
        asm volatile("s_waitcnt vmcnt(" #n ")" ::: "memory");                                                          \
        __syncthreads();                                                                                               \
    } while (0)

    // ---- scales of one K step, from its LDS table ---------------------------
    // A: word per tile of the wave (1x32: the 4 block bytes; 1x128: the byte),
    // packed for 1x128 into one word with byte t = tile t; likewise B (TJ
    // tiles), whose 128x128 form is one byte (the wave's columns lie in one
    // block).
    constexpr int NA = A32 ? 4 : 1, NB = B32 ? TJ : 1;
    // read_scales issues the LDS reads (raw dwords); pack_scales combines them
    // and is placed a few slots later so the reads have landed by then.
    auto read_scales = [&](int ks, uint32_t(&va)[4], uint32_t(&vb)[4]) {
        const uint32_t *ta = reinterpret_cast<const uint32_t *>(smem + SC_OFF + (ks & 1) * SC_SLOT);
        const uint32_t *tb = ta + 256;
#pragma unroll
        for (int t = 0; t < 4; t++) {
            va[t] = ta[wm * 128 + t * 32 + l32];
            vb[t] = (BG == BG_BLOCK || t >= TJ) ? (t == 0 ? tb[wn * WNC] : 0u) : tb[wn * WNC + t * 32 + l32];
        }
    };
    auto pack_scales = [&](const uint32_t(&va)[4], const uint32_t(&vb)[4], uint32_t(&wa)[NA], uint32_t(&wb)[NB]) {
        if constexpr (A32) {
#pragma unroll
            for (int t = 0; t < 4; t++)
                wa[t] = va[t];
        } else {
            wa[0] = va[0] | (va[1] << 8) | (va[2] << 16) | (va[3] << 24);
        }
        if constexpr (B32) {
#pragma unroll
            for (int t = 0; t < TJ; t++)
                wb[t] = vb[t];
        } else if constexpr (BG == BG_BLOCK) {
            wb[0] = vb[0];
        } else {
            wb[0] = vb[0] | (vb[1] << 8) | (vb[2] << 16) | (vb[3] << 24);
        }
    };

    // ---- fragment addressing ---------------------------------------------------
    // The wave's row t*32 + l32 of an operand tile (offset wm*128 or wn*WNC
    // rows); chunk c of it at qoff[c] + t*4096 (the swizzle depends on
    // l32 % 8 only).
    int qoff[8];
#pragma unroll
    for (int c = 0; c < 8; c++)
        qoff[c] = l32 * 128 + ((c ^ swz(l32)) * 16);
    auto lds_a = [&](int k) { return smem + RING_OFF + (k & 1) * BUF_BYTES + wm * 128 * 128; };
    auto lds_b = [&](int k) { return smem + RING_OFF + (k & 1) * BUF_BYTES + STEP_BYTES + wn * WNC * 128; };

    v16f acc[4][TJ];
#pragma unroll
    for (int i = 0; i < 4; i++)
#pragma unroll
        for (int j = 0; j < TJ; j++)
            acc[i][j] = (v16f){0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};

    if (nk32 > 0) { // an expert of the K-grouped form may have no rows: the tile is zero
    // ---- prologue ----------------------------------------------------------------
    // Step 0 and the first part of step 1 in flight (the rest of step 1 is
    // issued in the first slots of the main loop); wait for step 0 and sync.
    if constexpr (MODE == MODE_FAST) {
        dma_step(0, 0, 2 * IPO - 1);
        dma_step(1, 0, 11);
        FGB_WAIT_SYNC(14); // step 1's two scale and 12 tile instructions
    } else if constexpr (NW == 4) {
        dma_step(0, 0, 2 * IPO - 1);
        dma_step(1, 0, 7);
        FGB_WAIT_SYNC(10); // step 1's two scale and 8 tile instructions
    } else {
        dma_step(0, 0, 2 * IPO - 1);
        dma_step(1, 0, 2);
        FGB_WAIT_SYNC(4); // step 1's scale and 3 tile instructions
    }
    uint32_t ca[NA], cb[NB], sva[4], svb[4];
    read_scales(0, sva, svb);
    pack_scales(sva, svb, ca, cb);

    // ---- main loop ----------------------------------------------------------------
    // A K step is 8 slots.  One barrier per step waits for step ks+1's copies
    // (all issued at least four slots earlier) before its first reads and
    // frees buffer ks % 2 (every wave has issued its last read of step ks);
    // step ks+2's copies go out right after the barrier that frees its buffer.
    if constexpr (MODE == MODE_FAST) {
        // A half-step (64 of the step's 128 K) is one MFMA sub-step: 16 scaled
        // MFMAs, 4 per slot.  Lane half hk reads chunks 4hs+hk and 4hs+2+hk of
        // each tile row for half hs (hardware K blocks 0 and 1).  Half 1 of
        // step ks is read in slots 1 (A) and 2 (B); the barrier in slot 3 then
        // frees buffer ks % 2 and step ks+2's copies go out over slots 3-7 and
        // 0-1; the barrier in slot 5 waits for step ks+1, whose half 0 is read
        // in slots 5 (A) and 6 (B).  Each slot's 8 reads go out two after each
        // of its MFMAs: 16 reads in a row starved the matrix unit.
        uint4 f[2][2][4][2]; // [half][A/B][tile][chunk]
        auto read_frag = [&](int k, int hs, int op, uint4(&x)[4][2]) {
            const uint8_t *base = op == 0 ? lds_a(k) : lds_b(k);
#pragma unroll
            for (int t = 0; t < 4; t++) {
                x[t][0] = *reinterpret_cast<const uint4 *>(base + qoff[4 * hs + hk] + t * 4096);
                x[t][1] = *reinterpret_cast<const uint4 *>(base + qoff[4 * hs + 2 + hk] + t * 4096);
            }
        };
        // MFMAs of row tile i for half-step parity hs (32-blocks 2hs, 2hs+1 of the step)
        // Masked layout: row tiles past the expert's valid rows take no MFMAs
        // (uniform over the wave; see the exact-mode loop).
        const int nvf = GK != GK_MM ? 4
                                    : (int)min((int64_t)4, max((int64_t)0, (m_end - m0 - (int64_t)(wave_u / (NW / 2)) * 128 + 31) / 32));
        auto mfma_row = [&](int hs, int i, const uint4(&xa)[4][2], const uint4(&xb)[4][2]) {
            if (GK == GK_MM && i >= nvf)
                return;
            uint32_t wa = 0, wb = 0;
            if constexpr (A32) {
                const int sh = 8 * (2 * hs + hk);
#pragma unroll
                for (int t = 0; t < 4; t++)
                    wa |= ((ca[t] >> sh) & 0xFFu) << (8 * t);
            } else {
                wa = ca[0];
            }
            if constexpr (B32) {
                const int sh = 8 * (2 * hs + hk);
#pragma unroll
                for (int t = 0; t < 4; t++)
                    wb |= ((cb[t] >> sh) & 0xFFu) << (8 * t);
            } else {
                wb = cb[0];
            }
            const v8i av = cat(xa[i][0], xa[i][1]);
#define FGB_J(I, J)                                                                                                    \
    if (i == I)                                                                                                        \
        acc[I][J] = mfma_scaled<I, (BG == BG_BLOCK ? 0 : J), (AF == FMT_E5M2 ? 1 : 0)>(av, cat(xb[J][0], xb[J][1]),      \
                                                                                       acc[I][J], wa, wb);
#define FGB_I(I) FGB_J(I, 0) FGB_J(I, 1) FGB_J(I, 2) FGB_J(I, 3)
            FGB_I(0) FGB_I(1) FGB_I(2) FGB_I(3)
#undef FGB_I
#undef FGB_J
        };
        read_frag(0, 0, 0, f[0][0]);
        read_frag(0, 0, 1, f[0][1]);
        for (int ks = 0; ks < nk32; ks++) {
            // slot 0
            dma_tile(ks + 1, 12);
            dma_tile(ks + 1, 13);
            mfma_row(0, 0, f[0][0], f[0][1]);
            __builtin_amdgcn_sched_barrier(0);
            // slot 1
            dma_tile(ks + 1, 14);
            dma_tile(ks + 1, 15);
            read_frag(ks, 1, 0, f[1][0]);
            mfma_row(0, 1, f[0][0], f[0][1]);
            for (int k_ = 0; k_ < 4; k_++) {
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 0); // 1 MFMA
                __builtin_amdgcn_sched_group_barrier(0x100, 2, 0); // 2 LDS reads
            }
            __builtin_amdgcn_sched_barrier(0);
            // slot 2
            read_frag(ks, 1, 1, f[1][1]);
            mfma_row(0, 2, f[0][0], f[0][1]);
            for (int k_ = 0; k_ < 4; k_++) {
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 0); // 1 MFMA
                __builtin_amdgcn_sched_group_barrier(0x100, 2, 0); // 2 LDS reads
            }
            __builtin_amdgcn_sched_barrier(0);
            // slot 3: every wave's reads of step ks are done -> buffer ks % 2 is free
            __syncthreads();
            dma_step(ks + 2, 0, 1);
            mfma_row(0, 3, f[0][0], f[0][1]);
            __builtin_amdgcn_sched_barrier(0);
            // slot 4
            dma_tile(ks + 2, 2);
            dma_tile(ks + 2, 3);
            dma_tile(ks + 2, 4);
            mfma_row(1, 0, f[1][0], f[1][1]);
            __builtin_amdgcn_sched_barrier(0);
            // slot 5: step ks+1 has landed (6 instructions of step ks+2 were issued after it)
            FGB_WAIT_SYNC(6);
            read_scales(ks + 1, sva, svb);
            dma_tile(ks + 2, 5);
            dma_tile(ks + 2, 6);
            dma_tile(ks + 2, 7);
            read_frag(ks + 1, 0, 0, f[0][0]);
            mfma_row(1, 1, f[1][0], f[1][1]);
            for (int k_ = 0; k_ < 4; k_++) {
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 0); // 1 MFMA
                __builtin_amdgcn_sched_group_barrier(0x100, 2, 0); // 2 LDS reads
            }
            __builtin_amdgcn_sched_barrier(0);
            // slot 6
            dma_tile(ks + 2, 8);
            dma_tile(ks + 2, 9);
            read_frag(ks + 1, 0, 1, f[0][1]);
            mfma_row(1, 2, f[1][0], f[1][1]);
            for (int k_ = 0; k_ < 4; k_++) {
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 0); // 1 MFMA
                __builtin_amdgcn_sched_group_barrier(0x100, 2, 0); // 2 LDS reads
            }
            __builtin_amdgcn_sched_barrier(0);
            // slot 7: the next step's scales replace the current ones after
            // this slot's MFMAs
            dma_tile(ks + 2, 10);
            dma_tile(ks + 2, 11);
            mfma_row(1, 3, f[1][0], f[1][1]);
            pack_scales(sva, svb, ca, cb);
            __builtin_amdgcn_sched_barrier(0);
        }
    } else if constexpr (NW == 4) {
        // Exact mode, 4 waves (one per SIMD, each 128 x 128).  A slot is one
        // 16-deep sub-step s: its 16 bf16 MFMAs, with the 32 conversions of
        // sub-step s+1 into the other operand buffer issued between them, so
        // the single wave keeps the matrix unit fed while it converts.  Sub-step
        // s takes bytes 0-7 (s even) or 8-15 (s odd) of chunk 2q + hk of each
        // tile row, q = s/2 the 32-wide pair.  A slot is cut into quarters of
        // 4 MFMAs (row tile t) and 8 conversions (A and B tile t), each quarter
        // carrying its share of the slot's LDS reads and copies, so that no
        // run of memory instructions leaves the matrix unit idle.  Pair q's
        // reads are issued one slot before its first conversion; the barrier
        // before slot 6 waits for step ks+1 and frees buffer ks % 2 (pair 3
        // was converted in slot 5); step ks+2's copies go out in slots 6-7 and
        // 0-2.
        static_assert(GK != GK_MM, "the masked layout runs 8 waves");
        uint4 rA[2][4], rB[2][4]; // FP8 fragments of two pairs
        v8bf cA[2][4], cB[2][4];  // bf16 operands of two sub-steps
        float sfA[4], sfB[4];     // scale factors of the pair being converted
        auto factors = [&](int q) {
#pragma unroll
            for (int t = 0; t < 4; t++)
                if (A32 || q == 0)
                    sfA[t] = scale_f32(A32 ? (ca[t] >> (8 * q)) & 0xFFu : (ca[0] >> (8 * t)) & 0xFFu);
#pragma unroll
            for (int t = 0; t < 4; t++)
                if (B32 || q == 0)
                    sfB[t] = scale_f32(B32 ? (cb[t] >> (8 * q)) & 0xFFu
                                           : (BG == BG_BLOCK ? cb[0] : (cb[0] >> (8 * t)) & 0xFFu));
        };
        // Tile t of pair q of step k (A and B), its conversion for sub-step
        // half `half` into buffer `half`, and the MFMAs of row tile i.
        auto read_piece = [&](int k, int q, int t, uint4(&xa)[4], uint4(&xb)[4]) {
            const int c = 2 * q + hk;
            xa[t] = *reinterpret_cast<const uint4 *>(lds_a(k) + qoff[c] + t * 4096);
            xb[t] = *reinterpret_cast<const uint4 *>(lds_b(k) + qoff[c] + t * 4096);
        };
        auto cvt_piece = [&](int half, int t, const uint4(&xa)[4], const uint4(&xb)[4]) {
            if constexpr (AF == FMT_E5M2)
                cA[half][t] = half == 0 ? cvt8_bf16_e5m2(xa[t].x, xa[t].y, sfA[t]) : cvt8_bf16_e5m2(xa[t].z, xa[t].w, sfA[t]);
            else
                cA[half][t] = half == 0 ? cvt8_bf16(xa[t].x, xa[t].y, sfA[t]) : cvt8_bf16(xa[t].z, xa[t].w, sfA[t]);
            cB[half][t] = half == 0 ? cvt8_bf16(xb[t].x, xb[t].y, sfB[t]) : cvt8_bf16(xb[t].z, xb[t].w, sfB[t]);
        };
        auto mfma_row = [&](int buf, int i) {
#pragma unroll
            for (int j = 0; j < 4; j++)
                acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(cA[buf][i], cB[buf][j], acc[i][j], 0, 0, 0);
        };
        // Quarter T of a slot: the statements written before it (copies,
        // reads), then row tile T's 4 MFMAs on buffer 1 - HALF, each followed
        // by 2 of the 8 conversions of piece T of the next sub-step (from
        // fragments RX) into buffer HALF.
#define FGB_Q(HALF, RX, T)                                                                                             \
    do {                                                                                                               \
        cvt_piece(HALF, T, rA[RX], rB[RX]);                                                                            \
        mfma_row(1 - (HALF), T);                                                                                       \
        for (int k_ = 0; k_ < 4; k_++) {                                                                               \
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0); /* 1 MFMA */                                            \
            __builtin_amdgcn_sched_group_barrier(0x002, 2, 0); /* 2 VALU */                                            \
        }                                                                                                              \
        __builtin_amdgcn_sched_barrier(0);                                                                             \
    } while (0)

        // sub-step 0 of step 0 into buffer 0
        factors(0);
#pragma unroll
        for (int t = 0; t < 4; t++)
            read_piece(0, 0, t, rA[0], rB[0]);
#pragma unroll
        for (int t = 0; t < 4; t++)
            cvt_piece(0, t, rA[0], rB[0]);
        __builtin_amdgcn_sched_barrier(0);
        for (int ks = 0; ks < nk32; ks++) {
            // slot s: MFMAs of sub-step s (buffer s % 2); conversions of
            // sub-step s+1 (pair (s+1)/2, half (s+1) % 2) into buffer (s+1) % 2
            // slot 0: pair 1's reads; step ks+1's copies 8-11
#pragma unroll
            for (int t = 0; t < 4; t++) {
                read_piece(ks, 1, t, rA[1], rB[1]);
                dma_tile(ks + 1, 8 + t);
                FGB_Q(1, 0, t);
            }
            // slot 1: copies 12-13
            factors(1);
            dma_tile(ks + 1, 12);
            FGB_Q(0, 1, 0);
            dma_tile(ks + 1, 13);
            FGB_Q(0, 1, 1);
            FGB_Q(0, 1, 2);
            FGB_Q(0, 1, 3);
            // slot 2: pair 2's reads; copies 14-15
#pragma unroll
            for (int t = 0; t < 4; t++) {
                read_piece(ks, 2, t, rA[0], rB[0]);
                if (t < 2)
                    dma_tile(ks + 1, 14 + t);
                FGB_Q(1, 1, t);
            }
            // slot 3
            factors(2);
#pragma unroll
            for (int t = 0; t < 4; t++)
                FGB_Q(0, 0, t);
            // slot 4: pair 3's reads
#pragma unroll
            for (int t = 0; t < 4; t++) {
                read_piece(ks, 3, t, rA[1], rB[1]);
                FGB_Q(1, 0, t);
            }
            // slot 5
            factors(3);
#pragma unroll
            for (int t = 0; t < 4; t++)
                FGB_Q(0, 1, t);
            // slot 6: step ks+1 has landed (nothing issued after it) and buffer
            // ks % 2 is free; step ks+1's scales and pair 0, step ks+2's scales
            // and copies 0-3.  After the last step these reads touch only LDS
            // and are discarded.
            FGB_WAIT_SYNC(0);
            read_scales(ks + 1, sva, svb);
            dma_scales(ks + 2);
#pragma unroll
            for (int t = 0; t < 4; t++) {
                read_piece(ks + 1, 0, t, rA[0], rB[0]);
                dma_tile(ks + 2, t);
                FGB_Q(1, 1, t);
            }
            // slot 7: step ks+1's scales replace the current ones; copies 4-7
            pack_scales(sva, svb, ca, cb);
            factors(0);
#pragma unroll
            for (int t = 0; t < 4; t++) {
                dma_tile(ks + 2, 4 + t);
                FGB_Q(0, 0, t);
            }
        }
#undef FGB_Q
    } else {
        // Exact mode, 8 waves (the masked layout; two per SIMD, each 128 x 64): a slot is one
        // 16-deep sub-step -- the 24 conversions of its FP8 fragments (4 A
        // tiles, 2 B tiles; the scale folded in) and its 8 bf16 MFMAs; while
        // one wave of a SIMD converts, the other keeps the matrix unit busy.
        // Sub-step s of a step takes bytes 0-7 (s even) or 8-15 (s odd) of
        // chunk 2q + hk, q = s/2 the 32-wide pair.  Pair q+1's LDS reads are
        // issued two slots before its first conversion.  The barrier before
        // slot 6 (after the reads of pair 3) waits for step ks+1 and frees
        // buffer ks % 2; step ks+2's copies go out in slots 6-7 and 0-2.
        static_assert(NW == 8, "exact mode runs 8 waves");
        uint4 rA[2][4], rB[2][TJ]; // FP8 fragments of two pairs
        v8bf cA[4], cB[TJ];        // bf16 operands of the current sub-step
        float sfA[4], sfB[TJ];     // scale factors of the pair being converted
        auto read_pair = [&](int k, int q, uint4(&xa)[4], uint4(&xb)[TJ]) {
            const uint8_t *la = lds_a(k), *lb = lds_b(k);
            const int c = 2 * q + hk;
#pragma unroll
            for (int t = 0; t < 4; t++)
                xa[t] = *reinterpret_cast<const uint4 *>(la + qoff[c] + t * 4096);
#pragma unroll
            for (int t = 0; t < TJ; t++)
                xb[t] = *reinterpret_cast<const uint4 *>(lb + qoff[c] + t * 4096);
        };
        auto factors = [&](int q) {
#pragma unroll
            for (int t = 0; t < 4; t++)
                if (A32 || q == 0)
                    sfA[t] = scale_f32(A32 ? (ca[t] >> (8 * q)) & 0xFFu : (ca[0] >> (8 * t)) & 0xFFu);
#pragma unroll
            for (int t = 0; t < TJ; t++)
                if (B32 || q == 0)
                    sfB[t] = scale_f32(B32 ? (cb[t] >> (8 * q)) & 0xFFu
                                           : (BG == BG_BLOCK ? cb[0] : (cb[0] >> (8 * t)) & 0xFFu));
        };
        // Masked layout (decode: experts with few valid rows): the wave's
        // 32-row tiles past the expert's valid rows take neither conversions
        // nor MFMAs, and a wave with no valid row (NV = 0) only makes its
        // copies and meets every barrier.  The main loop is specialised on the
        // wave's count NV of valid row tiles (uniform over the wave, read into
        // a scalar register): tested inside the loop, the conditional MFMAs
        // made the compiler copy and spill the accumulators.
        auto main_loop = [&](auto nv_tag) {
            constexpr int NV = decltype(nv_tag)::value;
            auto convert = [&](int sub, const uint4(&xa)[4], const uint4(&xb)[TJ]) {
#pragma unroll
                for (int t = 0; t < NV; t++)
                    if constexpr (AF == FMT_E5M2)
                        cA[t] = sub == 0 ? cvt8_bf16_e5m2(xa[t].x, xa[t].y, sfA[t]) : cvt8_bf16_e5m2(xa[t].z, xa[t].w, sfA[t]);
                    else
                        cA[t] = sub == 0 ? cvt8_bf16(xa[t].x, xa[t].y, sfA[t]) : cvt8_bf16(xa[t].z, xa[t].w, sfA[t]);
#pragma unroll
                for (int t = 0; t < TJ; t++)
                    cB[t] = sub == 0 ? cvt8_bf16(xb[t].x, xb[t].y, sfB[t]) : cvt8_bf16(xb[t].z, xb[t].w, sfB[t]);
            };
            auto mfmas = [&]() {
#pragma unroll
                for (int i = 0; i < NV; i++)
#pragma unroll
                    for (int j = 0; j < TJ; j++)
                        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(cA[i], cB[j], acc[i][j], 0, 0, 0);
            };
#define FGB_SLOT(SUB, RX, DMA)                                                                                         \
    do {                                                                                                               \
        if constexpr (NV > 0) {                                                                                        \
            convert(SUB, rA[RX], rB[RX]);                                                                              \
            mfmas();                                                                                                   \
        }                                                                                                              \
        __builtin_amdgcn_sched_barrier(0);                                                                             \
        DMA;                                                                                                           \
        __builtin_amdgcn_sched_barrier(0);                                                                             \
    } while (0)

            read_pair(0, 0, rA[0], rB[0]);
            factors(0);
            for (int ks = 0; ks < nk32; ks++) {
                // slots 0-1: read pair 1; sub-steps 0, 1 (pair 0)
                read_pair(ks, 1, rA[1], rB[1]);
                FGB_SLOT(0, 0, (dma_tile(ks + 1, 3), dma_tile(ks + 1, 4)));
                FGB_SLOT(1, 0, (dma_tile(ks + 1, 5), dma_tile(ks + 1, 6)));
                // slots 2-3: read pair 2; sub-steps 2, 3 (pair 1)
                read_pair(ks, 2, rA[0], rB[0]);
                factors(1);
                FGB_SLOT(0, 1, dma_tile(ks + 1, 7));
                FGB_SLOT(1, 1, (void)0);
                // slots 4-5: read pair 3; sub-steps 4, 5 (pair 2)
                read_pair(ks, 3, rA[1], rB[1]);
                factors(2);
                FGB_SLOT(0, 0, (void)0);
                FGB_SLOT(1, 0, (void)0);
                // slots 6-7: step ks+1 has landed (nothing issued after it) and
                // buffer ks % 2 is free; the next step's scales and pair 0; sub-steps
                // 6, 7 (pair 3).  After the last step these reads touch only LDS
                // and are discarded.
                FGB_WAIT_SYNC(0);
                read_scales(ks + 1, sva, svb);
                read_pair(ks + 1, 0, rA[0], rB[0]);
                factors(3);
                FGB_SLOT(0, 1, (dma_step(ks + 2, 0, 0)));
                FGB_SLOT(1, 1, (dma_tile(ks + 2, 1), dma_tile(ks + 2, 2)));
                pack_scales(sva, svb, ca, cb);
                factors(0);
            }
        };
        if constexpr (GK != GK_MM) {
            main_loop(std::integral_constant<int, 4>{});
        } else {
            const int nv = __builtin_amdgcn_readfirstlane(
                (int)min((int64_t)4, max((int64_t)0, (m_end - m0 - (int64_t)(wave_u / (NW / 2)) * 128 + 31) / 32)));
            switch (nv) {
            case 0: main_loop(std::integral_constant<int, 0>{}); break;
            case 1: main_loop(std::integral_constant<int, 1>{}); break;
            case 2: main_loop(std::integral_constant<int, 2>{}); break;
            case 3: main_loop(std::integral_constant<int, 3>{}); break;
            default: main_loop(std::integral_constant<int, 4>{}); break;
            }
        }
#undef FGB_SLOT
    }
#undef FGB_WAIT_SYNC
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); // trailing copies land before LDS is reused
    } // nk32 > 0

    // ---- epilogue --------------------------------------------------------------
    // 32x32 accumulator layout: lane l, register r -> row (r/4)*8 + (l/32)*4 + r%4,
    // column l%32.
    // FP32 out: every register goes straight to memory; one store writes 32
    //   consecutive columns (128 bytes) of two rows.
    // BF16 out: the block is staged through LDS (free after the barrier below;
    //   from buffer 1 on) so that global stores are 16 bytes per lane along
    //   rows: each wave writes its 128 x WNC block, EPI_ROWS rows at a time, and
    //   reads it back row-contiguous, as row pairs: a lane's registers
    //   4q..4q+3 are rows 2p..2p+3 of one column, so one conversion packs rows
    //   (2p, 2p+1) into a dword at [pair][column]; the read-back takes 32
    //   bytes of one pair (8 columns) and splits them into the two rows' 16
    //   bytes with byte permutes, with no exchange between lanes.
    // The instruction count sets this phase's time (measured: the stores
    // drain within 0.2-0.4 us), so a block inside D (16-byte aligned rows)
    // carries no per-row bound tests, and only the kernels with 1x32 B scales
    // (the only ones given level-1 factors) multiply by them.
    __syncthreads();
    constexpr int ESZ = OUT_BF16 ? 2 : 4;
    constexpr int ROWB = WNC * ESZ + 16; // padded LDS row (bytes)
    constexpr int RPB = 2 * WNC * 2 + 16; // BF16 out: padded LDS row pair (bytes; 2 * ROWB - 16)
    constexpr int EPI_ROWS = NW * 128 * ROWB <= EPI_CAP ? 128 : NW * 64 * ROWB <= EPI_CAP ? 64 : 32;
    static_assert(NW * EPI_ROWS * ROWB <= EPI_CAP, "the staging fits");
    static_assert(!OUT_BF16 || (EPI_ROWS / 2) * RPB <= EPI_ROWS * ROWB, "the row-pair staging fits the wave's share");
    uint8_t *ep = smem + EPI_OFF + wave * (EPI_ROWS * ROWB);
    // level-1 factor of each column (MOSS)
    const bool has_l1 = p.l1 != nullptr; // uniform
    float l1v[TJ];
#pragma unroll
    for (int j = 0; j < TJ; j++) {
        const int64_t col = n0 + wn * WNC + j * 32 + l32;
        l1v[j] = (has_l1 && col < N) ? p.l1[col] : 1.0f;
    }
    // read-back geometry: one row segment of 16 bytes per lane
    constexpr int LPR = WNC * ESZ / 16; // lanes per row
    constexpr int RPI = 64 / LPR;       // rows per instruction
    const int lr = lane / LPR, lc = lane % LPR;
    const int64_t colw = n0 + wn * WNC; // the wave's first column
    const int64_t col0 = colw + lc * (16 / ESZ);
    const int64_t row_w = m0 + wm * 128; // the wave's first row
    const int64_t ld_bytes = p.ldd * ESZ;
    uint8_t *const dblock = (uint8_t *)p.d + (ke * p.d_stride + row_w * p.ldd + colw) * ESZ;
    uint8_t *const dwave = dblock + (col0 - colw) * ESZ;
    // rows of the wave below m_end (0..128) and whether this lane's 16 bytes are a whole aligned segment
    const int rows_ok = (int)min((int64_t)128, max((int64_t)0, m_end - row_w));
    const bool col_ok = col0 < N;
    const bool full = col0 + 16 / ESZ <= N && (((uintptr_t)dwave & 15) == 0) && ((ld_bytes & 15) == 0);
    // the whole block inside D with aligned rows (uniform over the wave)
    const bool block_full = rows_ok == 128 && colw + WNC <= N && ((((uintptr_t)dblock) | (uintptr_t)ld_bytes) & 15) == 0;

    // Level-1 factors come only with 1x32 B scales (MOSS); other kernels
    // store the accumulators as they are.  Without factors l1v is 1.0, which
    // leaves every value unchanged.
    constexpr bool L1 = BG == BG_ROW32;
    if constexpr (!OUT_BF16) {
        // FP32 out, every block: raw buffer accesses, one descriptor per 32-row
        // tile whose record count covers only the tile's rows below m_end, at
        // byte offset row * ld + the lane's column (4 rows down for the upper
        // half-wave).  A lane whose column lies past N gets an offset of at
        // least 2^30, above every record count (the launcher keeps 32 * ld
        // below 2^30), so the range check drops its stores and zeroes its
        // loads, as it does for rows past m_end.  One batch per 32 x 32 tile:
        // its 16 values.  Accumulation is a template parameter: tested at run
        // time, the two store sequences made the compiler move every
        // accumulator into vector registers first and spill 40-57 of them.
        // Accumulating, the old values of D are read AHEAD batches before
        // their use, one register set per batch in flight: read batch by
        // batch, every batch waited out the full HBM latency of its loads
        // (34 us of epilogue per tile against 7 us without accumulation).
        constexpr int OOB = 1 << 30;
        int lane_off[TJ];
#pragma unroll
        for (int j = 0; j < TJ; j++)
            lane_off[j] = (colw + j * 32 + l32 < N ? 0 : OOB) + (int)(hk * 4 * ld_bytes) + l32 * 4 + j * 128;
        auto tile_rsrc = [&](int i) {
            const int rows_i = min(32, max(0, rows_ok - i * 32));
            return __builtin_amdgcn_make_buffer_rsrc((void *)uniform(dblock + (int64_t)i * 32 * ld_bytes), 0,
                                                     __builtin_amdgcn_readfirstlane(rows_i * (int)ld_bytes),
                                                     BUF_DWORD3);
        };
        auto batch = [&](int b, float (&v)[16]) { // the 16 output values of batch b = (i, j)
            const int i = b / TJ, j = b % TJ;
#pragma unroll
            for (int r = 0; r < 16; r++)
                v[r] = L1 ? acc[i][j][r] * l1v[j] : acc[i][j][r];
        };
        auto store = [&](int b, const float (&v)[16]) {
            const __amdgpu_buffer_rsrc_t rs = tile_rsrc(b / TJ);
#pragma unroll
            for (int r = 0; r < 16; r++)
                __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(v[r]), rs,
                                                      lane_off[b % TJ] + ((r / 4) * 8 + (r % 4)) * (int)ld_bytes, 0,
                                                      0);
        };
        constexpr int NB = 4 * TJ; // batches per wave
        if constexpr (ACC) {
            constexpr int AHEAD = 3;
            float o[AHEAD][16];
            auto load = [&](int b, float (&dst)[16]) {
                const __amdgpu_buffer_rsrc_t rs = tile_rsrc(b / TJ);
#pragma unroll
                for (int r = 0; r < 16; r++)
                    dst[r] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(
                        rs, lane_off[b % TJ] + ((r / 4) * 8 + (r % 4)) * (int)ld_bytes, 0, 0));
            };
#pragma unroll
            for (int b = 0; b < AHEAD; b++)
                load(b, o[b]);
#pragma unroll
            for (int b = 0; b < NB; b++) {
                float v[16];
                batch(b, v);
#pragma unroll
                for (int r = 0; r < 16; r++)
                    v[r] += o[b % AHEAD][r];
                store(b, v);
                if (b + AHEAD < NB)
                    load(b + AHEAD, o[b % AHEAD]);
                __builtin_amdgcn_sched_barrier(0);
            }
        } else {
#pragma unroll
            for (int i = 0; i < 4; i++) {
                const int rows_i = min(32, max(0, rows_ok - i * 32));
                const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
                    (void *)uniform(dblock + (int64_t)i * 32 * ld_bytes), 0,
                    __builtin_amdgcn_readfirstlane(rows_i * (int)ld_bytes), BUF_DWORD3);
#pragma unroll
                for (int j = 0; j < TJ; j++) {
                    float v[16];
#pragma unroll
                    for (int r = 0; r < 16; r++)
                        v[r] = L1 ? acc[i][j][r] * l1v[j] : acc[i][j][r];
#pragma unroll
                    for (int r = 0; r < 16; r++)
                        __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(v[r]), rs,
                                                              lane_off[j] + ((r / 4) * 8 + (r % 4)) * (int)ld_bytes,
                                                              0, 0);
                }
            }
        }
    } else {
#pragma unroll
        for (int part = 0; part < 128 / EPI_ROWS; part++) {
#pragma unroll
            for (int ii = 0; ii < EPI_ROWS / 32; ii++) {
                const int i = part * (EPI_ROWS / 32) + ii;
#pragma unroll
                for (int j = 0; j < TJ; j++) {
#pragma unroll
                    for (int q = 0; q < 4; q++) {
                        // Rows ii*32 + q*8 + hk*4 + 0..3 of column j*32 + l32, as
                        // two row pairs: one dword per pair (low half the even row).
                        float v[4];
#pragma unroll
                        for (int t = 0; t < 4; t++)
                            v[t] = L1 ? acc[i][j][4 * q + t] * l1v[j] : acc[i][j][4 * q + t];
                        const int rp = ii * 16 + q * 4 + hk * 2;
                        const int col = j * 32 + l32;
                        // 16-byte chunk c of a row pair sits at chunk c ^ ((c >> 3) & 1)
                        const int cs = col ^ (((col >> 5) & 1) << 2);
                        *reinterpret_cast<uint32_t *>(ep + rp * RPB + cs * 4) = pack_bf16x2(v[0], v[1]);
                        *reinterpret_cast<uint32_t *>(ep + (rp + 1) * RPB + cs * 4) = pack_bf16x2(v[2], v[3]);
                    }
                }
            }
            __builtin_amdgcn_s_waitcnt(0xc07f); // lgkmcnt(0): this wave's LDS writes done
            __builtin_amdgcn_wave_barrier();
            // a lane takes 8 columns of one row pair: 32 bytes of pairs -> 16 bytes of each row
            constexpr int NRD = EPI_ROWS / 2 / RPI; // read-backs per lane
            const int flip = (lc >> 2) & 1;         // chunks 2 lc and 2 lc + 1, swizzled as written
            // low halves (the even row) and high halves (the odd row) of two pair words
            auto unpair = [](const uint4 &x, const uint4 &y, uint4 &ev, uint4 &od) {
                const uint32_t w[8] = {x.x, x.y, x.z, x.w, y.x, y.y, y.z, y.w};
                uint32_t *e4 = &ev.x, *o4 = &od.x;
#pragma unroll
                for (int k = 0; k < 4; k++) {
                    e4[k] = __builtin_amdgcn_perm(w[2 * k + 1], w[2 * k], 0x05040100u);
                    o4[k] = __builtin_amdgcn_perm(w[2 * k + 1], w[2 * k], 0x07060302u);
                }
            };
            if (block_full) {
                // The whole block inside D: every LDS read first, then the
                // stores, in one straight-line sequence with no per-row tests.
                uint4 xs[NRD], ys[NRD];
#pragma unroll
                for (int t = 0; t < NRD; t++) {
                    const uint8_t *src = ep + (t * RPI + lr) * RPB;
                    xs[t] = *reinterpret_cast<const uint4 *>(src + ((2 * lc) ^ flip) * 16);
                    ys[t] = *reinterpret_cast<const uint4 *>(src + ((2 * lc + 1) ^ flip) * 16);
                }
                uint8_t *dst = dwave + (int64_t)(part * EPI_ROWS + 2 * lr) * ld_bytes;
#pragma unroll
                for (int t = 0; t < NRD; t++) {
                    uint4 ev, od;
                    unpair(xs[t], ys[t], ev, od);
                    *reinterpret_cast<uint4 *>(dst) = ev;
                    *reinterpret_cast<uint4 *>(dst + ld_bytes) = od;
                    dst += 2 * RPI * ld_bytes;
                }
            } else {
#pragma unroll
            for (int rr = 0; rr < EPI_ROWS / 2; rr += RPI) {
                const int rp = rr + lr;
                const uint4 x = *reinterpret_cast<const uint4 *>(ep + rp * RPB + ((2 * lc) ^ flip) * 16);
                const uint4 y = *reinterpret_cast<const uint4 *>(ep + rp * RPB + ((2 * lc + 1) ^ flip) * 16);
                uint4 ev, od;
                unpair(x, y, ev, od);
#pragma unroll
                for (int s = 0; s < 2; s++) {
                    const int row_l = part * EPI_ROWS + 2 * rp + s; // row within the wave's 128
                    const uint4 v = s ? od : ev;
                    uint8_t *dst = dwave + row_l * ld_bytes;
                    if (row_l >= rows_ok || !col_ok)
                        continue;
                    if (full) {
                        *reinterpret_cast<uint4 *>(dst) = v;
                    } else {
                        uint32_t w4[4] = {v.x, v.y, v.z, v.w};
                        for (int e = 0; e < 8 && col0 + e < N; e++)
                            reinterpret_cast<uint16_t *>(dst)[e] = (uint16_t)(w4[e / 2] >> (16 * (e & 1)));
                    }
                }
            }
            }
            __builtin_amdgcn_s_waitcnt(0xc07f);
            __builtin_amdgcn_wave_barrier();
        }
    }
}

template <int MODE, int AG, int BG, bool OUT_BF16, int GK, int AF = FMT_E4M3, bool ACC = false>
static int launch_one(const GemmArgs &p, int64_t grid, hipStream_t st)
{
    auto kern = gemm_fp8_kernel<MODE, AG, BG, OUT_BF16, GK, AF, ACC>;
    // FP32 output: the epilogue's buffer offsets stay below 2^31 for rows up to 2^23 elements
    if (!OUT_BF16 && p.ldd >= ((int64_t)1 << 23))
        return set_error(FGB_EUNSUPPORTED, "gemm: FP32 output rows (ldd) must be shorter than 2^23 elements");
    // The LDS limit is raised once per instantiation and device (a process may
    // use several devices); devices beyond the table set it on every call.
    // Threads that launch at once may both set it, which is harmless.
    static std::atomic<bool> attr_set[64] = {};
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess)
        dev = -1;
    const bool cached = dev >= 0 && dev < 64;
    if (!cached || !attr_set[dev].load(std::memory_order_acquire)) {
        hipError_t e = hipFuncSetAttribute((const void *)kern, hipFuncAttributeMaxDynamicSharedMemorySize, LDS_BYTES);
        if (e != hipSuccess)
            return set_error(FGB_EHIP, "gemm: hipFuncSetAttribute failed: %s", hipGetErrorString(e));
        if (cached)
            attr_set[dev].store(true, std::memory_order_release);
    }
    kern<<<(unsigned)grid, Waves<MODE, GK>::NW * 64, LDS_BYTES, st>>>(p);
    FGB_LAUNCHED("gemm_fp8_kernel");
    return FGB_OK;
}

// The instantiation for the output type and, with FP32 output in the dense
// and K-grouped forms, accumulation into D.
template <int MODE, int AG, int BG, int GK, int AF = FMT_E4M3>
static int launch_out(bool bf16, const GemmArgs &p, int64_t grid, hipStream_t st)
{
    if (bf16)
        return launch_one<MODE, AG, BG, true, GK, AF>(p, grid, st);
    if constexpr (GK == GK_NONE || GK == GK_K) {
        if (p.accumulate)
            return launch_one<MODE, AG, BG, false, GK, AF, true>(p, grid, st);
    }
    return launch_one<MODE, AG, BG, false, GK, AF>(p, grid, st);
}

template <int MODE, int GK>
static int dispatch_mode(int ag, int bg, bool bf16, const GemmArgs &p, int64_t grid, hipStream_t st)
{
    if constexpr (GK == GK_M || GK == GK_MM) {
        if (ag == AG_ROW128 && bg == BG_BLOCK)
            return launch_out<MODE, AG_ROW128, BG_BLOCK, GK>(bf16, p, grid, st);
    } else if constexpr (GK == GK_K) {
        if (ag == AG_ROW128 && bg == BG_ROW128)
            return launch_out<MODE, AG_ROW128, BG_ROW128, GK_K>(bf16, p, grid, st);
    } else {
        if (ag == AG_ROW128 && bg == BG_BLOCK)
            return launch_out<MODE, AG_ROW128, BG_BLOCK, GK_NONE>(bf16, p, grid, st);
        if (ag == AG_ROW128 && bg == BG_ROW128)
            return launch_out<MODE, AG_ROW128, BG_ROW128, GK_NONE>(bf16, p, grid, st);
        if (ag == AG_ROW32 && bg == BG_ROW32)
            return launch_out<MODE, AG_ROW32, BG_ROW32, GK_NONE>(bf16, p, grid, st);
    }
    return set_error(FGB_EUNSUPPORTED, "gemm: unsupported scale granularity pair (%d, %d)", ag, bg);
}

template <int GK>
static int dispatch(int mode, int ag, int bg, bool bf16, const GemmArgs &p, int64_t grid, hipStream_t st)
{
    if (mode == FGB_GEMM_FAST)
        return dispatch_mode<MODE_FAST, GK>(ag, bg, bf16, p, grid, st);
    return dispatch_mode<MODE_EXACT, GK>(ag, bg, bf16, p, grid, st);
}

// E5M2 A operand (gradients): dense, 1x128 A scales, 128x128 or 1x128 B scales.
template <int MODE>
static int dispatch_e5m2_mode(int bg, bool bf16, const GemmArgs &p, int64_t grid, hipStream_t st)
{
    if (bg == BG_BLOCK)
        return launch_out<MODE, AG_ROW128, BG_BLOCK, GK_NONE, FMT_E5M2>(bf16, p, grid, st);
    return launch_out<MODE, AG_ROW128, BG_ROW128, GK_NONE, FMT_E5M2>(bf16, p, grid, st);
}

} // namespace fgb

using namespace fgb;

extern "C" int fp8_block_gemm_fmt(const uint8_t *a, const uint8_t *sa, int a_gran, int a_fmt, const uint8_t *b,
                                  const uint8_t *sb, int b_gran, int b_fmt, const float *b_l1, int64_t g1, int64_t M,
                                  int64_t N, int64_t K, int64_t lda, int64_t ldb, void *d, int d_dtype, int64_t ldd,
                                  int accumulate, int mode, void *stream)
{
    clear_error();
    FGB_REQUIRE(a_fmt == FGB_E4M3 || a_fmt == FGB_E5M2, FGB_EUNSUPPORTED,
                "fp8_block_gemm: a_fmt must be FGB_E4M3 or FGB_E5M2");
    FGB_REQUIRE(b_fmt == FGB_E4M3, FGB_EUNSUPPORTED, "fp8_block_gemm: b_fmt must be FGB_E4M3");
    FGB_REQUIRE(a_fmt == FGB_E4M3 || (a_gran == FGB_ROW1x128 && b_gran != FGB_ROW1x32 && !b_l1), FGB_EUNSUPPORTED,
                "fp8_block_gemm: an E5M2 A needs 1x128 A scales, 128x128 or 1x128 B scales and no b_l1");
    FGB_REQUIRE(M >= 0 && N >= 0 && K >= 0 && K % 128 == 0, FGB_EINVAL,
                "fp8_block_gemm: need M, N >= 0 and K a multiple of 128 (M=%lld N=%lld K=%lld)",
                (long long)M, (long long)N, (long long)K);
    // Empty D: nothing to write (the operands may be empty tensors without storage).
    if (M == 0 || N == 0)
        return FGB_OK;
    FGB_REQUIRE(d && (K == 0 || (a && sa && b && sb)), FGB_EINVAL, "fp8_block_gemm: null pointer");
    // (with K = 0 no operand is read: their layouts are not checked)
    FGB_REQUIRE(K == 0 || (lda >= K && ldb >= K && lda % 16 == 0 && ldb % 16 == 0), FGB_EINVAL,
                "fp8_block_gemm: lda/ldb must be >= K and multiples of 16");
    FGB_REQUIRE(K == 0 || (256 * lda < (1ll << 32) && 256 * ldb < (1ll << 32)), FGB_EINVAL,
                "fp8_block_gemm: lda/ldb too large");
    FGB_REQUIRE(ldd >= N, FGB_EINVAL, "fp8_block_gemm: ldd must be >= N");
    FGB_REQUIRE(K == 0 || (aligned16(a) && aligned16(b)), FGB_EINVAL,
                "fp8_block_gemm: a and b must be 16-byte aligned");
    FGB_REQUIRE(d_dtype == FGB_F32 || d_dtype == FGB_BF16, FGB_EUNSUPPORTED,
                "fp8_block_gemm: d_dtype must be FGB_F32 or FGB_BF16");
    FGB_REQUIRE(mode == FGB_GEMM_EXACT || mode == FGB_GEMM_FAST, FGB_EUNSUPPORTED,
                "fp8_block_gemm: mode must be FGB_GEMM_EXACT or FGB_GEMM_FAST");
    FGB_REQUIRE(!(accumulate && d_dtype != FGB_F32), FGB_EUNSUPPORTED,
                "fp8_block_gemm: accumulate needs FP32 output");
    int ag, bg;
    if (a_gran == FGB_ROW1x128)
        ag = AG_ROW128;
    else if (a_gran == FGB_ROW1x32)
        ag = AG_ROW32;
    else
        return set_error(FGB_EUNSUPPORTED, "fp8_block_gemm: a_gran must be FGB_ROW1x128 or FGB_ROW1x32");
    if (b_gran == FGB_BLOCK128)
        bg = BG_BLOCK;
    else if (b_gran == FGB_ROW1x128)
        bg = BG_ROW128;
    else if (b_gran == FGB_ROW1x32)
        bg = BG_ROW32;
    else
        return set_error(FGB_EUNSUPPORTED, "fp8_block_gemm: unknown b_gran");
    FGB_REQUIRE((ag == AG_ROW32) == (bg == BG_ROW32), FGB_EUNSUPPORTED,
                "fp8_block_gemm: FGB_ROW1x32 scales must be used on both operands");
    FGB_REQUIRE(!b_l1 || b_gran == FGB_ROW1x32, FGB_EUNSUPPORTED,
                "fp8_block_gemm: b_l1 needs 1x32 B scales (the level-2 scales of the two-level format)");
    FGB_REQUIRE(!b_l1 || (g1 > 0 && K <= g1), FGB_EUNSUPPORTED,
                "fp8_block_gemm: b_l1 needs K <= g1 (one level-1 group along K)");
    if (ag == AG_ROW32 && K > 0)
        FGB_REQUIRE(((uintptr_t)sa & 3) == 0 && ((uintptr_t)sb & 3) == 0, FGB_EINVAL,
                    "fp8_block_gemm: 1x32 scale tensors must be 4-byte aligned");
    GemmArgs p{};
    p.a = a; p.sa = sa; p.b = b; p.sb = sb; p.l1 = b_l1; p.d = d;
    p.M = M; p.N = N; p.K = K; p.lda = lda; p.ldb = ldb; p.ldd = ldd;
    p.accumulate = accumulate;
    p.tiles_n = (int)((N + BN - 1) / BN);
    int64_t tiles = ((M + BM - 1) / BM) * p.tiles_n;
    FGB_REQUIRE(tiles < (1ll << 31), FGB_EINVAL, "fp8_block_gemm: too many tiles");
    if (a_fmt == FGB_E5M2)
        return mode == FGB_GEMM_FAST
                   ? dispatch_e5m2_mode<MODE_FAST>(bg, d_dtype == FGB_BF16, p, tiles, (hipStream_t)stream)
                   : dispatch_e5m2_mode<MODE_EXACT>(bg, d_dtype == FGB_BF16, p, tiles, (hipStream_t)stream);
    return dispatch<GK_NONE>(mode, ag, bg, d_dtype == FGB_BF16, p, tiles, (hipStream_t)stream);
}

extern "C" int fp8_block_gemm(const uint8_t *a, const uint8_t *sa, int a_gran, const uint8_t *b, const uint8_t *sb,
                              int b_gran, const float *b_l1, int64_t g1, int64_t M, int64_t N, int64_t K, int64_t lda,
                              int64_t ldb, void *d, int d_dtype, int64_t ldd, int accumulate, int mode,
                              void *workspace, size_t ws_bytes, void *stream)
{
    (void)workspace;
    (void)ws_bytes;
    return fp8_block_gemm_fmt(a, sa, a_gran, FGB_E4M3, b, sb, b_gran, FGB_E4M3, b_l1, g1, M, N, K, lda, ldb, d,
                              d_dtype, ldd, accumulate, mode, stream);
}

extern "C" int fp8_grouped_gemm(const uint8_t *a, const uint8_t *sa, const uint8_t *b,
                                const uint8_t *sb, const int32_t *group_offsets, int G,
                                int64_t M_cap, int64_t N, int64_t K, void *d, int d_dtype,
                                int mode, void *stream)
{
    clear_error();
    FGB_REQUIRE(a && sa && b && sb && d && group_offsets, FGB_EINVAL, "fp8_grouped_gemm: null pointer");
    FGB_REQUIRE(G >= 1 && G <= 1024, FGB_EINVAL, "fp8_grouped_gemm: G must be in [1, 1024]");
    FGB_REQUIRE(M_cap >= 0 && N > 0 && K > 0 && K % 128 == 0, FGB_EINVAL,
                "fp8_grouped_gemm: need N > 0 and K a positive multiple of 128");
    FGB_REQUIRE(256 * K < (1ll << 32), FGB_EINVAL, "fp8_grouped_gemm: K too large");
    FGB_REQUIRE(aligned16(a) && aligned16(b), FGB_EINVAL, "fp8_grouped_gemm: a and b must be 16-byte aligned");
    FGB_REQUIRE(d_dtype == FGB_F32 || d_dtype == FGB_BF16, FGB_EUNSUPPORTED,
                "fp8_grouped_gemm: d_dtype must be FGB_F32 or FGB_BF16");
    FGB_REQUIRE(mode == FGB_GEMM_EXACT || mode == FGB_GEMM_FAST, FGB_EUNSUPPORTED,
                "fp8_grouped_gemm: mode must be FGB_GEMM_EXACT or FGB_GEMM_FAST");
    if (M_cap == 0)
        return FGB_OK;
    GemmArgs p{};
    p.a = a; p.sa = sa; p.b = b; p.sb = sb; p.l1 = nullptr; p.d = d;
    p.M = M_cap; p.N = N; p.K = K; p.lda = K; p.ldb = K; p.ldd = N;
    p.accumulate = 0;
    p.tiles_n = (int)((N + BN - 1) / BN);
    p.offs = group_offsets;
    p.G = G;
    p.b_stride = N * K;
    p.sb_stride = ((N + 127) / 128) * (K / 128);
    // sum over experts of ceil(rows_e / BM) <= ceil(M_cap / BM) + G
    int64_t tiles = ((M_cap + BM - 1) / BM + G) * p.tiles_n;
    FGB_REQUIRE(tiles < (1ll << 31), FGB_EINVAL, "fp8_grouped_gemm: too many tiles");
    return dispatch<GK_M>(mode, AG_ROW128, BG_BLOCK, d_dtype == FGB_BF16, p, tiles, (hipStream_t)stream);
}

extern "C" int fp8_grouped_gemm_masked(const uint8_t *a, const uint8_t *sa, const uint8_t *b, const uint8_t *sb,
                                       const int32_t *masked_m, int G, int64_t M_max, int64_t N, int64_t K, void *d,
                                       int d_dtype, int mode, void *stream)
{
    clear_error();
    FGB_REQUIRE(a && sa && b && sb && d && masked_m, FGB_EINVAL, "fp8_grouped_gemm_masked: null pointer");
    FGB_REQUIRE(G >= 1 && G <= 1024, FGB_EINVAL, "fp8_grouped_gemm_masked: G must be in [1, 1024]");
    FGB_REQUIRE(M_max > 0 && N > 0 && K > 0 && K % 128 == 0, FGB_EINVAL,
                "fp8_grouped_gemm_masked: need M_max, N > 0 and K a positive multiple of 128");
    FGB_REQUIRE(256 * K < (1ll << 32), FGB_EINVAL, "fp8_grouped_gemm_masked: K too large");
    FGB_REQUIRE(aligned16(a) && aligned16(b), FGB_EINVAL, "fp8_grouped_gemm_masked: a and b must be 16-byte aligned");
    FGB_REQUIRE(d_dtype == FGB_F32 || d_dtype == FGB_BF16, FGB_EUNSUPPORTED,
                "fp8_grouped_gemm_masked: d_dtype must be FGB_F32 or FGB_BF16");
    FGB_REQUIRE(mode == FGB_GEMM_EXACT || mode == FGB_GEMM_FAST, FGB_EUNSUPPORTED,
                "fp8_grouped_gemm_masked: mode must be FGB_GEMM_EXACT or FGB_GEMM_FAST");
    GemmArgs p{};
    p.a = a; p.sa = sa; p.b = b; p.sb = sb; p.l1 = nullptr; p.d = d;
    p.M = (int64_t)G * M_max; p.N = N; p.K = K; p.lda = K; p.ldb = K; p.ldd = N;
    p.accumulate = 0;
    p.tiles_n = (int)((N + BN - 1) / BN);
    p.G = G;
    p.b_stride = N * K;
    p.sb_stride = ((N + 127) / 128) * (K / 128);
    p.masked_m = masked_m;
    p.m_max = M_max;
    const int64_t tiles = (int64_t)G * ((M_max + BM - 1) / BM) * p.tiles_n;
    FGB_REQUIRE(tiles < (1ll << 31), FGB_EINVAL, "fp8_grouped_gemm_masked: too many tiles");
    return dispatch<GK_MM>(mode, AG_ROW128, BG_BLOCK, d_dtype == FGB_BF16, p, tiles, (hipStream_t)stream);
}

extern "C" int fp8_kgrouped_gemm(const uint8_t *a, const uint8_t *sa, const uint8_t *b, const uint8_t *sb,
                                 const int32_t *k_offsets, int G, int64_t M, int64_t N, int64_t K_cap, void *d,
                                 int d_dtype, int accumulate, int mode, void *stream)
{
    clear_error();
    FGB_REQUIRE(a && sa && b && sb && d && k_offsets, FGB_EINVAL, "fp8_kgrouped_gemm: null pointer");
    FGB_REQUIRE(G >= 1 && G <= 1024, FGB_EINVAL, "fp8_kgrouped_gemm: G must be in [1, 1024]");
    FGB_REQUIRE(M > 0 && N > 0 && K_cap > 0 && K_cap % 128 == 0, FGB_EINVAL,
                "fp8_kgrouped_gemm: need M, N > 0 and K_cap a positive multiple of 128");
    FGB_REQUIRE(256 * K_cap < (1ll << 32), FGB_EINVAL, "fp8_kgrouped_gemm: K_cap too large");
    FGB_REQUIRE(aligned16(a) && aligned16(b), FGB_EINVAL, "fp8_kgrouped_gemm: a and b must be 16-byte aligned");
    FGB_REQUIRE(d_dtype == FGB_F32 || d_dtype == FGB_BF16, FGB_EUNSUPPORTED,
                "fp8_kgrouped_gemm: d_dtype must be FGB_F32 or FGB_BF16");
    FGB_REQUIRE(mode == FGB_GEMM_EXACT || mode == FGB_GEMM_FAST, FGB_EUNSUPPORTED,
                "fp8_kgrouped_gemm: mode must be FGB_GEMM_EXACT or FGB_GEMM_FAST");
    FGB_REQUIRE(!(accumulate && d_dtype != FGB_F32), FGB_EUNSUPPORTED, "fp8_kgrouped_gemm: accumulate needs FP32 output");
    GemmArgs p{};
    p.a = a; p.sa = sa; p.b = b; p.sb = sb; p.l1 = nullptr; p.d = d;
    p.M = M; p.N = N; p.K = K_cap; p.lda = K_cap; p.ldb = K_cap; p.ldd = N;
    p.accumulate = accumulate;
    p.tiles_n = (int)((N + BN - 1) / BN);
    p.G = G;
    p.koffs = k_offsets;
    p.d_stride = M * N;
    const int64_t tiles = ((M + BM - 1) / BM) * p.tiles_n * G;
    FGB_REQUIRE(tiles < (1ll << 31), FGB_EINVAL, "fp8_kgrouped_gemm: too many tiles");
    return dispatch<GK_K>(mode, AG_ROW128, BG_ROW128, d_dtype == FGB_BF16, p, tiles, (hipStream_t)stream);
}
