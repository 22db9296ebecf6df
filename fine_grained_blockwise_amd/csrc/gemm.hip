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
// Tiling: 256x256 output tile per workgroup of 4 waves (each wave 128x128 =
// 4x4 tiles of 32x32), K step 128.  A and B tiles (256 rows x 128 bytes) are
// copied HBM -> LDS with global_load_lds_dwordx4 into a double buffer
// (2 x 64 KB).  LDS rows are 128 bytes with the 16-byte chunk index
// XOR-swizzled by f(row) = (row ^ row>>3) & 7 so the operand reads of 32
// consecutive rows hit distinct banks.  All fragment reads of a K step are
// issued before the next step's copies, so no wait on those copies ever
// stands in front of an LDS read.  Tiles are mapped to XCDs in contiguous
// ranges so neighbouring tiles share an XCD's L2.
//
// Fragment layout, per lane (row r = lane%32 of a 32-row tile, half h =
// lane/32), per 128-byte K step: the four 16-byte chunks h, h+2, h+4, h+6.
//   FAST : 64-wide sub-step s uses chunks 4s+h (bytes 0-15, hardware K block
//          0) and 4s+2+h (bytes 16-31, block 1); the hardware takes block
//          b's scale from lane r + 32b, so lane half h supplies the scale of
//          logical 32-block 2s+h.
//   EXACT: 32-wide pair p uses chunk 2p+h; its bytes 0-7 feed the bf16 MFMA
//          of sub-step 2p and bytes 8-15 that of sub-step 2p+1.
#include "fgb_internal.h"

namespace fgb {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));

constexpr int BM = 256, BN = 256, BK = 128;
constexpr int TILE_BYTES = BM * BK; // one operand tile: 32 KB
constexpr int STAGE_BYTES = 2 * TILE_BYTES;
constexpr int LDS_BYTES = 2 * STAGE_BYTES; // double buffer: 128 KB

enum { MODE_EXACT = 0, MODE_FAST = 1 };
enum { AG_ROW128 = 0, AG_ROW32 = 1 };
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
    int64_t b_stride, sb_stride; // grouped: per-expert B / SB strides
};

// Contiguous tile ranges per XCD: workgroup b runs on XCD b % 8.
__device__ __forceinline__ int64_t xcd_remap(int64_t b, int64_t nb)
{
    int64_t x = b & 7, i = b >> 3, q = nb >> 3, r = nb & 7;
    return x < r ? x * (q + 1) + i : r * (q + 1) + (x - r) * q + i;
}

__device__ __forceinline__ int swz(int row) { return (row ^ (row >> 3)) & 7; }

// 16 E4M3 codes -> two 8-element bf16 operands, each value times 2^e (sc = 2^e).
__device__ __forceinline__ void cvt16_bf16(uint4 w, float sc, v8bf &lo, v8bf &hi)
{
    uint4 a, b;
    a.x = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w.x, sc, false));
    a.y = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w.x, sc, true));
    a.z = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w.y, sc, false));
    a.w = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w.y, sc, true));
    b.x = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w.z, sc, false));
    b.y = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w.z, sc, true));
    b.z = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w.w, sc, false));
    b.w = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w.w, sc, true));
    lo = __builtin_bit_cast(v8bf, a);
    hi = __builtin_bit_cast(v8bf, b);
}

// Scale byte -> the fp32 whose exponent field it is (byte 0 is taken as 1).
__device__ __forceinline__ float scale_f32(uint32_t byte) { return __uint_as_float(max(byte, 1u) << 23); }

__device__ __forceinline__ v8i cat(uint4 x, uint4 y)
{
    return (v8i){(int)x.x, (int)x.y, (int)x.z, (int)x.w, (int)y.x, (int)y.y, (int)y.z, (int)y.w};
}

template <int OPA, int OPB>
__device__ __forceinline__ v16f mfma_scaled(v8i a, v8i b, v16f c, uint32_t sa, uint32_t sb)
{
    return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, OPA, (int)sa, OPB, (int)sb);
}

template <int MODE, int AG, int BG, bool OUT_BF16, bool GROUPED>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1))) void
gemm_fp8_kernel(GemmArgs p)
{
    extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wm = wave >> 1, wn = wave & 1;
    const int l32 = lane & 31, hk = lane >> 5;
    const int64_t K = p.K, nk = K / BK;
    const int64_t N = p.N;

    // ---- tile -> (m0, n0) ------------------------------------------------
    int64_t tile = xcd_remap(blockIdx.x, gridDim.x);
    int64_t m0 = 0, m_end = 0, tn;
    const uint8_t *B = p.b, *SB = p.sb;
    if constexpr (!GROUPED) {
        m0 = (tile / p.tiles_n) * BM;
        tn = tile % p.tiles_n;
        m_end = p.M;
    } else {
        int64_t tm = tile / p.tiles_n;
        tn = tile % p.tiles_n;
        int e = -1;
        int64_t base = 0;
        for (int g = 0; g < p.G; g++) {
            int64_t lo = p.offs[g], hi = p.offs[g + 1];
            int64_t nt = (hi - lo + BM - 1) / BM;
            if (tm >= base && tm < base + nt) {
                e = g;
                m0 = lo + (tm - base) * BM;
                m_end = hi;
            }
            base += nt;
        }
        if (e < 0)
            return; // past the last expert tile (uniform per workgroup)
        B += (int64_t)e * p.b_stride;
        SB += (int64_t)e * p.sb_stride;
    }
    const int64_t n0 = tn * BN;

    // ---- global -> LDS copy plan -----------------------------------------
    // Operand tile = 32 groups of 8 rows (1 KB each); wave w copies groups
    // w*8 .. w*8+7 of A and of B.  Lane l lands at LDS offset l*16 of its
    // group: row g*8 + l/8, physical chunk l%8, which holds logical chunk
    // (l%8) ^ swz(row).  Rows past the end re-read the last valid row.
    const uint8_t *a_base = p.a + m0 * p.lda;
    const uint8_t *b_base = B + n0 * p.ldb;
    uint32_t a_off[8], b_off[8];
#pragma unroll
    for (int i = 0; i < 8; i++) {
        int r = (wave * 8 + i) * 8 + (lane >> 3);
        int chunk = (lane & 7) ^ swz(r);
        int64_t ar = m0 + r < m_end ? r : m_end - 1 - m0;
        int64_t br = n0 + r < N ? r : N - 1 - n0;
        a_off[i] = (uint32_t)(ar * p.lda + chunk * 16);
        b_off[i] = (uint32_t)(br * p.ldb + chunk * 16);
    }
    auto issue_copy = [&](int stage, int64_t ks) {
        uint8_t *sa_ = smem + stage * STAGE_BYTES;
        uint8_t *sb_ = sa_ + TILE_BYTES;
#pragma unroll
        for (int i = 0; i < 8; i++) {
            __builtin_amdgcn_global_load_lds(a_base + a_off[i] + ks * BK,
                                             (__attribute__((address_space(3))) void *)(sa_ + (wave * 8 + i) * 1024), 16, 0, 0);
            __builtin_amdgcn_global_load_lds(b_base + b_off[i] + ks * BK,
                                             (__attribute__((address_space(3))) void *)(sb_ + (wave * 8 + i) * 1024), 16, 0, 0);
        }
    };

    // ---- scale plan ----------------------------------------------------------
    // Per K step and operand tile t, a lane needs the scale(s) of its row of
    // that tile: one byte (128-element groups) or the four consecutive bytes
    // of the step's 32-element blocks, read as one dword.  They are loaded one
    // step ahead into raw registers and decoded after the next barrier.
    constexpr bool A32 = AG == AG_ROW32, B32 = BG == BG_ROW32;
    const int64_t sa_row = A32 ? K / 32 : K / 128;
    const int64_t sb_row = B32 ? K / 32 : K / 128;
    const uint8_t *sa_base = p.sa + m0 * sa_row;
    uint32_t sa_off[4];
#pragma unroll
    for (int t = 0; t < 4; t++) {
        int64_t r = wm * 128 + t * 32 + l32;
        r = m0 + r < m_end ? r : m_end - 1 - m0;
        sa_off[t] = (uint32_t)(r * sa_row);
    }
    const uint8_t *sb_base;
    uint32_t sb_off[4];
    if constexpr (BG == BG_BLOCK) {
        // a wave's 128 columns lie in one 128-row block of B; past the last
        // block (ragged N) clamp to it -- those columns are never stored
        int64_t nb = (n0 + wn * 128) / 128, nb_last = (N - 1) / 128;
        sb_base = SB + (nb < nb_last ? nb : nb_last) * (K / 128);
#pragma unroll
        for (int t = 0; t < 4; t++)
            sb_off[t] = 0;
    } else {
        sb_base = SB + n0 * sb_row;
#pragma unroll
        for (int t = 0; t < 4; t++) {
            int64_t c = wn * 128 + t * 32 + l32;
            c = n0 + c < N ? c : N - 1 - n0;
            sb_off[t] = (uint32_t)(c * sb_row);
        }
    }
    uint32_t raw_a[4], raw_b[4];
    auto load_scales = [&](int64_t ks) {
#pragma unroll
        for (int t = 0; t < 4; t++) {
            raw_a[t] = A32 ? *reinterpret_cast<const uint32_t *>(sa_base + sa_off[t] + ks * 4)
                           : (uint32_t)sa_base[sa_off[t] + ks];
            if constexpr (BG == BG_BLOCK)
                raw_b[t] = t == 0 ? (uint32_t)sb_base[ks] : 0u;
            else
                raw_b[t] = B32 ? *reinterpret_cast<const uint32_t *>(sb_base + sb_off[t] + ks * 4)
                               : (uint32_t)sb_base[sb_off[t] + ks];
        }
    };

    // ---- fragment addressing ---------------------------------------------------
    // operand row r = t*32 + lane%32 within the wave's 128 rows (the wave's
    // 128-row offset leaves swz unchanged); chunk 2q + h.
    int frag_off[4][4];
#pragma unroll
    for (int t = 0; t < 4; t++) {
        int r = t * 32 + l32;
#pragma unroll
        for (int q = 0; q < 4; q++)
            frag_off[t][q] = r * 128 + (((2 * q + hk) ^ swz(r)) * 16);
    }

    v16f acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; i++)
#pragma unroll
        for (int j = 0; j < 4; j++)
            acc[i][j] = (v16f){0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};

    load_scales(0);
    issue_copy(0, 0);

    for (int64_t ks = 0; ks < nk; ks++) {
        const int cur = (int)(ks & 1);
        __builtin_amdgcn_s_waitcnt(0);
        __syncthreads();
        uint32_t ca[4], cb[4];
#pragma unroll
        for (int t = 0; t < 4; t++) {
            ca[t] = raw_a[t];
            cb[t] = raw_b[t];
        }
        const uint8_t *la = smem + cur * STAGE_BYTES + wm * 128 * 128;
        const uint8_t *lb = smem + cur * STAGE_BYTES + TILE_BYTES + wn * 128 * 128;
        uint4 fa[4][4], fb[4][4];
#pragma unroll
        for (int q = 0; q < 4; q++)
#pragma unroll
            for (int t = 0; t < 4; t++) {
                fa[t][q] = *reinterpret_cast<const uint4 *>(la + frag_off[t][q]);
                fb[t][q] = *reinterpret_cast<const uint4 *>(lb + frag_off[t][q]);
            }
        if (ks + 1 < nk) {
            load_scales(ks + 1);
            issue_copy(cur ^ 1, ks + 1);
        }
        if constexpr (MODE == MODE_FAST) {
#pragma unroll
            for (int s = 0; s < 2; s++) {
                // scale words: byte t = tile t's scale for this lane's 32-block
                uint32_t wa = 0, wb = 0;
                const int sh = A32 ? 8 * (2 * s + hk) : 0;
#pragma unroll
                for (int t = 0; t < 4; t++)
                    wa |= ((ca[t] >> sh) & 0xFFu) << (8 * t);
                if constexpr (BG == BG_BLOCK) {
                    wb = cb[0];
                } else {
                    const int shb = B32 ? 8 * (2 * s + hk) : 0;
#pragma unroll
                    for (int t = 0; t < 4; t++)
                        wb |= ((cb[t] >> shb) & 0xFFu) << (8 * t);
                }
                v8i av[4], bv[4];
#pragma unroll
                for (int t = 0; t < 4; t++) {
                    av[t] = cat(fa[t][2 * s], fa[t][2 * s + 1]);
                    bv[t] = cat(fb[t][2 * s], fb[t][2 * s + 1]);
                }
#define FGB_J(I, J) acc[I][J] = mfma_scaled<I, (BG == BG_BLOCK ? 0 : J)>(av[I], bv[J], acc[I][J], wa, wb);
#define FGB_I(I) FGB_J(I, 0) FGB_J(I, 1) FGB_J(I, 2) FGB_J(I, 3)
                FGB_I(0) FGB_I(1) FGB_I(2) FGB_I(3)
#undef FGB_I
#undef FGB_J
            }
        } else {
#pragma unroll
            for (int q = 0; q < 4; q++) {
                v8bf alo[4], ahi[4], blo[4], bhi[4];
#pragma unroll
                for (int t = 0; t < 4; t++) {
                    uint32_t ba = A32 ? (ca[t] >> (8 * q)) & 0xFFu : ca[t];
                    cvt16_bf16(fa[t][q], scale_f32(ba), alo[t], ahi[t]);
                    uint32_t bb = BG == BG_BLOCK ? cb[0] : (B32 ? (cb[t] >> (8 * q)) & 0xFFu : cb[t]);
                    cvt16_bf16(fb[t][q], scale_f32(bb), blo[t], bhi[t]);
                }
#pragma unroll
                for (int i = 0; i < 4; i++)
#pragma unroll
                    for (int j = 0; j < 4; j++) {
                        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(alo[i], blo[j], acc[i][j], 0, 0, 0);
                        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ahi[i], bhi[j], acc[i][j], 0, 0, 0);
                    }
            }
        }
    }

    // ---- epilogue --------------------------------------------------------------
    // 32x32 accumulator layout: lane l, register r -> row (r/4)*8 + (l/32)*4 + r%4,
    // column l%32.
#pragma unroll
    for (int j = 0; j < 4; j++) {
        int64_t col = n0 + wn * 128 + j * 32 + l32;
        if (col >= N)
            continue;
        float l1 = p.l1 ? p.l1[col] : 1.0f;
#pragma unroll
        for (int i = 0; i < 4; i++)
#pragma unroll
            for (int r = 0; r < 16; r++) {
                int64_t row = m0 + wm * 128 + i * 32 + (r / 4) * 8 + hk * 4 + (r % 4);
                if (row >= m_end)
                    continue;
                float v = acc[i][j][r];
                if (p.l1)
                    v *= l1;
                if constexpr (OUT_BF16) {
                    ((uint16_t *)p.d)[row * p.ldd + col] = (uint16_t)bf16_rne(v);
                } else {
                    float *dst = (float *)p.d + row * p.ldd + col;
                    *dst = p.accumulate ? *dst + v : v;
                }
            }
    }
}

template <int MODE, int AG, int BG, bool OUT_BF16, bool GROUPED>
static int launch_one(const GemmArgs &p, int64_t grid, hipStream_t st)
{
    auto kern = gemm_fp8_kernel<MODE, AG, BG, OUT_BF16, GROUPED>;
    static bool attr_set = false; // per instantiation, set once per process
    if (!attr_set) {
        hipError_t e = hipFuncSetAttribute((const void *)kern, hipFuncAttributeMaxDynamicSharedMemorySize, LDS_BYTES);
        if (e != hipSuccess)
            return set_error(FGB_EHIP, "gemm: hipFuncSetAttribute failed: %s", hipGetErrorString(e));
        attr_set = true;
    }
    kern<<<(unsigned)grid, 256, LDS_BYTES, st>>>(p);
    FGB_LAUNCHED("gemm_fp8_kernel");
    return FGB_OK;
}

template <int MODE, bool GROUPED>
static int dispatch_mode(int ag, int bg, bool bf16, const GemmArgs &p, int64_t grid, hipStream_t st)
{
    if (ag == AG_ROW128 && bg == BG_BLOCK)
        return bf16 ? launch_one<MODE, AG_ROW128, BG_BLOCK, true, GROUPED>(p, grid, st)
                    : launch_one<MODE, AG_ROW128, BG_BLOCK, false, GROUPED>(p, grid, st);
    if constexpr (!GROUPED) {
        if (ag == AG_ROW128 && bg == BG_ROW128)
            return bf16 ? launch_one<MODE, AG_ROW128, BG_ROW128, true, false>(p, grid, st)
                        : launch_one<MODE, AG_ROW128, BG_ROW128, false, false>(p, grid, st);
        if (ag == AG_ROW32 && bg == BG_ROW32)
            return bf16 ? launch_one<MODE, AG_ROW32, BG_ROW32, true, false>(p, grid, st)
                        : launch_one<MODE, AG_ROW32, BG_ROW32, false, false>(p, grid, st);
    }
    return set_error(FGB_EUNSUPPORTED, "gemm: unsupported scale granularity pair (%d, %d)", ag, bg);
}

template <bool GROUPED>
static int dispatch(int mode, int ag, int bg, bool bf16, const GemmArgs &p, int64_t grid, hipStream_t st)
{
    if (mode == FGB_GEMM_FAST)
        return dispatch_mode<MODE_FAST, GROUPED>(ag, bg, bf16, p, grid, st);
    return dispatch_mode<MODE_EXACT, GROUPED>(ag, bg, bf16, p, grid, st);
}

} // namespace fgb

using namespace fgb;

extern "C" int fp8_block_gemm(const uint8_t *a, const uint8_t *sa, int a_gran, const uint8_t *b,
                              const uint8_t *sb, int b_gran, const float *b_l1, int64_t g1,
                              int64_t M, int64_t N, int64_t K, int64_t lda, int64_t ldb, void *d,
                              int d_dtype, int64_t ldd, int accumulate, int mode, void *workspace,
                              size_t ws_bytes, void *stream)
{
    (void)workspace;
    (void)ws_bytes;
    clear_error();
    FGB_REQUIRE(a && sa && b && sb && d, FGB_EINVAL, "fp8_block_gemm: null pointer");
    FGB_REQUIRE(M > 0 && N > 0 && K > 0 && K % 128 == 0, FGB_EINVAL,
                "fp8_block_gemm: need M, N > 0 and K a positive multiple of 128 (M=%lld N=%lld K=%lld)",
                (long long)M, (long long)N, (long long)K);
    FGB_REQUIRE(lda >= K && ldb >= K && lda % 16 == 0 && ldb % 16 == 0, FGB_EINVAL,
                "fp8_block_gemm: lda/ldb must be >= K and multiples of 16");
    FGB_REQUIRE(256 * lda < (1ll << 32) && 256 * ldb < (1ll << 32), FGB_EINVAL,
                "fp8_block_gemm: lda/ldb too large");
    FGB_REQUIRE(ldd >= N, FGB_EINVAL, "fp8_block_gemm: ldd must be >= N");
    FGB_REQUIRE(aligned16(a) && aligned16(b), FGB_EINVAL, "fp8_block_gemm: a and b must be 16-byte aligned");
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
    FGB_REQUIRE(!b_l1 || (g1 > 0 && K <= g1), FGB_EUNSUPPORTED,
                "fp8_block_gemm: b_l1 needs K <= g1 (one level-1 group along K)");
    if (ag == AG_ROW32)
        FGB_REQUIRE(((uintptr_t)sa & 3) == 0 && ((uintptr_t)sb & 3) == 0, FGB_EINVAL,
                    "fp8_block_gemm: 1x32 scale tensors must be 4-byte aligned");
    GemmArgs p{};
    p.a = a; p.sa = sa; p.b = b; p.sb = sb; p.l1 = b_l1; p.d = d;
    p.M = M; p.N = N; p.K = K; p.lda = lda; p.ldb = ldb; p.ldd = ldd;
    p.accumulate = accumulate;
    p.tiles_n = (int)((N + BN - 1) / BN);
    int64_t tiles = ((M + BM - 1) / BM) * p.tiles_n;
    FGB_REQUIRE(tiles < (1ll << 31), FGB_EINVAL, "fp8_block_gemm: too many tiles");
    return dispatch<false>(mode, ag, bg, d_dtype == FGB_BF16, p, tiles, (hipStream_t)stream);
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
    return dispatch<true>(mode, AG_ROW128, BG_BLOCK, d_dtype == FGB_BF16, p, tiles, (hipStream_t)stream);
}
