// gemm.hip -- blockwise-scaled FP8 GEMM (dense and M-grouped) on gfx950 MFMA.
//
// llm-infra-atlas, "01 · DeepSeek FP8 and DeepGEMM: Hopper software recipe":
//   §1 a Linear's Fprop / Dgrad / Wgrad; §4 two-level accumulation -- the
//   partial sum of each 128-element K group is multiplied by the product of
//   the A and B scales and added to an FP32 accumulator; §5.2 1D2D (1x128 A,
//   128x128 B scales) vs 1D1D (1x128 scales on both sides, Wgrad); §5.6
//   M-grouped contiguous layout for MoE experts; §5.7 NT, K-major operands.
// xllm-io review "MOSS", §3: 32-element E8M0 scales plus an FP32 level-1
//   factor (the b_l1 epilogue).
//
// Design (gfx950, not the Hopper one): the per-K-group scaling runs inside
// the matrix core.  V_MFMA_SCALE_F32_32X32X64_F8F6F4 takes, per lane, one
// E8M0 scale byte for A and one for B that multiply that lane's 32-element K
// slice before accumulation in FP32.  Our scales are already E8M0 bytes
// (2^(b-127)), so the 128-element group scale is fed to all four 32-element
// slices of the group, and 1x32 (MX) scales are fed as they are: no VALU
// promotion step, one code path for 1D2D, 1D1D and MX.
//
// Tiling: 256x256 output tile per workgroup of 4 waves (each wave 128x128 =
// 4x4 MFMA tiles of 32x32), K step 128 (one scale group).  A and B tiles
// (256 rows x 128 bytes each) are copied HBM -> LDS with
// global_load_lds_dwordx4 (no VGPR round trip) into a double buffer
// (2 x 64 KB).  LDS rows are 128 bytes; the 16-byte chunk index is XOR-swizzled
// with f(row) = (row ^ row>>3) & 7 so that the column reads of the MFMA
// operand fetch hit distinct banks.  Tiles are mapped to XCDs in contiguous
// ranges so neighbouring tiles share an XCD's L2.
#include "fgb_internal.h"

namespace fgb {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v16f __attribute__((ext_vector_type(16)));

constexpr int BM = 256, BN = 256, BK = 128;
constexpr int TILE_BYTES = BM * BK; // one operand tile: 32 KB
constexpr int STAGE_BYTES = 2 * TILE_BYTES;
constexpr int LDS_BYTES = 2 * STAGE_BYTES; // double buffer: 128 KB

enum { AG_ROW128 = 0, AG_ROW32 = 1 };
enum { BG_ROW128 = 0, BG_ROW32 = 1, BG_BLOCK = 2 };

struct GemmArgs {
    const uint8_t *a, *sa, *b, *sb;
    const float *l1;
    void *d;
    int64_t M, N, K, lda, ldb, ldd;
    int accumulate;
    int tiles_n;
    int64_t tiles;          // dense: tiles_m * tiles_n; grouped: grid upper bound
    const int32_t *offs;    // grouped: group offsets [G+1]
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

template <int AG, int BG, bool OUT_BF16, bool GROUPED>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1))) void
gemm_fp8_kernel(GemmArgs p)
{
    extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wm = wave >> 1, wn = wave & 1;
    const int64_t K = p.K, nk = K / BK;

    // ---- tile -> (m0, n0) ------------------------------------------------
    int64_t tile = xcd_remap(blockIdx.x, gridDim.x);
    int64_t m0, m_end, tn;
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
    const int64_t N = p.N;

    // ---- global -> LDS copy plan -----------------------------------------
    // Operand tile = 32 groups of 8 rows (1 KB each); wave w copies groups
    // w*8 .. w*8+7 of A and of B.  Lane l lands at LDS offset l*16 of its
    // group: row g*8 + l/8, physical chunk l%8, which holds logical chunk
    // (l%8) ^ swz(row).
    const uint8_t *ga[8], *gb[8];
    {
        const int l8 = lane >> 3;
#pragma unroll
        for (int i = 0; i < 8; i++) {
            int g = wave * 8 + i;
            int r = g * 8 + l8;
            int chunk = (lane & 7) ^ swz(r);
            int64_t ar = m0 + r;
            ar = ar < m_end ? ar : m_end - 1;
            int64_t br = n0 + r;
            br = br < N ? br : N - 1;
            ga[i] = p.a + ar * p.lda + chunk * 16;
            gb[i] = B + br * p.ldb + chunk * 16;
        }
    }
    auto issue_copy = [&](int stage, int64_t ks) {
        uint8_t *sa_ = smem + stage * STAGE_BYTES;
        uint8_t *sb_ = sa_ + TILE_BYTES;
#pragma unroll
        for (int i = 0; i < 8; i++) {
            __builtin_amdgcn_global_load_lds(ga[i] + ks * BK,
                                             (__attribute__((address_space(3))) void *)(sa_ + (wave * 8 + i) * 1024), 16, 0, 0);
            __builtin_amdgcn_global_load_lds(gb[i] + ks * BK,
                                             (__attribute__((address_space(3))) void *)(sb_ + (wave * 8 + i) * 1024), 16, 0, 0);
        }
    };

    // ---- scale plan ----------------------------------------------------------
    // A: lane's rows wm*128 + i*32 + lane%32 (i = 0..3), one byte each per K
    // group, packed so that byte i feeds MFMA row tile i (op_sel).
    const int l32 = lane & 31, hk = lane >> 5;
    const uint8_t *sa_row[4];
    const int64_t ga_per_row = AG == AG_ROW32 ? K / 32 : K / 128;
#pragma unroll
    for (int i = 0; i < 4; i++) {
        int64_t r = m0 + wm * 128 + i * 32 + l32;
        r = r < m_end ? r : m_end - 1;
        sa_row[i] = p.sa + r * ga_per_row;
    }
    const uint8_t *sb_row[4];
    const int64_t gb_per_row = BG == BG_ROW32 ? K / 32 : K / 128;
#pragma unroll
    for (int j = 0; j < 4; j++) {
        if constexpr (BG == BG_BLOCK) {
            // a wave's 128 columns lie in one 128-row block of B; past the last
            // block (ragged N) clamp to it -- those columns are never stored
            int64_t nb = (n0 + wn * 128) / 128, nb_last = (N - 1) / 128;
            sb_row[j] = SB + (nb < nb_last ? nb : nb_last) * (K / 128);
        } else {
            int64_t c = n0 + wn * 128 + j * 32 + l32;
            c = c < N ? c : N - 1;
            sb_row[j] = SB + c * gb_per_row;
        }
    }
    // Scale bytes for K step ks are loaded one step ahead into raw[] and
    // packed into MFMA scale words only after the next barrier, so no wait on
    // them is ever placed between the LDS copies and the MFMAs.
    //   raw[s*8 + i]     : A byte for row tile i, sub-step s
    //   raw[s*8 + 4 + j] : B byte for column tile j (BLOCK: j = 0 only)
    constexpr bool PER32 = AG == AG_ROW32;
    constexpr int NS = PER32 ? 2 : 1;
    auto load_scales = [&](int64_t ks, uint32_t(&raw)[16]) {
#pragma unroll
        for (int s = 0; s < NS; s++) {
#pragma unroll
            for (int i = 0; i < 4; i++)
                raw[s * 8 + i] = PER32 ? sa_row[i][ks * 4 + s * 2 + hk] : sa_row[i][ks];
            if constexpr (BG == BG_BLOCK) {
                raw[s * 8 + 4] = sb_row[0][ks];
            } else {
#pragma unroll
                for (int j = 0; j < 4; j++)
                    raw[s * 8 + 4 + j] = PER32 ? sb_row[j][ks * 4 + s * 2 + hk] : sb_row[j][ks];
            }
        }
    };
    auto pack_scales = [&](const uint32_t(&raw)[16], uint32_t(&wa)[2], uint32_t(&wb)[2]) {
#pragma unroll
        for (int s = 0; s < NS; s++) {
            wa[s] = raw[s * 8 + 0] | (raw[s * 8 + 1] << 8) | (raw[s * 8 + 2] << 16) | (raw[s * 8 + 3] << 24);
            if constexpr (BG == BG_BLOCK)
                wb[s] = raw[s * 8 + 4];
            else
                wb[s] = raw[s * 8 + 4] | (raw[s * 8 + 5] << 8) | (raw[s * 8 + 6] << 16) | (raw[s * 8 + 7] << 24);
        }
        if constexpr (NS == 1) {
            wa[1] = wa[0];
            wb[1] = wb[0];
        }
    };

    // ---- main loop -----------------------------------------------------------
    v16f acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; i++)
#pragma unroll
        for (int j = 0; j < 4; j++)
            acc[i][j] = (v16f){0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};

    uint32_t raw[16] = {0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0};
    uint32_t wa_cur[2], wb_cur[2];
    load_scales(0, raw);
    issue_copy(0, 0);

    // fragment addressing: operand row r = w*128 + t*32 + lane%32, logical
    // chunks s*4 + hk*2 + {0,1}
    int frag_off[4][2][2];
#pragma unroll
    for (int t = 0; t < 4; t++) {
        int r = t * 32 + l32; // + w*128 added below (w*128 keeps swz unchanged)
#pragma unroll
        for (int s = 0; s < 2; s++)
#pragma unroll
            for (int h = 0; h < 2; h++)
                frag_off[t][s][h] = r * 128 + (((s * 4 + hk * 2 + h) ^ swz(r)) * 16);
    }

    for (int64_t ks = 0; ks < nk; ks++) {
        const int cur = (int)(ks & 1);
        __builtin_amdgcn_s_waitcnt(0);
        __syncthreads();
        pack_scales(raw, wa_cur, wb_cur);
        const uint8_t *la = smem + cur * STAGE_BYTES + wm * 128 * 128;
        const uint8_t *lb = smem + cur * STAGE_BYTES + TILE_BYTES + wn * 128 * 128;
        v8i af[2][4], bfr[2][4];
#pragma unroll
        for (int s = 0; s < 2; s++)
#pragma unroll
            for (int t = 0; t < 4; t++) {
                uint4 x0 = *reinterpret_cast<const uint4 *>(la + frag_off[t][s][0]);
                uint4 x1 = *reinterpret_cast<const uint4 *>(la + frag_off[t][s][1]);
                af[s][t] = (v8i){(int)x0.x, (int)x0.y, (int)x0.z, (int)x0.w, (int)x1.x, (int)x1.y, (int)x1.z, (int)x1.w};
                uint4 y0 = *reinterpret_cast<const uint4 *>(lb + frag_off[t][s][0]);
                uint4 y1 = *reinterpret_cast<const uint4 *>(lb + frag_off[t][s][1]);
                bfr[s][t] = (v8i){(int)y0.x, (int)y0.y, (int)y0.z, (int)y0.w, (int)y1.x, (int)y1.y, (int)y1.z, (int)y1.w};
            }
        if (ks + 1 < nk) {
            load_scales(ks + 1, raw);
            issue_copy(cur ^ 1, ks + 1);
        }
#pragma unroll
        for (int s = 0; s < 2; s++)
#pragma unroll
            for (int i = 0; i < 4; i++)
#pragma unroll
                for (int j = 0; j < 4; j++) {
                    if constexpr (BG == BG_BLOCK) {
                        switch (i) {
                        case 0: acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(af[s][i], bfr[s][j], acc[i][j], 0, 0, 0, (int)wa_cur[s], 0, (int)wb_cur[s]); break;
                        case 1: acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(af[s][i], bfr[s][j], acc[i][j], 0, 0, 1, (int)wa_cur[s], 0, (int)wb_cur[s]); break;
                        case 2: acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(af[s][i], bfr[s][j], acc[i][j], 0, 0, 2, (int)wa_cur[s], 0, (int)wb_cur[s]); break;
                        default: acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(af[s][i], bfr[s][j], acc[i][j], 0, 0, 3, (int)wa_cur[s], 0, (int)wb_cur[s]); break;
                        }
                    } else {
#define FGB_MFMA_IJ(I, J)                                                                          \
    if (i == I && j == J)                                                                          \
        acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(af[s][i], bfr[s][j], acc[i][j], 0, 0, I, (int)wa_cur[s], J, (int)wb_cur[s]);
                        FGB_MFMA_IJ(0, 0) FGB_MFMA_IJ(0, 1) FGB_MFMA_IJ(0, 2) FGB_MFMA_IJ(0, 3)
                        FGB_MFMA_IJ(1, 0) FGB_MFMA_IJ(1, 1) FGB_MFMA_IJ(1, 2) FGB_MFMA_IJ(1, 3)
                        FGB_MFMA_IJ(2, 0) FGB_MFMA_IJ(2, 1) FGB_MFMA_IJ(2, 2) FGB_MFMA_IJ(2, 3)
                        FGB_MFMA_IJ(3, 0) FGB_MFMA_IJ(3, 1) FGB_MFMA_IJ(3, 2) FGB_MFMA_IJ(3, 3)
#undef FGB_MFMA_IJ
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

template <int AG, int BG, bool OUT_BF16, bool GROUPED>
static int launch_one(const GemmArgs &p, int64_t grid, hipStream_t st)
{
    auto kern = gemm_fp8_kernel<AG, BG, OUT_BF16, GROUPED>;
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

template <bool GROUPED>
static int dispatch(int ag, int bg, bool bf16, const GemmArgs &p, int64_t grid, hipStream_t st)
{
    if (ag == AG_ROW128 && bg == BG_BLOCK)
        return bf16 ? launch_one<AG_ROW128, BG_BLOCK, true, GROUPED>(p, grid, st)
                    : launch_one<AG_ROW128, BG_BLOCK, false, GROUPED>(p, grid, st);
    if constexpr (!GROUPED) {
        if (ag == AG_ROW128 && bg == BG_ROW128)
            return bf16 ? launch_one<AG_ROW128, BG_ROW128, true, false>(p, grid, st)
                        : launch_one<AG_ROW128, BG_ROW128, false, false>(p, grid, st);
        if (ag == AG_ROW32 && bg == BG_ROW32)
            return bf16 ? launch_one<AG_ROW32, BG_ROW32, true, false>(p, grid, st)
                        : launch_one<AG_ROW32, BG_ROW32, false, false>(p, grid, st);
    }
    return set_error(FGB_EUNSUPPORTED, "gemm: unsupported scale granularity pair (%d, %d)", ag, bg);
}

} // namespace fgb

using namespace fgb;

extern "C" int fp8_block_gemm(const uint8_t *a, const uint8_t *sa, int a_gran, const uint8_t *b,
                              const uint8_t *sb, int b_gran, const float *b_l1, int64_t g1,
                              int64_t M, int64_t N, int64_t K, int64_t lda, int64_t ldb, void *d,
                              int d_dtype, int64_t ldd, int accumulate, void *workspace,
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
    FGB_REQUIRE(ldd >= N, FGB_EINVAL, "fp8_block_gemm: ldd must be >= N");
    FGB_REQUIRE(aligned16(a) && aligned16(b), FGB_EINVAL, "fp8_block_gemm: a and b must be 16-byte aligned");
    FGB_REQUIRE(d_dtype == FGB_F32 || d_dtype == FGB_BF16, FGB_EUNSUPPORTED,
                "fp8_block_gemm: d_dtype must be FGB_F32 or FGB_BF16");
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
    GemmArgs p{};
    p.a = a; p.sa = sa; p.b = b; p.sb = sb; p.l1 = b_l1; p.d = d;
    p.M = M; p.N = N; p.K = K; p.lda = lda; p.ldb = ldb; p.ldd = ldd;
    p.accumulate = accumulate;
    p.tiles_n = (int)((N + BN - 1) / BN);
    p.tiles = ((M + BM - 1) / BM) * p.tiles_n;
    FGB_REQUIRE(p.tiles < (1ll << 31), FGB_EINVAL, "fp8_block_gemm: too many tiles");
    return dispatch<false>(ag, bg, d_dtype == FGB_BF16, p, p.tiles, (hipStream_t)stream);
}

extern "C" int fp8_grouped_gemm(const uint8_t *a, const uint8_t *sa, const uint8_t *b,
                                const uint8_t *sb, const int32_t *group_offsets, int G,
                                int64_t M_cap, int64_t N, int64_t K, void *d, int d_dtype,
                                void *stream)
{
    clear_error();
    FGB_REQUIRE(a && sa && b && sb && d && group_offsets, FGB_EINVAL, "fp8_grouped_gemm: null pointer");
    FGB_REQUIRE(G >= 1 && G <= 1024, FGB_EINVAL, "fp8_grouped_gemm: G must be in [1, 1024]");
    FGB_REQUIRE(M_cap >= 0 && N > 0 && K > 0 && K % 128 == 0, FGB_EINVAL,
                "fp8_grouped_gemm: need N > 0 and K a positive multiple of 128");
    FGB_REQUIRE(aligned16(a) && aligned16(b), FGB_EINVAL, "fp8_grouped_gemm: a and b must be 16-byte aligned");
    FGB_REQUIRE(d_dtype == FGB_F32 || d_dtype == FGB_BF16, FGB_EUNSUPPORTED,
                "fp8_grouped_gemm: d_dtype must be FGB_F32 or FGB_BF16");
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
    p.tiles = ((M_cap + BM - 1) / BM + G) * p.tiles_n;
    FGB_REQUIRE(p.tiles < (1ll << 31), FGB_EINVAL, "fp8_grouped_gemm: too many tiles");
    return dispatch<true>(AG_ROW128, BG_BLOCK, d_dtype == FGB_BF16, p, p.tiles, (hipStream_t)stream);
}
