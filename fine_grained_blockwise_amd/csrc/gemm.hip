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
// consecutive rows hit distinct banks.  The K loop is software-pipelined by
// half steps (see the main loop) so the matrix units work right after every
// barrier while LDS reads and HBM copies are in flight.  Tiles are mapped to
// XCDs in contiguous ranges so neighbouring tiles share an XCD's L2.
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
constexpr int EPI_BYTES = 4 * 128 * (128 * 2 + 16); // epilogue staging, 4 waves (bf16; fp32 halves fit too)
constexpr int LDS_BYTES = 2 * STAGE_BYTES > EPI_BYTES ? 2 * STAGE_BYTES : EPI_BYTES; // 136 KB

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
    // Within an XCD's contiguous range, tiles run in bands of GM m-tiles:
    // consecutive tiles walk down a band first, so the ~32 tiles an XCD runs
    // at once form a GM x 8 block sharing A rows and B columns in L2.
    int64_t tile = xcd_remap(blockIdx.x, gridDim.x);
    int64_t tm, tn;
    {
        constexpr int64_t GM = 4;
        const int64_t tiles_m = gridDim.x / p.tiles_n;
        const int64_t band = tile / (GM * p.tiles_n), in = tile % (GM * p.tiles_n);
        const int64_t bm = min(GM, tiles_m - band * GM); // rows in this (possibly last) band
        tm = band * GM + in % bm;
        tn = in / bm;
    }
    int64_t m0 = 0, m_end = 0;
    const uint8_t *B = p.b, *SB = p.sb;
    if constexpr (!GROUPED) {
        m0 = tm * BM;
        m_end = p.M;
    } else {
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
    // One 16-byte-per-lane HBM -> LDS copy; M0 holds the wave-uniform LDS
    // base, lane l lands at M0 + 16*l.  Issued as inline asm so that the
    // compiler does not place a wait on it in front of unrelated LDS reads:
    // the kernel itself waits for all copies (s_waitcnt vmcnt(0)) before the
    // barrier that precedes reading a stage.
    auto dma16 = [](const uint8_t *g, uint32_t lds_addr) {
        asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, off"
                     :
                     : "s"(lds_addr), "v"(g)
                     : "memory", "m0");
    };
    const uint32_t lds_base = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) uint8_t *)smem;
    auto issue_copy = [&](int stage, int64_t ks) {
        const uint32_t sa_ = lds_base + stage * STAGE_BYTES, sb_ = sa_ + TILE_BYTES;
#pragma unroll
        for (int i = 0; i < 8; i++) {
            dma16(a_base + a_off[i] + ks * BK, __builtin_amdgcn_readfirstlane(sa_ + (wave * 8 + i) * 1024));
            dma16(b_base + b_off[i] + ks * BK, __builtin_amdgcn_readfirstlane(sb_ + (wave * 8 + i) * 1024));
        }
    };

    // ---- scale plan ----------------------------------------------------------
    // Per K step and operand tile t, a lane needs the scale(s) of its row of
    // that tile: one byte (128-element groups) or the four consecutive bytes
    // of the step's 32-element blocks, read as one dword.  They are loaded one
    // step ahead and consumed after the next barrier.
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
    auto load_scales = [&](int64_t ks, uint32_t(&ra)[4], uint32_t(&rb)[4]) {
#pragma unroll
        for (int t = 0; t < 4; t++) {
            ra[t] = A32 ? *reinterpret_cast<const uint32_t *>(sa_base + sa_off[t] + ks * 4)
                        : (uint32_t)sa_base[sa_off[t] + ks];
            if constexpr (BG == BG_BLOCK)
                rb[t] = t == 0 ? (uint32_t)sb_base[ks] : 0u;
            else
                rb[t] = B32 ? *reinterpret_cast<const uint32_t *>(sb_base + sb_off[t] + ks * 4)
                            : (uint32_t)sb_base[sb_off[t] + ks];
        }
    };

    // ---- fragment addressing ---------------------------------------------------
    // operand row r = t*32 + lane%32 within the wave's 128 rows (the wave's
    // 128-row offset leaves swz unchanged); chunk 2q + h.  swz(r) for odd t is
    // swz for even t with bit 2 flipped, i.e. chunk 2q+h of an odd tile sits
    // where chunk 2(q^2)+h of an even tile does; t*4096 is an immediate.
    int qoff[4];
#pragma unroll
    for (int q = 0; q < 4; q++)
        qoff[q] = l32 * 128 + (((2 * q + hk) ^ swz(l32)) * 16);
    // half hf of a K step = chunks q = 2hf, 2hf+1 of every A and B tile
    auto read_half = [&](int stage, int hf, uint4(&fa)[4][2], uint4(&fb)[4][2]) {
        const uint8_t *la = smem + stage * STAGE_BYTES + wm * 128 * 128;
        const uint8_t *lb = smem + stage * STAGE_BYTES + TILE_BYTES + wn * 128 * 128;
#pragma unroll
        for (int qq = 0; qq < 2; qq++)
#pragma unroll
            for (int t = 0; t < 4; t++) {
                const int q = 2 * hf + qq;
                const int off = qoff[(t & 1) ? (q ^ 2) : q] + t * 4096;
                fa[t][qq] = *reinterpret_cast<const uint4 *>(la + off);
                fb[t][qq] = *reinterpret_cast<const uint4 *>(lb + off);
            }
    };

    v16f acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; i++)
#pragma unroll
        for (int j = 0; j < 4; j++)
            acc[i][j] = (v16f){0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};

    // MFMAs of half hf of a K step whose scales are ca/cb.
    // Scales of one K step, compact: for a 128-element group operand one
    // word with byte t = tile t; for 1x32 one word per tile (byte = 32-block
    // of the step); for 128x128 B one byte.
    constexpr int NA = A32 ? 4 : 1, NB = B32 ? 4 : 1;
    auto pack = [&](const uint32_t(&ra)[4], const uint32_t(&rb)[4], uint32_t(&wa)[NA], uint32_t(&wb)[NB]) {
        if constexpr (A32) {
#pragma unroll
            for (int t = 0; t < 4; t++)
                wa[t] = ra[t];
        } else {
            wa[0] = ra[0] | (ra[1] << 8) | (ra[2] << 16) | (ra[3] << 24);
        }
        if constexpr (B32) {
#pragma unroll
            for (int t = 0; t < 4; t++)
                wb[t] = rb[t];
        } else if constexpr (BG == BG_BLOCK) {
            wb[0] = rb[0];
        } else {
            wb[0] = rb[0] | (rb[1] << 8) | (rb[2] << 16) | (rb[3] << 24);
        }
    };
    auto compute_half = [&](int hf, const uint4(&fa)[4][2], const uint4(&fb)[4][2], const uint32_t(&ca)[NA],
                            const uint32_t(&cb)[NB]) {
        if constexpr (MODE == MODE_FAST) {
            const int s = hf; // 64-wide sub-step
            uint32_t wa = 0, wb = 0;
            if constexpr (A32) {
                const int sh = 8 * (2 * s + hk);
#pragma unroll
                for (int t = 0; t < 4; t++)
                    wa |= ((ca[t] >> sh) & 0xFFu) << (8 * t);
            } else {
                wa = ca[0];
            }
            if constexpr (B32) {
                const int shb = 8 * (2 * s + hk);
#pragma unroll
                for (int t = 0; t < 4; t++)
                    wb |= ((cb[t] >> shb) & 0xFFu) << (8 * t);
            } else {
                wb = cb[0];
            }
            v8i av[4], bv[4];
#pragma unroll
            for (int t = 0; t < 4; t++) {
                av[t] = cat(fa[t][0], fa[t][1]);
                bv[t] = cat(fb[t][0], fb[t][1]);
            }
#define FGB_J(I, J) acc[I][J] = mfma_scaled<I, (BG == BG_BLOCK ? 0 : J)>(av[I], bv[J], acc[I][J], wa, wb);
#define FGB_I(I) FGB_J(I, 0) FGB_J(I, 1) FGB_J(I, 2) FGB_J(I, 3)
            FGB_I(0) FGB_I(1) FGB_I(2) FGB_I(3)
#undef FGB_I
#undef FGB_J
        } else {
#pragma unroll
            for (int qq = 0; qq < 2; qq++) {
                const int q = 2 * hf + qq; // 32-wide pair
                float sa_f[4], sb_f[4];
#pragma unroll
                for (int t = 0; t < 4; t++) {
                    sa_f[t] = scale_f32(A32 ? (ca[t] >> (8 * q)) & 0xFFu : (ca[0] >> (8 * t)) & 0xFFu);
                    sb_f[t] = scale_f32(B32 ? (cb[t] >> (8 * q)) & 0xFFu
                                            : (BG == BG_BLOCK ? cb[0] : (cb[0] >> (8 * t)) & 0xFFu));
                }
                // bytes 0-7 of the chunk feed sub-step 2q, bytes 8-15 sub-step 2q+1
#pragma unroll
                for (int sub = 0; sub < 2; sub++) {
                    v8bf av[4], bv[4];
#pragma unroll
                    for (int t = 0; t < 4; t++) {
                        av[t] = sub == 0 ? cvt8_bf16(fa[t][qq].x, fa[t][qq].y, sa_f[t])
                                         : cvt8_bf16(fa[t][qq].z, fa[t][qq].w, sa_f[t]);
                        bv[t] = sub == 0 ? cvt8_bf16(fb[t][qq].x, fb[t][qq].y, sb_f[t])
                                         : cvt8_bf16(fb[t][qq].z, fb[t][qq].w, sb_f[t]);
                    }
#pragma unroll
                    for (int i = 0; i < 4; i++)
#pragma unroll
                        for (int j = 0; j < 4; j++)
                            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av[i], bv[j], acc[i][j], 0, 0, 0);
                    __builtin_amdgcn_sched_barrier(0); // keep each sub-step's converts next to its MFMAs
                }
            }
        }
    };

    // ---- main loop ---------------------------------------------------------------
    // Iteration j: wait for stage j's copy and sync; start the copy of step
    // j+1 into the other stage (free: every wave finished reading it before
    // this barrier); read half 0 of step j; multiply half 1 of step j-1
    // (already in registers); read half 1 of step j; multiply half 0 of step j.
    // The matrix units start right after each barrier, LDS reads overlap the
    // MFMAs of the other half, and each copy has a full step to land.
    uint4 f0a[4][2], f0b[4][2], f1a[4][2], f1b[4][2];
    uint32_t ca_cur[NA], cb_cur[NB], ca_prev[NA], cb_prev[NB], ra[4], rb[4];
    load_scales(0, ra, rb);
    issue_copy(0, 0);
    for (int64_t ks = 0; ks < nk; ks++) {
        const int cur = (int)(ks & 1);
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        __syncthreads();
        pack(ra, rb, ca_cur, cb_cur);
        if (ks + 1 < nk) {
            issue_copy(cur ^ 1, ks + 1);
            load_scales(ks + 1, ra, rb);
        }
        read_half(cur, 0, f0a, f0b);
        __builtin_amdgcn_sched_barrier(0);
        if (ks > 0)
            compute_half(1, f1a, f1b, ca_prev, cb_prev);
        __builtin_amdgcn_sched_barrier(0);
        read_half(cur, 1, f1a, f1b);
        __builtin_amdgcn_sched_barrier(0);
        compute_half(0, f0a, f0b, ca_cur, cb_cur);
#pragma unroll
        for (int t = 0; t < NA; t++)
            ca_prev[t] = ca_cur[t];
#pragma unroll
        for (int t = 0; t < NB; t++)
            cb_prev[t] = cb_cur[t];
    }
    compute_half(1, f1a, f1b, ca_prev, cb_prev);

    // ---- epilogue --------------------------------------------------------------
    // 32x32 accumulator layout: lane l, register r -> row (r/4)*8 + (l/32)*4 + r%4,
    // column l%32.  The tile is staged through LDS (free after the last
    // barrier) so that global stores are 16 bytes per lane along rows: each
    // wave writes its 128x128 block, 64 rows at a time, as [row][128 + pad]
    // and reads it back row-contiguous.
    __syncthreads();
    constexpr int ESZ = OUT_BF16 ? 2 : 4;
    constexpr int ROWB = 128 * ESZ + 16;   // padded LDS row (bytes)
    constexpr int EPI_ROWS = OUT_BF16 ? 128 : 64;
    uint8_t *ep = smem + wave * (EPI_ROWS * ROWB);
    float l1v[4];
#pragma unroll
    for (int j = 0; j < 4; j++) {
        int64_t col = n0 + wn * 128 + j * 32 + l32;
        l1v[j] = (p.l1 && col < N) ? p.l1[col] : 1.0f;
    }
#pragma unroll
    for (int part = 0; part < 128 / EPI_ROWS; part++) {
#pragma unroll
        for (int ii = 0; ii < EPI_ROWS / 32; ii++) {
            const int i = part * (EPI_ROWS / 32) + ii;
#pragma unroll
            for (int j = 0; j < 4; j++)
#pragma unroll
                for (int r = 0; r < 16; r++) {
                    int row = ii * 32 + (r / 4) * 8 + hk * 4 + (r % 4);
                    int col = j * 32 + l32;
                    float v = acc[i][j][r];
                    if (p.l1)
                        v *= l1v[j];
                    if constexpr (OUT_BF16)
                        *reinterpret_cast<uint16_t *>(ep + row * ROWB + col * 2) = (uint16_t)bf16_rne(v);
                    else
                        *reinterpret_cast<float *>(ep + row * ROWB + col * 4) = v;
                }
        }
        __builtin_amdgcn_s_waitcnt(0xc07f); // lgkmcnt(0): this wave's LDS writes done
        __builtin_amdgcn_wave_barrier();
        // read back: one row segment of 16 bytes per lane
        constexpr int LPR = 128 * ESZ / 16; // lanes per row
        constexpr int RPI = 64 / LPR;       // rows per instruction
        const int lr = lane / LPR, lc = lane % LPR;
#pragma unroll
        for (int rr = 0; rr < EPI_ROWS; rr += RPI) {
            const int row_l = rr + lr;
            const int64_t row = m0 + wm * 128 + part * EPI_ROWS + row_l;
            const int64_t col0 = n0 + wn * 128 + lc * (16 / ESZ);
            uint4 v = *reinterpret_cast<const uint4 *>(ep + row_l * ROWB + lc * 16);
            if (row >= m_end || col0 >= N)
                continue;
            uint8_t *dst = (uint8_t *)p.d + (row * p.ldd + col0) * ESZ;
            const bool full = col0 + 16 / ESZ <= N && (((uintptr_t)dst & 15) == 0);
            if constexpr (OUT_BF16) {
                if (full) {
                    *reinterpret_cast<uint4 *>(dst) = v;
                } else {
                    uint32_t w4[4] = {v.x, v.y, v.z, v.w};
                    for (int e = 0; e < 8 && col0 + e < N; e++)
                        reinterpret_cast<uint16_t *>(dst)[e] = (uint16_t)(w4[e / 2] >> (16 * (e & 1)));
                }
            } else {
                float f4[4] = {__uint_as_float(v.x), __uint_as_float(v.y), __uint_as_float(v.z), __uint_as_float(v.w)};
                float *fd = reinterpret_cast<float *>(dst);
                if (full) {
                    if (p.accumulate) {
                        float4 o = *reinterpret_cast<const float4 *>(fd);
                        f4[0] += o.x; f4[1] += o.y; f4[2] += o.z; f4[3] += o.w;
                    }
                    *reinterpret_cast<float4 *>(fd) = make_float4(f4[0], f4[1], f4[2], f4[3]);
                } else {
                    for (int e = 0; e < 4 && col0 + e < N; e++)
                        fd[e] = p.accumulate ? fd[e] + f4[e] : f4[e];
                }
            }
        }
        __builtin_amdgcn_s_waitcnt(0xc07f);
        __builtin_amdgcn_wave_barrier();
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
