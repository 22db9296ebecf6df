/*
 * fgb.h -- C ABI of libfgb.so: fine-grained blockwise FP8 (E4M3 codes with
 * power-of-two UE8M0 scales) for AMD Instinct MI355X (gfx950).
 *
 * Sources cited below (page title, section):
 *   [DSV3]  llm-infra-atlas, "01 · DeepSeek FP8 and DeepGEMM: Hopper software recipe"
 *   [LP]    llm-infra-atlas, "Low precision" chapter index
 *   [FLOW]  awesome-system-papers, "FP8-Flow-MoE: A Casting-Free FP8 Recipe without
 *           Double Quantization Error (MLSys 2026)"
 *   [MOSS]  xllm-io paper review, "MOSS: Efficient and Accurate FP8 LLM Training with
 *           Microscaling and Automatic Scaling"
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 *  - Codes are uint8 OCP E4M3FN ([LP] §2: 1/4/3 bits, max 448, no Inf): bias 7,
 *    NaN only at 0x7F/0xFF.  Conversions round to nearest even and keep the
 *    sign (negative underflow gives 0x80).
 *  - A scale is one byte b = e + 127 meaning the power of two 2^e; a value is
 *    decode(code) * 2^e ([DSV3] §3 multiplier convention, §8 UE8M0).  For an
 *    amax over a group, e is the smallest integer with amax <= 448 * 2^e,
 *    floored at -22 for 128-element groups ([DSV3] §3, the 1e-4 amax clamp)
 *    and at -127 for 32-element groups (E8M0 range, [MOSS] §3).
 *  - Matrices are row-major.  ld* arguments are leading dimensions in
 *    elements.  Every data pointer is a device pointer owned by the caller;
 *    the library allocates nothing, keeps no pointer after return and holds
 *    no global state.
 *  - stream is a hipStream_t (NULL = the null stream).  Every call only
 *    enqueues work: no host synchronisation, no implicit copies.  Results are
 *    deterministic (no floating-point atomics).
 *  - Return value: FGB_OK or an error code; arguments are validated on the
 *    host before anything is enqueued, so an error leaves the outputs
 *    untouched.  fgb_last_error() gives a thread-local message.
 *  - Data pointers must be 16-byte aligned, and every ld* times the element
 *    size must be a multiple of 16 bytes, except where stated.
 *  - Inputs are assumed finite; non-finite inputs give unspecified outputs.
 */
#ifndef FGB_H
#define FGB_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* status codes */
#define FGB_OK 0
#define FGB_EINVAL 1       /* null pointer, bad size, misalignment, bad ld */
#define FGB_EUNSUPPORTED 2 /* dtype / granularity combination not provided */
#define FGB_EWORKSPACE 3   /* workspace missing or too small */
#define FGB_EHIP 4         /* a HIP runtime call failed (launch error) */

/* element types */
#define FGB_F32 0
#define FGB_BF16 1

/* GEMM arithmetic modes */
#define FGB_GEMM_EXACT 0 /* FP32 accumulation of exact products (bf16 matrix unit) */
#define FGB_GEMM_FAST 1  /* FP8 matrix unit with its own product-sum precision */

/* element formats of the format-variant entry points ([LP] §2 format table) */
#define FGB_E4M3 0 /* OCP E4M3FN: bias 7, max 448, no Inf (the path's default) */
#define FGB_E5M2 1 /* OCP E5M2: bias 15, max 57344, Inf/NaN at exponent field 31 */

/* scale rules of the format-variant entry points */
#define FGB_SCALE_CEIL 0      /* smallest e with amax <= max * 2^e (the rule everywhere else) */
#define FGB_SCALE_OCP_FLOOR 1 /* MX standard: e = floor(log2 amax) - emax (8 for E4M3, 15 for E5M2);
                                 scaled values above the format's maximum clip to it */

/* scale granularities */
#define FGB_ROW1x128 0 /* one scale per row per 128 columns: s[rows, cols/128] */
#define FGB_ROW1x32 1  /* one scale per row per 32 columns:  s[rows, cols/32] */
#define FGB_BLOCK128 2 /* one scale per 128x128 block: s[ceil(rows/128), cols/128] */

/* Thread-local text of the last error raised on this thread ("" if none). */
const char *fgb_last_error(void);

/* Library version string. */
const char *fgb_version(void);

/*
 * fp8_quant_rowwise -- 1 x group activation quantization.
 * [DSV3] §2 (online quantization: amax of every 1x128 activation tile is
 * computed at run time) and §3 (per token per 128 channels, scale tensor
 * [T, C/128]); group 32 is the MX single-level activation scaling of [MOSS] §3.
 *   x      [rows, cols], ld ldx, dtype x_dtype (FGB_F32 or FGB_BF16)
 *   group  128 or 32; cols % group == 0
 *   q      [rows, cols] E4M3 codes, ld ldq (bytes; multiple of 16)
 *   s      [rows, cols/group] scale bytes, ld lds (any ld >= cols/group)
 * For each row and group: e = scale exponent of the group's amax, q = E4M3
 * of x * 2^-e (an exact product, |x * 2^-e| <= 448), s = e + 127.
 */
int fp8_quant_rowwise(const void *x, int x_dtype, int64_t rows, int64_t cols, int64_t ldx,
                      int group, uint8_t *q, int64_t ldq, uint8_t *s, int64_t lds, void *stream);

/*
 * fp8_quant_rowwise_fmt -- fp8_quant_rowwise with the element format and the
 * scale rule chosen ([MOSS] §3: E5M2 for backward-pass gradients; its
 * two-level section names the MX standard for the 32-element level, whose
 * shared exponent is floor(log2 amax) - emax).  fmt = FGB_E4M3 or FGB_E5M2;
 * rule = FGB_SCALE_CEIL or FGB_SCALE_OCP_FLOOR.  The floor is the 1e-4 amax
 * clamp for 128-element groups (e >= -22 for E4M3, e >= -29 for E5M2) and
 * e >= -127 for 32-element groups.  Codes: the format's code of x * 2^-e,
 * round to nearest even, clipped at the format's maximum (only the floor
 * rule reaches it).  Other arguments as fp8_quant_rowwise, which equals
 * fmt = FGB_E4M3, rule = FGB_SCALE_CEIL.
 */
int fp8_quant_rowwise_fmt(const void *x, int x_dtype, int64_t rows, int64_t cols, int64_t ldx, int group, int fmt,
                          int rule, uint8_t *q, int64_t ldq, uint8_t *s, int64_t lds, void *stream);

/*
 * fp8_quant_blockwise -- 128 x 128 weight-block quantization.
 * [DSV3] §3: per 128 input channels x 128 output channels; scale tensor
 * [Cout/128, Cin/128].  The last row block may be partial (rows % 128 != 0,
 * e.g. Cout = 2112 in [DSV3] §5.7); its amax covers the rows present.
 *   w  [rows, cols], ld ldw, FGB_F32 or FGB_BF16; cols % 128 == 0
 *   q  [rows, cols], ld ldq;  s [ceil(rows/128), cols/128], ld lds
 */
int fp8_quant_blockwise(const void *w, int w_dtype, int64_t rows, int64_t cols, int64_t ldw,
                        uint8_t *q, int64_t ldq, uint8_t *s, int64_t lds, void *stream);

/*
 * fp8_quant_blockwise_t -- fp8_quant_blockwise of G stacked bf16 matrices
 * that also writes each matrix's transposed codes and scales, the copy the
 * Dgrad GEMM reads ([DSV3] §1: Dgrad multiplies by W, so the NT GEMM needs
 * W^T K-major; §3: 128x128 blocks, whose scale is the same for the
 * transposed block).  One pass: the transposed copy is the exact byte
 * transpose of each block (fp8_block_transpose_batched of the codes), so no
 * code is read back ([FLOW] "Core method": the FP8 copies a recipe needs are
 * produced where the data is quantized).
 *   w  [G, rows, cols] bf16 dense; rows % 128 == 0, cols % 128 == 0
 *   q  [G, rows, cols], s [G, rows/128, cols/128]  (as fp8_quant_blockwise)
 *   qt [G, cols, rows], st [G, cols/128, rows/128]
 */
int fp8_quant_blockwise_t(const void *w, int w_dtype, int G, int64_t rows, int64_t cols, uint8_t *q, uint8_t *s,
                          uint8_t *qt, uint8_t *st, void *stream);

/*
 * fp8_dequant -- decode(q) * 2^(s - 127) into FP32 or BF16 (diagnostic helper).
 *   q [rows, cols] dense; s dense in the layout gran names; out [rows, cols]
 *   dense, dtype out_dtype.  BF16 output rounds to nearest even.
 */
int fp8_dequant(const uint8_t *q, const uint8_t *s, int gran, int64_t rows, int64_t cols,
                void *out, int out_dtype, void *stream);

/*
 * fp8_dequant_fmt -- fp8_dequant for codes of format fmt (FGB_E4M3 or
 * FGB_E5M2); fp8_dequant is fmt = FGB_E4M3.
 */
int fp8_dequant_fmt(const uint8_t *q, const uint8_t *s, int gran, int fmt, int64_t rows, int64_t cols, void *out,
                    int out_dtype, void *stream);

/*
 * fgb_fp8_encode -- the device conversion of fmt (FGB_E4M3 or FGB_E5M2) for
 * each fp32 value: round to nearest even, clipped at +-448 or +-57344, sign
 * kept; exposed for exhaustive checks.  x 16-byte, q 4-byte aligned.
 */
int fgb_fp8_encode(const float *x, int64_t n, int fmt, uint8_t *q, void *stream);

/*
 * fgb_e4m3_encode -- E4M3 of each fp32 value (round to nearest even,
 * saturating at +-448, sign kept).  Exposes the device conversion the
 * kernels use, for exhaustive checks.  x, q dense, n elements.
 */
int fgb_e4m3_encode(const float *x, int64_t n, uint8_t *q, void *stream);

/*
 * fp8_direct_transpose -- scaling-aware transpose ([FLOW] "Core method" and
 * key observation 2): inside each 128x128 block the block's largest scale
 * e_max is taken, and each code of row t is shifted by k_t = e_max - e_t in
 * the exponent (with round-to-nearest-even when the result falls into the
 * subnormal range), i.e. the result equals requantizing the dequantized
 * block at 2^e_max, with no dequantize/requantize pass.
 *   s_gran = FGB_ROW1x128: q [rows=T, cols=C] with s [T, C/128]
 *            -> qt [C, T], st [C, T/128] (all 128 entries of a block equal);
 *   s_gran = FGB_BLOCK128: the k = 0 case for weights, an exact byte
 *            transpose: s [T/128, C/128] -> st [C/128, T/128].
 *   rows % 128 == 0 and cols % 128 == 0; all tensors dense.
 */
int fp8_direct_transpose(const uint8_t *q, const uint8_t *s, int s_gran, int64_t rows,
                         int64_t cols, uint8_t *qt, uint8_t *st, void *stream);

/*
 * fp8_direct_transpose_fmt -- fp8_direct_transpose with s_gran =
 * FGB_ROW1x128 for codes of format fmt (FGB_E4M3 or FGB_E5M2): E5M2
 * gradients ([MOSS] §3) take the same block-max exponent shift ([FLOW]
 * "Core method"), re-rounded with round-to-nearest-even in E5M2.
 */
int fp8_direct_transpose_fmt(const uint8_t *q, const uint8_t *s, int fmt, int64_t rows, int64_t cols, uint8_t *qt,
                             uint8_t *st, void *stream);

/*
 * fp8_block_transpose_batched -- fp8_direct_transpose with s_gran =
 * FGB_BLOCK128 applied to each of G stacked matrices (the expert weights of
 * the MoE Dgrad: [DSV3] §1, Dgrad multiplies by W, and the grouped NT GEMM
 * needs each W_e^T K-major).  q [G, rows, cols], s [G, rows/128, cols/128]
 * -> qt [G, cols, rows], st [G, cols/128, rows/128]; all dense; rows % 128 ==
 * 0, cols % 128 == 0; exact byte transposes.  One kernel on `stream`.
 */
int fp8_block_transpose_batched(const uint8_t *q, const uint8_t *s, int G, int64_t rows, int64_t cols,
                                uint8_t *qt, uint8_t *st, void *stream);

/*
 * fp8_grouped_direct_transpose -- the direct transpose applied to each expert
 * segment of a permuted, padded row-wise FP8 activation, for the K-grouped
 * Wgrad of the expert backward ([FLOW] "Core method", per 128x128 block;
 * [DSV3] §5.6 grouped layouts).  Segment e = rows [off[e], off[e+1]) of q
 * (off = group_offsets on the device, as from permute_pad); its transpose
 * fills columns [koff[e], koff[e] + ceil(len_e/128)*128) of qt [cols, K_cap],
 * koff[e+1] = koff[e] + ceil(len_e/128)*128 (written to k_offsets [G+1] on
 * the device).  A segment's last 128-row block may be short: the block's
 * scale is the largest over the rows present and the columns of the absent
 * rows hold code 0.  st [cols, K_cap/128] (all 128 entries of a block
 * equal).  Columns past koff[G] are not written.
 *   q [M_cap, cols], s [M_cap, cols/128] 1x128 scales; cols % 128 == 0;
 *   K_cap % 128 == 0 and K_cap >= M_cap + 127*G rounded up to 128; 1 <= G <= 1024.
 */
int fp8_grouped_direct_transpose(const uint8_t *q, const uint8_t *s, int64_t M_cap, int64_t cols,
                                 const int32_t *group_offsets, int G, uint8_t *qt, uint8_t *st, int64_t K_cap,
                                 int32_t *k_offsets, void *stream);

/*
 * fp8_naive_transpose -- the three-pass conversion that the direct transpose
 * replaces ([FLOW] "Core method" and Fig. 1, the baseline it is 2-3x faster
 * than): dequantize the row-wise codes to bf16 (exact for power-of-two
 * scales), transpose, and requantize 1x128 along the new rows (power-of-two
 * scales, the rule of fp8_quant_rowwise).  Provided as the measured baseline;
 * its result can differ from fp8_direct_transpose (column scales instead of
 * block-max scales).
 *   q [rows=T, cols=C], s [T, C/128] -> qt [C, T], st [C, T/128]; all dense;
 *   rows % 128 == 0, cols % 128 == 0.
 *   workspace: >= fp8_naive_transpose_workspace_size(rows, cols) bytes
 *   (4*rows*cols: the bf16 copy and its transpose), 16-byte aligned, owned by
 *   the caller; FGB_EWORKSPACE if too small.  Three kernels on `stream`.
 */
int fp8_naive_transpose(const uint8_t *q, const uint8_t *s, int64_t rows, int64_t cols,
                        uint8_t *qt, uint8_t *st, void *workspace, size_t ws_bytes, void *stream);
size_t fp8_naive_transpose_workspace_size(int64_t rows, int64_t cols);

/*
 * fp8_block_gemm -- blockwise-scaled FP8 GEMM, D = A * B^T ("NT": A [M,K] and
 * B [N,K] both K-contiguous, [DSV3] §5.7).  Covers a Linear's three GEMMs
 * ([DSV3] §1): Fprop A = X, B = W; Dgrad A = dY, B = W^T (block transpose);
 * Wgrad A = dY^T, B = X^T (both from fp8_direct_transpose, 1x128 scales).
 * Every K group's product sum is scaled by 2^(ea + eb) and accumulated in
 * FP32 ([DSV3] §4, §5.3).  M, N >= 0 and K >= 0 a multiple of 128: M = 0 or
 * N = 0 writes nothing (operand pointers may be NULL); K = 0 gives the empty
 * sum, D = 0 (D unchanged when accumulating).
 *   a, sa, a_gran : A codes [M, K] (ld lda) and scales, FGB_ROW1x128 -> sa
 *                   [M, K/128], FGB_ROW1x32 -> sa [M, K/32] (dense)
 *   b, sb, b_gran : B codes [N, K] (ld ldb) and scales, FGB_BLOCK128 -> sb
 *                   [ceil(N/128), K/128], FGB_ROW1x128 -> sb [N, K/128],
 *                   FGB_ROW1x32 -> sb [N, K/32] (dense).  ROW1x32 must be
 *                   paired with ROW1x32; 1x32 scale tensors 4-byte aligned.
 *   b_l1, g1      : optional [MOSS] §3 level-1 FP32 factor per column of D,
 *                   b_l1 [N] (dense), applied to the FP32 result; requires
 *                   b_gran = FGB_ROW1x32 (the level-2 scales it goes with)
 *                   and K <= g1 (one level-1 group along K); NULL = none.
 *   d, d_dtype    : D [M, N], ld ldd, FGB_F32 or FGB_BF16 (round to nearest
 *                   even); FP32 output needs ldd < 2^23 (else
 *                   FGB_EUNSUPPORTED).  accumulate != 0 (FP32 only):
 *                   D += A * B^T.
 *   mode          : FGB_GEMM_EXACT -- each code times its scale 2^(byte-127)
 *                   (byte 0 included, meaning 2^-127) becomes a bf16, products
 *                   are exact and summed in FP32 (round to nearest even),
 *                   matching an FP32 accumulation of the dequantized operands.
 *                   The bf16 step is exact whenever the scaled value has a
 *                   bf16 representation: always for 1x128 and 128x128 scales
 *                   (exponents >= -22); with 1x32 scale exponents below -123
 *                   codes of small magnitude round to the nearest bf16.  FGB_GEMM_FAST -- the FP8
 *                   matrix unit with E8M0 scales, twice the rate; within
 *                   each run of 8 consecutive K its products are summed
 *                   with each cut (toward zero) to 13 bits below the run's
 *                   largest, so |error| <= 2^-10 * sum over runs of the
 *                   run's largest |scaled product| plus FP32 rounding.
 *   workspace     : unused, may be NULL (ws_bytes ignored).
 * 256 * lda and 256 * ldb below 2^32 (when K > 0).
 */
int fp8_block_gemm(const uint8_t *a, const uint8_t *sa, int a_gran, const uint8_t *b,
                   const uint8_t *sb, int b_gran, const float *b_l1, int64_t g1, int64_t M,
                   int64_t N, int64_t K, int64_t lda, int64_t ldb, void *d, int d_dtype,
                   int64_t ldd, int accumulate, int mode, void *workspace, size_t ws_bytes,
                   void *stream);

/*
 * fp8_block_gemm_fmt -- fp8_block_gemm with each operand's element format
 * chosen: a_fmt = FGB_E4M3 or FGB_E5M2 (a gradient in E5M2, [MOSS] §3, as A
 * of Dgrad dY x W or Wgrad dY^T x X), b_fmt = FGB_E4M3.  An E5M2 A needs
 * a_gran = FGB_ROW1x128, b_gran = FGB_BLOCK128 or FGB_ROW1x128 and no b_l1.
 * In FGB_GEMM_EXACT mode E5M2 values times their power-of-two scale are
 * exact in bf16 as E4M3 ones are, so the result is again the FP32
 * accumulation of exact products; FGB_GEMM_FAST feeds the codes to the
 * matrix unit as E5M2.  Other arguments as fp8_block_gemm (no workspace).
 */
int fp8_block_gemm_fmt(const uint8_t *a, const uint8_t *sa, int a_gran, int a_fmt, const uint8_t *b,
                       const uint8_t *sb, int b_gran, int b_fmt, const float *b_l1, int64_t g1, int64_t M,
                       int64_t N, int64_t K, int64_t lda, int64_t ldb, void *d, int d_dtype, int64_t ldd,
                       int accumulate, int mode, void *stream);

/*
 * fp8_grouped_gemm_masked -- the masked grouped layout of [DSV3] §5.6: each
 * expert owns a fixed block of M_max rows of which only the first
 * masked_m[e] are valid (the count is known on the device only, as after a
 * low-latency dispatch for decode).
 *   a  [G, M_max, K] codes, sa [G, M_max, K/128] (1x128 scales), dense
 *   b  [G, N, K] codes, sb [G, ceil(N/128), K/128] (128x128 scales), dense
 *   masked_m : device int32 [G]; values are clamped to [0, M_max]
 *   d  [G, M_max, N] dense, FGB_BF16 or FGB_F32 (FP32: N < 2^23); for each
 *      expert e only rows [0, masked_m[e]) are computed and written.
 *   mode as for fp8_block_gemm.  K % 128 == 0.
 */
int fp8_grouped_gemm_masked(const uint8_t *a, const uint8_t *sa, const uint8_t *b, const uint8_t *sb,
                            const int32_t *masked_m, int G, int64_t M_max, int64_t N, int64_t K, void *d,
                            int d_dtype, int mode, void *stream);

/*
 * fp8_grouped_gemm -- M-grouped contiguous FP8 GEMM for MoE experts ([DSV3]
 * §5.6: experts concatenated along M, each expert's 128x128 weight scales
 * picked by its group; [FLOW] assumption 2: the expert linears emit BF16).
 *   a  [M_cap, K] codes, sa [M_cap, K/128] (1x128 scales), dense
 *   b  [G, N, K] codes, sb [G, ceil(N/128), K/128] (128x128 scales), dense
 *   group_offsets : device int32 [G+1], non-decreasing, off[0] = 0,
 *                   off[G] <= M_cap (as written by permute_pad).  Rows
 *                   [off[g], off[g+1]) use expert g.  Read on the device:
 *                   no host synchronisation.
 *   d  [M_cap, N], dense, FGB_BF16 or FGB_F32 (FP32: N < 2^23).  Rows >=
 *      off[G] are neither read nor written.
 *   mode: FGB_GEMM_EXACT or FGB_GEMM_FAST as for fp8_block_gemm.
 * K % 128 == 0.
 */
int fp8_grouped_gemm(const uint8_t *a, const uint8_t *sa, const uint8_t *b, const uint8_t *sb,
                     const int32_t *group_offsets, int G, int64_t M_cap, int64_t N, int64_t K,
                     void *d, int d_dtype, int mode, void *stream);

/*
 * fp8_kgrouped_gemm -- K-grouped FP8 GEMM, the Wgrad of the MoE experts
 * ([DSV3] §1: Wgrad multiplies dY^T by X, here per expert; §5.6 grouped
 * layouts with the experts concatenated along K).  For each expert e,
 *   D_e = A[:, koff[e]:koff[e+1]] * B[:, koff[e]:koff[e+1]]^T,
 * with 1x128 scales on both operands (both as written by
 * fp8_grouped_direct_transpose) and FP32 accumulation as in fp8_block_gemm.
 *   a  [M, K_cap] codes, sa [M, K_cap/128] scales, dense (A_e = dY_e^T)
 *   b  [N, K_cap] codes, sb [N, K_cap/128] scales, dense (B_e = X_e^T)
 *   k_offsets : device int32 [G+1], non-decreasing multiples of 128,
 *               k_offsets[0] >= 0, k_offsets[G] <= K_cap (as written by
 *               fp8_grouped_direct_transpose).  Read on the device: no host
 *               synchronisation and no check of these conditions.
 *   d  [G, M, N] dense, FGB_F32 (N < 2^23) or FGB_BF16; an expert with an empty range
 *      gets D_e = 0 (or keeps D_e when accumulating).  accumulate != 0
 *      (FP32 only): D_e += A_e * B_e^T.
 *   mode: FGB_GEMM_EXACT or FGB_GEMM_FAST as for fp8_block_gemm.
 * K_cap % 128 == 0, 256 * K_cap below 2^32, 1 <= G <= 1024; a and b 16-byte
 * aligned.  One kernel on `stream`.
 */
int fp8_kgrouped_gemm(const uint8_t *a, const uint8_t *sa, const uint8_t *b, const uint8_t *sb,
                      const int32_t *k_offsets, int G, int64_t M, int64_t N, int64_t K_cap, void *d,
                      int d_dtype, int accumulate, int mode, void *stream);

/*
 * permute_pad -- fused permute + pad ([FLOW] "Core method": expert reordering
 * fused with 16-aligned padding, on row-wise FP8 with its scales).
 *   xq [T, H] codes, xs [T, H/128] scales, topk_idx [T, topk] int32 (device)
 *   Rows are grouped by expert id ascending and, inside an expert, by
 *   (token, slot) ascending; each expert's segment is padded at its end to a
 *   multiple of pad_multiple rows with code 0x00 and scale byte 105 (the
 *   scale the 1x128 rule gives an all-zero tile, so padding never raises a
 *   block-max scale when a segment is transposed).  A slot
 *   whose id lies outside [0, G) is dropped (row_map = -1).
 *   out_q [M_cap, H], out_s [M_cap, H/128]: rows >= off[G] untouched.
 *   row_map [T, topk] int32: destination row of each slot, or -1.
 *   group_offsets [G+1] int32: segment starts (multiples of pad_multiple).
 *   M_cap must be >= T*topk + (pad_multiple-1)*G (the host-side bound).
 *   workspace: device memory of permute_pad_workspace_size(T, topk, G)
 *   bytes; its contents on entry do not matter.
 * H % 128 == 0, 1 <= G <= 1024, pad_multiple in [1, 256].
 */
int permute_pad(const uint8_t *xq, const uint8_t *xs, const int32_t *topk_idx, int64_t T, int topk,
                int G, int64_t H, int pad_multiple, uint8_t *out_q, uint8_t *out_s,
                int32_t *row_map, int32_t *group_offsets, int64_t M_cap, void *workspace,
                size_t ws_bytes, void *stream);

/* Workspace bytes permute_pad needs for these sizes. */
size_t permute_pad_workspace_size(int64_t T, int topk, int G);

/* Size of the scratch array that permute_pad_noalloc uses on each GPU. */
#define FGB_PERMUTE_PAD_NOALLOC_SCRATCH_BYTES (1 << 20)

/*
 * permute_pad_noalloc -- permute_pad for callers that cannot allocate device
 * memory (code under HIP graph capture, tight serving loops, harnesses that
 * forbid hipMalloc): the same kernels and the same outputs, bit for bit, with
 * the workspace taken from a scratch array of FGB_PERMUTE_PAD_NOALLOC_SCRATCH_BYTES
 * (1 MiB) that the library holds on each GPU it runs on, from the first call
 * on that GPU until the process ends.  The call allocates nothing (no
 * hipMalloc, hipFree or allocating library routine); the caller passes every
 * input and output, as for permute_pad.
 *   Arguments: as permute_pad, without workspace and ws_bytes.
 *   Limit: permute_pad_workspace_size(T, topk, G) <= 1 MiB, i.e.
 *          2*ceil(T/256)*G + G <= 262144 (e.g. T <= 1,048,320 tokens at G = 32);
 *          larger sizes return FGB_EWORKSPACE before anything is enqueued.
 *   Concurrency: every call on one GPU shares that GPU's scratch array (its
 *          contents on entry do not matter: every word is written before it is
 *          read), so calls that overlap in time on one GPU -- on different
 *          streams, or from different threads -- race; calls on one stream are
 *          ordered and safe.
 *   Errors: as permute_pad; FGB_EHIP if the scratch address cannot be looked up.
 */
int permute_pad_noalloc(const uint8_t *xq, const uint8_t *xs, const int32_t *topk_idx, int64_t T, int topk,
                        int G, int64_t H, int pad_multiple, uint8_t *out_q, uint8_t *out_s, int32_t *row_map,
                        int32_t *group_offsets, int64_t M_cap, void *stream);

/*
 * unpermute_unpad -- inverse of permute_pad on the expert output ([FLOW]
 * "Core method": fused unpermute + unpadding).
 *   out[t][h] = bf16_rne( fold k = 0..topk-1 of acc = fmaf(w, y[row_map[t][k]][h], acc) )
 *   with acc starting at 0, w = probs[t][k] (or 1 when probs == NULL), slots
 *   with row_map < 0 skipped; padding rows are never read.
 *   y [*, H] bf16 dense; row_map [T, topk] int32; probs [T, topk] fp32 or
 *   NULL; out [T, H] bf16 dense.  H % 8 == 0.
 */
int unpermute_unpad(const void *y, const int32_t *row_map, const float *probs, int64_t T,
                    int topk, int64_t H, void *out, void *stream);

/*
 * unpermute_backward -- gradient of unpermute_unpad for the MoE expert
 * backward ([FLOW] "Core method", the fused unpermute): out[t] = sum_k
 * w[t,k] * y[row_map[t,k]] gives dy[row_map[t,k]] = bf16(fp32(w[t,k] *
 * dout[t])) (round to nearest even; w = 1 when probs is NULL); rows that no
 * slot maps to (the padding) are written as zeros.
 *   dout bf16 [T, H]; row_map, probs [T, topk] (device); dy bf16 [M_cap, H].
 *   workspace: >= unpermute_backward_workspace_size(M_cap) bytes (an inverse
 *   map), caller-owned, contents on entry irrelevant.  H % 8 == 0, topk <= 64;
 *   dout and dy 16-byte aligned.  Three kernels on `stream`.
 */
int unpermute_backward(const void *dout, const int32_t *row_map, const float *probs, int64_t T, int topk,
                       int64_t H, int64_t M_cap, void *dy, void *workspace, size_t ws_bytes, void *stream);
size_t unpermute_backward_workspace_size(int64_t M_cap);

/*
 * unpermute_backward_quant -- unpermute_backward followed by 1x128
 * quantization of its bf16 rows, in one pass ([FLOW] "Core method": the
 * expert path stays in FP8 from the boundary on; the expert backward's two
 * GEMMs read dy only as 1x128 FP8).  Bit for bit fp8_quant_rowwise of the dy
 * unpermute_backward writes: padding and unreferenced rows become code 0x00
 * with scale byte 105.  q [M_cap, H], s [M_cap, H/128] dense; H % 128 == 0;
 * workspace as for unpermute_backward; dout and q 16-byte aligned.
 */
int unpermute_backward_quant(const void *dout, const int32_t *row_map, const float *probs, int64_t T, int topk,
                             int64_t H, int64_t M_cap, uint8_t *q, uint8_t *s, void *workspace, size_t ws_bytes,
                             void *stream);

/*
 * swiglu_quant -- fused SwiGLU + 1x128 quantization ([FLOW] "Core method":
 * the activation emits FP8 directly; assumption 2: the first linear's
 * output is BF16).
 *   h [M, 2F] bf16, ld ldh, gate columns [0, F), up columns [F, 2F).
 *   a = (g / (1 + exp(-g))) * u, each operation rounded to fp32; exp is the
 *   library's own fp32 function (Cody-Waite reduction with a two-part ln2,
 *   degree-7 Taylor polynomial in Horner form with fused multiply-adds,
 *   scaling by 2^n in two exact steps), so results are reproducible
 *   bit for bit.  Then 1x128 quantization of a into q [M, F] (dense) and
 *   s [M, F/128] (dense).
 *   group_offsets: NULL, or device int32 [G+1]; rows >= off[G] are skipped.
 * F % 128 == 0.
 */
int swiglu_quant(const void *h, int64_t M, int64_t F, int64_t ldh, const int32_t *group_offsets,
                 int G, uint8_t *q, uint8_t *s, void *stream);

/*
 * swiglu_quant_cache -- swiglu_quant that also writes, from the same read of
 * h, the FP8 copy of its input the backward recomputes the activation from
 * ([DSV3] §3, low-precision activations: the SwiGLU input is cached in FP8).
 * q, s as in swiglu_quant; hq [M, 2F] and hs [M, 2F/128] (dense) are the
 * 1x128 quantization of the row [g | u] by the rule of fp8_quant_rowwise,
 * bit for bit (the hq, hs that dswiglu_quant reads).  Rows >= off[G] are
 * not written.  h, q and hq 16-byte aligned; F % 128 == 0.
 */
int swiglu_quant_cache(const void *h, int64_t M, int64_t F, int64_t ldh, const int32_t *group_offsets,
                       int G, uint8_t *q, uint8_t *s, uint8_t *hq, uint8_t *hs, void *stream);

/*
 * dswiglu_quant -- SwiGLU backward from the FP8-cached input, emitting FP8
 * ([DSV3] §3, low-precision activations: the MoE SwiGLU input is cached in
 * FP8 and the activation recomputed in the backward pass; [FLOW] "Core
 * method": activation boundaries emit FP8).  With g, u the dequantized cached
 * input and da the gradient of a = silu(g) * u, each operation one fp32
 * rounding in this order:
 *   e = exp(-g) (the library exponential of swiglu_quant), d = 1 + e,
 *   sg = 1 / d, silu = g / d, du = da * silu,
 *   dsilu = sg * (1 + g * (1 - sg)), dg = (da * u) * dsilu;
 * then 1x128 quantization (the rule of fp8_quant_rowwise) of the row [dg | du].
 *   hq [M, 2F] codes (gate first) with hs [M, 2F/128] 1x128 scales; da bf16
 *   [M, F]; dq [M, 2F], ds [M, 2F/128]; all dense; F % 128 == 0.
 *   group_offsets (device, may be NULL) as in swiglu_quant: rows >= offsets[G]
 *   are not written.  da 16-byte, hq and dq 8-byte aligned.
 */
int dswiglu_quant(const uint8_t *hq, const uint8_t *hs, const void *da, int64_t M, int64_t F,
                  const int32_t *group_offsets, int G, uint8_t *dq, uint8_t *ds, void *stream);

/*
 * swiglu_f32, dswiglu_f32 -- diagnostic forms of swiglu_quant and
 * dswiglu_quant: the same per-element fp32 arithmetic (the operations and
 * order declared above), on fp32 inputs given directly and without the
 * quantization, so that the values before rounding to FP8 can be compared
 * bit for bit.
 *   swiglu_f32:  a[i] = (g[i] / (1 + exp(-g[i]))) * u[i].
 *   dswiglu_f32: du[i], dg[i] of dswiglu_quant for g[i], u[i] and the
 *                gradient da[i].
 *   All arrays are device fp32 [n], dense; outputs may not alias inputs.
 *   Errors: FGB_EINVAL for n < 0 or a null pointer (n > 0).
 */
int swiglu_f32(const float *g, const float *u, int64_t n, float *a, void *stream);
int dswiglu_f32(const float *g, const float *u, const float *da, int64_t n, float *du, float *dg, void *stream);

/*
 * mx2_quant -- MOSS two-level microscaling ([MOSS] §3 two-level
 * microscaling, Fig. 2): level 1 is an FP32 factor alpha1 per g1 contiguous
 * elements of a row (last group partial), alpha1 = fp32(amax / 448), or 1
 * for an all-zero group; y = fp32(x / alpha1) (correctly rounded division);
 * level 2 is an E8M0 scale per 32 elements of y (floor -127); elements E4M3.
 *   x [R, C] bf16 dense; q [R, C]; s2 [R, C/32]; s1 [R, ceil(C/g1)] fp32.
 * C % 32 == 0, g1 % 32 == 0.
 */
int mx2_quant(const void *x, int64_t R, int64_t C, int64_t g1, uint8_t *q, uint8_t *s2, float *s1,
              void *stream);

/*
 * mx2_quant_rule -- mx2_quant with the level-2 exponent rule chosen: rule =
 * FGB_SCALE_CEIL (mx2_quant) or FGB_SCALE_OCP_FLOOR, the MX standard's
 * floor(log2 amax32) - 8 ([MOSS] §3 names the MX standard for k2 = 32),
 * codes clipped at 448.
 */
int mx2_quant_rule(const void *x, int64_t R, int64_t C, int64_t g1, int rule, uint8_t *q, uint8_t *s2, float *s1,
                   void *stream);

/*
 * mx2_dequant -- x_hat = fp32( fp32(decode(q) * 2^(s2 - 127)) * alpha1 ).
 *   out [R, C] fp32 dense.
 */
int mx2_dequant(const uint8_t *q, const uint8_t *s2, const float *s1, int64_t R, int64_t C,
                int64_t g1, float *out, void *stream);

/* access patterns of fgb_hbm_probe */
#define FGB_PROBE_COPY 0
#define FGB_PROBE_READ 1
#define FGB_PROBE_FILL 2
#define FGB_PROBE_STRIDED_READ 3
#define FGB_PROBE_STRIDED_WRITE 4

/*
 * fgb_hbm_probe -- diagnostic, not part of the method: plain byte movement in
 * the access patterns of the data-movement kernels, with their 16-byte
 * nontemporal loads and stores, so that each kernel's bandwidth can be set
 * beside what its pattern sustains on the same device.  src and dst are
 * device buffers of rows * cols bytes (rows % 128 == 0, cols % 128 == 0),
 * 16-byte aligned, not overlapping:
 *   FGB_PROBE_COPY          dst = src;
 *   FGB_PROBE_READ          dst[16*b .. 16*b+15] = XOR of the 16-byte words of
 *                           src[4096*b .. 4096*b+4095] (dst needs rows*cols/256
 *                           bytes);
 *   FGB_PROBE_FILL          dst = 0 (src unused, may be null);
 *   FGB_PROBE_STRIDED_READ  src read as [rows, cols] by 128x128 blocks, the
 *                           way the direct transpose reads its codes (16
 *                           rows of 16 bytes per lane, 8 lanes per 128-byte
 *                           row piece); block b = tb + (rows/128)*cb written
 *                           to dst[16384*b ..] as 16 rows of 1 KB, row j of
 *                           the lane's 16 at dst[16384*b + 1024*j + 16*lane];
 *   FGB_PROBE_STRIDED_WRITE the inverse map: dst as [rows, cols] written by
 *                           128-byte row pieces from contiguous src blocks.
 * One kernel on `stream`; FGB_EINVAL / FGB_EUNSUPPORTED on bad arguments.
 */
int fgb_hbm_probe(const void *src, void *dst, int64_t rows, int64_t cols, int pattern, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* FGB_H */
