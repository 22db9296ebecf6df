/*
 * fgb_oracle.c -- plain, slow, single-threaded CPU oracle for the fine-grained
 * blockwise FP8 path.  TEST INFRASTRUCTURE ONLY: nothing in the product library
 * links, includes or calls this file; only the tests, the smoke check and the
 * bench's CPU-baseline leg load it.  It shares no code, header, table or
 * constant with the HIP kernels.
 *
 * Build: gcc -O2 -ffp-contract=off -fno-fast-math -fPIC -shared (see build.py).
 * Floating point: fp64 wherever the pages leave the precision open; fp32 where
 * the operation is defined as a sequence of fp32 roundings (the SwiGLU
 * activation, the MOSS level-1 scale and division, the unpermute fold).
 *
 * Sources (page title + section), cited per function:
 *   [DSV3]  llm-infra-atlas, "01 · DeepSeek FP8 and DeepGEMM: Hopper software recipe"
 *   [LP]    llm-infra-atlas, "Low precision" chapter index
 *   [FLOW]  awesome-system-papers, "FP8-Flow-MoE: A Casting-Free FP8 Recipe without
 *           Double Quantization Error (MLSys 2026)"
 *   [MOSS]  xllm-io paper review, "MOSS: Efficient and Accurate FP8 LLM Training with
 *           Microscaling and Automatic Scaling"
 *
 * Parity status: every function below is pinned by a CPU test against an
 * independent check (exhaustive tables, brute force, closed forms, exact
 * integer arithmetic).  The only readings without a printed value to pin are
 * listed in the design notes (routing distribution, exp coefficients).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORC_F32 0
#define ORC_BF16 1
#define ORC_ROW1x128 0
#define ORC_ROW1x32 1
#define ORC_BLOCK128 2

/* ------------------------------------------------------------------------ */
/* Element formats.  [LP] §2 format table: E4M3 is 1 sign / 4 exponent /    */
/* 3 mantissa bits, largest magnitude 448, no infinity.  [MOSS] §3 data-    */
/* format table gives the same E4M3 range.  Bias 7 and the single NaN       */
/* pattern S.1111.111 follow from "448, no Inf" (OCP E4M3FN).               */
/* ------------------------------------------------------------------------ */

/* Value of an E4M3 code, exactly, in double. */
double orc_e4m3_decode(uint8_t c)
{
    int s = c >> 7, E = (c >> 3) & 15, m = c & 7;
    if (E == 15 && m == 7)
        return NAN;
    double mag = (E == 0) ? ldexp((double)m, -9) : ldexp((double)(8 + m), E - 10);
    return s ? -mag : mag;
}

/* Round a real value to E4M3: nearest representable value, ties to the code
 * whose mantissa LSB is even, magnitudes at or above 448 saturate to 448, and
 * the sign is kept (so -0 and negative underflow give 0x80).  The rounding
 * rule (round-to-nearest-even with saturation) is the one the method fixes for
 * its FP8 casts. */
uint8_t orc_e4m3_encode(double v)
{
    uint8_t sign = signbit(v) ? 0x80 : 0x00;
    double a = fabs(v);
    if (a >= 448.0)
        return sign | 0x7E;
    /* spacing of representable values near a: 2^(x-3) in the normal binade
     * [2^x, 2^(x+1)) with x >= -6; 2^-9 below 2^-6 (subnormals). */
    int fx;
    frexp(a, &fx); /* a in [2^(fx-1), 2^fx) */
    int x = fx - 1;
    double quantum = (a >= ldexp(1.0, -6)) ? ldexp(1.0, x - 3) : ldexp(1.0, -9);
    double n = nearbyint(a / quantum); /* a/quantum is exact; default mode = nearest-even */
    double r = n * quantum;            /* rounded magnitude, exact */
    if (r == 0.0)
        return sign;
    if (r < ldexp(1.0, -6))
        return sign | (uint8_t)(r / ldexp(1.0, -9)); /* subnormal: m = r / 2^-9 */
    int rx;
    frexp(r, &rx);
    int e = rx - 1;                                  /* r in [2^e, 2^(e+1)) */
    int m = (int)(r / ldexp(1.0, e - 3)) - 8;        /* 8..15 -> 0..7 */
    return sign | (uint8_t)(((e + 7) << 3) | m);
}

/* bf16 bit pattern -> value (a bf16 is the upper half of an fp32). */
static double bf16_value(uint16_t h)
{
    uint32_t u = (uint32_t)h << 16;
    float f;
    memcpy(&f, &u, 4);
    return (double)f;
}

/* fp32 -> bf16 bits, round to nearest even (finite inputs). */
static uint16_t bf16_round(float f)
{
    uint32_t u;
    memcpy(&u, &f, 4);
    uint32_t lsb = (u >> 16) & 1u;
    u += 0x7FFFu + lsb;
    return (uint16_t)(u >> 16);
}

static double load_elem(const void *x, int dtype, int64_t idx)
{
    if (dtype == ORC_F32)
        return (double)((const float *)x)[idx];
    return bf16_value(((const uint16_t *)x)[idx]);
}

/* ------------------------------------------------------------------------ */
/* Scale rule.  [DSV3] §3: the scaling factor is amax/448 with amax clamped */
/* below at 1e-4; [DSV3] §8: the UE8M0 variant rounds the factor up to a    */
/* power of two.  Together: S = 2^e with e the smallest integer such that   */
/* amax <= 448 * 2^e, never below a floor.  The 1e-4 clamp is the floor     */
/* e >= -22 (1e-4/448 lies between 2^-23 and 2^-22).  For the MX level-2    */
/* scale the floor is the E8M0 range, e >= -127 ([MOSS] §3 two-level        */
/* microscaling; [LP] §2 MXFP8 row).  Stored byte: e + 127.                 */
/* ------------------------------------------------------------------------ */
int orc_scale_exp(double amax, int emin)
{
    if (!(amax > 0.0))
        return emin;
    int e = (int)ceil(log2(amax / 448.0));
    while (ldexp(448.0, e) < amax)
        e++;
    while (ldexp(448.0, e - 1) >= amax)
        e--;
    return e < emin ? emin : e;
}

/* Bulk encode of fp32 values (used by the codec pins). */
void orc_e4m3_encode_f32(const float *x, int64_t n, uint8_t *q)
{
    for (int64_t i = 0; i < n; i++)
        q[i] = orc_e4m3_encode((double)x[i]);
}

void orc_e4m3_decode_all(double *out256)
{
    for (int c = 0; c < 256; c++)
        out256[c] = orc_e4m3_decode((uint8_t)c);
}

void orc_scale_exp_f32(const float *amax, int64_t n, int emin, int32_t *e)
{
    for (int64_t i = 0; i < n; i++)
        e[i] = orc_scale_exp((double)amax[i], emin);
}

/* ------------------------------------------------------------------------ */
/* Format variants.  [LP] §2 format table: E5M2 is 1 sign / 5 exponent /    */
/* 2 mantissa bits, largest finite magnitude 57344, with infinity; [MOSS]   */
/* §3 uses it for backward-pass gradients.  Bias 15 and the Inf/NaN codes   */
/* (exponent field 31) follow from "57344, has Inf" (OCP E5M2).             */
/* ------------------------------------------------------------------------ */
#define ORC_E4M3 0
#define ORC_E5M2 1
#define ORC_SCALE_CEIL 0
#define ORC_SCALE_OCP_FLOOR 1

/* Value of an E5M2 code, exactly, in double. */
double orc_e5m2_decode(uint8_t c)
{
    int s = c >> 7, E = (c >> 2) & 31, m = c & 3;
    double mag;
    if (E == 31)
        mag = m ? NAN : INFINITY;
    else
        mag = (E == 0) ? ldexp((double)m, -16) : ldexp((double)(4 + m), E - 17);
    return s ? -mag : mag;
}

/* Round a real value to E5M2: nearest representable value, ties to the even
 * mantissa, magnitudes at or above 57344 clipped to 57344 (the pages'
 * quantize clips to the format's largest value), sign kept. */
uint8_t orc_e5m2_encode(double v)
{
    uint8_t sign = signbit(v) ? 0x80 : 0x00;
    double a = fabs(v);
    if (a >= 57344.0)
        return sign | 0x7B;
    /* spacing: 2^(x-2) in the normal binade [2^x, 2^(x+1)), x >= -14;
     * 2^-16 below 2^-14 (subnormals) */
    int fx;
    frexp(a, &fx);
    int x = fx - 1;
    double quantum = (a >= ldexp(1.0, -14)) ? ldexp(1.0, x - 2) : ldexp(1.0, -16);
    double r = nearbyint(a / quantum) * quantum;
    if (r == 0.0)
        return sign;
    if (r < ldexp(1.0, -14))
        return sign | (uint8_t)(r / ldexp(1.0, -16));
    int rx;
    frexp(r, &rx);
    int e = rx - 1;
    if (e > 15)
        return sign | 0x7B;
    int m = (int)(r / ldexp(1.0, e - 2)) - 4; /* 4..7 -> 0..3 */
    return sign | (uint8_t)(((e + 15) << 2) | m);
}

double orc_fp8_decode(uint8_t c, int fmt) { return fmt == ORC_E5M2 ? orc_e5m2_decode(c) : orc_e4m3_decode(c); }
uint8_t orc_fp8_encode(double v, int fmt) { return fmt == ORC_E5M2 ? orc_e5m2_encode(v) : orc_e4m3_encode(v); }

void orc_fp8_encode_f32(const float *x, int64_t n, int fmt, uint8_t *q)
{
    for (int64_t i = 0; i < n; i++)
        q[i] = orc_fp8_encode((double)x[i], fmt);
}

void orc_fp8_decode_all(int fmt, double *out256)
{
    for (int c = 0; c < 256; c++)
        out256[c] = orc_fp8_decode((uint8_t)c, fmt);
}

/* Scale exponent of an amax for an element format and a rule.
 *   ORC_SCALE_CEIL: the rule used everywhere else in this path, with the
 *     element format's largest value: the smallest e with amax <= max * 2^e
 *     ([DSV3] §3 and §8 with max = 448, or 57344 for E5M2).
 *   ORC_SCALE_OCP_FLOOR: the rule of the MX standard that [MOSS] §3 names for
 *     its 32-element level: e = floor(log2 amax) - emax, emax the exponent of
 *     the format's largest normal (8 for E4M3, 15 for E5M2); scaled values
 *     above the largest finite value then clip in the encoder.
 * Both are floored at emin; an all-zero group gets emin. */
int orc_scale_exp_fmt(double amax, int fmt, int rule, int emin)
{
    if (!(amax > 0.0))
        return emin;
    int e;
    if (rule == ORC_SCALE_OCP_FLOOR) {
        int fx;
        frexp(amax, &fx); /* amax in [2^(fx-1), 2^fx) */
        e = (fx - 1) - (fmt == ORC_E5M2 ? 15 : 8);
    } else {
        double mx = fmt == ORC_E5M2 ? 57344.0 : 448.0;
        e = (int)ceil(log2(amax / mx));
        while (ldexp(mx, e) < amax)
            e++;
        while (ldexp(mx, e - 1) >= amax)
            e--;
    }
    return e < emin ? emin : e;
}

void orc_scale_exp_fmt_f32(const float *amax, int64_t n, int fmt, int rule, int emin, int32_t *e)
{
    for (int64_t i = 0; i < n; i++)
        e[i] = orc_scale_exp_fmt((double)amax[i], fmt, rule, emin);
}

/* 1 x g quantization in a chosen element format and scale rule (the
 * gradient form of [MOSS] §3 uses E5M2; the 1e-4 amax clamp of [DSV3] §3
 * becomes the floor emin = -22 for E4M3 and -29 for E5M2 with 128-element
 * groups, -127 (E8M0) with 32-element groups). */
void orc_quant_rowwise_fmt(const void *x, int dtype, int64_t rows, int64_t cols, int64_t ldx, int group,
                           int fmt, int rule, int emin, uint8_t *q, int64_t ldq, uint8_t *s, int64_t lds)
{
    for (int64_t r = 0; r < rows; r++) {
        for (int64_t j = 0; j < cols / group; j++) {
            double amax = 0.0;
            for (int64_t k = 0; k < group; k++) {
                double v = fabs(load_elem(x, dtype, r * ldx + j * group + k));
                if (v > amax)
                    amax = v;
            }
            int e = orc_scale_exp_fmt(amax, fmt, rule, emin);
            for (int64_t k = 0; k < group; k++)
                q[r * ldq + j * group + k] = orc_fp8_encode(ldexp(load_elem(x, dtype, r * ldx + j * group + k), -e), fmt);
            s[r * lds + j] = (uint8_t)(e + 127);
        }
    }
}

/* decode(q) * 2^(s - 127) in the given format (row-wise 1 x g scales). */
void orc_dequant_fmt(const uint8_t *q, const uint8_t *s, int group, int fmt, int64_t rows, int64_t cols,
                     double *out)
{
    for (int64_t r = 0; r < rows; r++)
        for (int64_t c = 0; c < cols; c++)
            out[r * cols + c] = ldexp(orc_fp8_decode(q[r * cols + c], fmt), (int)s[r * (cols / group) + c / group] - 127);
}

/* The direct transpose of orc_direct_transpose for codes of format fmt:
 * dequantize, requantize at the 128x128 block's largest scale. */
void orc_direct_transpose_fmt(const uint8_t *q, const uint8_t *s, int64_t T, int64_t C, int fmt,
                              uint8_t *qt, uint8_t *st)
{
    for (int64_t tb = 0; tb < T / 128; tb++)
        for (int64_t cb = 0; cb < C / 128; cb++) {
            int emax = 0;
            for (int64_t t = tb * 128; t < tb * 128 + 128; t++) {
                int e = (int)s[t * (C / 128) + cb] - 127;
                if (t == tb * 128 || e > emax)
                    emax = e;
            }
            for (int64_t t = tb * 128; t < tb * 128 + 128; t++) {
                int e = (int)s[t * (C / 128) + cb] - 127;
                for (int64_t c = cb * 128; c < cb * 128 + 128; c++)
                    qt[c * T + t] = orc_fp8_encode(ldexp(orc_fp8_decode(q[t * C + c], fmt), e - emax), fmt);
            }
            for (int64_t c = cb * 128; c < cb * 128 + 128; c++)
                st[c * (T / 128) + tb] = (uint8_t)(emax + 127);
        }
}

/* ------------------------------------------------------------------------ */
/* 1 x g activation quantization.  [DSV3] §2 (online quantization: amax per */
/* 1x128 activation tile, computed at run time) and §3 (1x128 tiles = per   */
/* token per 128 channels; scale tensor [T, C/128]).  g = 32 is the MX      */
/* single-level activation scaling of [MOSS] §3 training flow.              */
/*   x: [rows, cols] (ld ldx), fp32 or bf16; q: [rows, cols] (ld ldq);      */
/*   s: [rows, cols/g] (ld lds).  emin = -22 for g = 128, -127 for g = 32.  */
/* ------------------------------------------------------------------------ */
void orc_quant_rowwise(const void *x, int dtype, int64_t rows, int64_t cols, int64_t ldx,
                       int group, int emin, uint8_t *q, int64_t ldq, uint8_t *s, int64_t lds)
{
    for (int64_t r = 0; r < rows; r++) {
        for (int64_t j = 0; j < cols / group; j++) {
            double amax = 0.0;
            for (int64_t k = 0; k < group; k++) {
                double v = fabs(load_elem(x, dtype, r * ldx + j * group + k));
                if (v > amax)
                    amax = v;
            }
            int e = orc_scale_exp(amax, emin);
            for (int64_t k = 0; k < group; k++) {
                double v = load_elem(x, dtype, r * ldx + j * group + k);
                q[r * ldq + j * group + k] = orc_e4m3_encode(ldexp(v, -e));
            }
            s[r * lds + j] = (uint8_t)(e + 127);
        }
    }
}

/* ------------------------------------------------------------------------ */
/* 128 x 128 weight-block quantization.  [DSV3] §3: weights are grouped per */
/* 128 input channels x 128 output channels; scale tensor                   */
/* [Cout/128, Cin/128].  A partial last row block uses the rows present.    */
/* ------------------------------------------------------------------------ */
void orc_quant_blockwise(const void *w, int dtype, int64_t rows, int64_t cols, int64_t ldw,
                         uint8_t *q, int64_t ldq, uint8_t *s, int64_t lds)
{
    for (int64_t rb = 0; rb < (rows + 127) / 128; rb++) {
        int64_t r0 = rb * 128, r1 = r0 + 128 < rows ? r0 + 128 : rows;
        for (int64_t cb = 0; cb < cols / 128; cb++) {
            double amax = 0.0;
            for (int64_t r = r0; r < r1; r++)
                for (int64_t c = cb * 128; c < cb * 128 + 128; c++) {
                    double v = fabs(load_elem(w, dtype, r * ldw + c));
                    if (v > amax)
                        amax = v;
                }
            int e = orc_scale_exp(amax, -22);
            for (int64_t r = r0; r < r1; r++)
                for (int64_t c = cb * 128; c < cb * 128 + 128; c++)
                    q[r * ldq + c] = orc_e4m3_encode(ldexp(load_elem(w, dtype, r * ldw + c), -e));
            s[rb * lds + cb] = (uint8_t)(e + 127);
        }
    }
}

/* Dequantization: value = decode(q) * 2^(s - 127), fp64 result.  The      */
/* multiplier convention is that of [DSV3] §3 (sf = amax/448 multiplies).   */
void orc_dequant(const uint8_t *q, const uint8_t *s, int gran, int64_t rows, int64_t cols,
                 double *out)
{
    int64_t g = gran == ORC_ROW1x32 ? 32 : 128;
    for (int64_t r = 0; r < rows; r++)
        for (int64_t c = 0; c < cols; c++) {
            int sb = (gran == ORC_BLOCK128) ? s[(r / 128) * (cols / 128) + c / 128]
                                            : s[r * (cols / g) + c / g];
            out[r * cols + c] = ldexp(orc_e4m3_decode(q[r * cols + c]), sb - 127);
        }
}

/* ------------------------------------------------------------------------ */
/* Scaling-aware direct transpose.  [FLOW] "Core method": with power-of-two */
/* scales the row-wise -> column-wise conversion is done inside each        */
/* 128x128 block by taking the block's largest scale and moving each code's */
/* exponent by k = log2(Smax / S) with mantissa recombination; [FLOW] key   */
/* observation 2 (align to the block's largest scale to avoid overflow).    */
/* Its defining property: the output equals requantizing the dequantized    */
/* block at the block-max scale, which is what this oracle computes.        */
/*   q: [rows=T, cols=C] row-wise codes, s: [T, C/128];                     */
/*   qt: [C, T], st: [C, T/128] (every entry of a 128x128 block equal).     */
/* ------------------------------------------------------------------------ */
void orc_direct_transpose(const uint8_t *q, const uint8_t *s, int64_t T, int64_t C,
                          uint8_t *qt, uint8_t *st)
{
    for (int64_t tb = 0; tb < T / 128; tb++)
        for (int64_t cb = 0; cb < C / 128; cb++) {
            int emax = 0;
            for (int64_t t = tb * 128; t < tb * 128 + 128; t++) {
                int e = (int)s[t * (C / 128) + cb] - 127;
                if (t == tb * 128 || e > emax)
                    emax = e;
            }
            for (int64_t t = tb * 128; t < tb * 128 + 128; t++) {
                int e = (int)s[t * (C / 128) + cb] - 127;
                for (int64_t c = cb * 128; c < cb * 128 + 128; c++) {
                    double v = ldexp(orc_e4m3_decode(q[t * C + c]), e); /* dequantize */
                    qt[c * T + t] = orc_e4m3_encode(ldexp(v, -emax));    /* requantize */
                }
            }
            for (int64_t c = cb * 128; c < cb * 128 + 128; c++)
                st[c * (T / 128) + tb] = (uint8_t)(emax + 127);
        }
}

/* ------------------------------------------------------------------------ */
/* The three-pass conversion the direct transpose replaces ([FLOW] "Core    */
/* method" and Fig. 1: dequantize, transpose, requantize).  Steps in that   */
/* order: x = decode(q) * 2^e (exact), x^T, then the 1x128 rule of          */
/* orc_quant_rowwise on the rows of x^T (power-of-two scales, floor -22).   */
/*   q: [T, C], s: [T, C/128] -> qt: [C, T], st: [C, T/128].                */
/* ------------------------------------------------------------------------ */
void orc_naive_transpose(const uint8_t *q, const uint8_t *s, int64_t T, int64_t C,
                         uint8_t *qt, uint8_t *st)
{
    double *xt = (double *)malloc((size_t)(T * C) * sizeof(double));
    for (int64_t t = 0; t < T; t++)
        for (int64_t c = 0; c < C; c++)
            xt[c * T + t] = ldexp(orc_e4m3_decode(q[t * C + c]), (int)s[t * (C / 128) + c / 128] - 127);
    for (int64_t c = 0; c < C; c++)
        for (int64_t j = 0; j < T / 128; j++) {
            double amax = 0.0;
            for (int64_t k = 0; k < 128; k++)
                if (fabs(xt[c * T + j * 128 + k]) > amax)
                    amax = fabs(xt[c * T + j * 128 + k]);
            int e = orc_scale_exp(amax, -22);
            for (int64_t k = 0; k < 128; k++)
                qt[c * T + j * 128 + k] = orc_e4m3_encode(ldexp(xt[c * T + j * 128 + k], -e));
            st[c * (T / 128) + j] = (uint8_t)(e + 127);
        }
    free(xt);
}

/* ------------------------------------------------------------------------ */
/* Non-power-of-two scaling, for the double-quantization study only.        */
/* [DSV3] §3: sf = amax / 448 is an fp32 multiplier per 1x128 tile (1 for   */
/* an all-zero tile); a code is E4M3(RN32(x / sf)) and decodes to           */
/* RN32(decode(code) * sf).  orc_naive_transpose_sf runs the three passes   */
/* with this rule (dequantized values kept in fp32).                        */
/*   x: [rows, cols] fp32; q: [rows, cols]; sf: [rows, cols/128] fp32.      */
/* ------------------------------------------------------------------------ */
void orc_quant_rowwise_sf(const float *x, int64_t rows, int64_t cols, uint8_t *q, float *sf)
{
    for (int64_t r = 0; r < rows; r++)
        for (int64_t j = 0; j < cols / 128; j++) {
            float amax = 0.0f;
            for (int64_t k = 0; k < 128; k++)
                if (fabsf(x[r * cols + j * 128 + k]) > amax)
                    amax = fabsf(x[r * cols + j * 128 + k]);
            float f = amax > 0.0f ? amax / 448.0f : 1.0f;
            for (int64_t k = 0; k < 128; k++) {
                float y = x[r * cols + j * 128 + k] / f;
                q[r * cols + j * 128 + k] = orc_e4m3_encode((double)y);
            }
            sf[r * (cols / 128) + j] = f;
        }
}

void orc_dequant_sf(const uint8_t *q, const float *sf, int64_t rows, int64_t cols, float *out)
{
    for (int64_t r = 0; r < rows; r++)
        for (int64_t c = 0; c < cols; c++)
            out[r * cols + c] = (float)orc_e4m3_decode(q[r * cols + c]) * sf[r * (cols / 128) + c / 128];
}

void orc_naive_transpose_sf(const uint8_t *q, const float *sf, int64_t T, int64_t C, uint8_t *qt,
                            float *sft)
{
    float *x = (float *)malloc((size_t)(T * C) * sizeof(float));
    float *xt = (float *)malloc((size_t)(T * C) * sizeof(float));
    orc_dequant_sf(q, sf, T, C, x);
    for (int64_t t = 0; t < T; t++)
        for (int64_t c = 0; c < C; c++)
            xt[c * T + t] = x[t * C + c];
    orc_quant_rowwise_sf(xt, C, T, qt, sft);
    free(x);
    free(xt);
}

/* ------------------------------------------------------------------------ */
/* Direct transpose of the expert segments of a permuted, padded activation */
/* (the expert backward's Wgrad contracts over each expert's own rows;      */
/* [FLOW] "Core method": the transpose is applied per 128x128 block).       */
/* Segment e = rows [off[e], off[e+1]) of q; its transpose fills columns    */
/* [koff[e], koff[e] + ceil(len_e/128)*128) of qt [C, Kc], with             */
/* koff[e+1] = koff[e] + ceil(len_e/128)*128.  Each block takes the largest */
/* scale over the rows present (the last block of a segment may be short); */
/* the columns of absent rows hold code 0.  st [C, Kc/128].                 */
/* Columns past koff[G] are not written.                                   */
/* ------------------------------------------------------------------------ */
void orc_grouped_direct_transpose(const uint8_t *q, const uint8_t *s, int64_t C, const int32_t *off,
                                  int G, uint8_t *qt, uint8_t *st, int64_t Kc, int32_t *koff)
{
    koff[0] = 0;
    for (int e = 0; e < G; e++) {
        int64_t len = off[e + 1] - off[e];
        koff[e + 1] = koff[e] + (int32_t)(((len + 127) / 128) * 128);
    }
    for (int e = 0; e < G; e++) {
        for (int64_t b = 0; b < (koff[e + 1] - koff[e]) / 128; b++) {
            int64_t t0 = off[e] + b * 128, n = off[e + 1] - t0 < 128 ? off[e + 1] - t0 : 128;
            int64_t kc = koff[e] + b * 128;
            for (int64_t cb = 0; cb < C / 128; cb++) {
                int emax = -1000;
                for (int64_t t = t0; t < t0 + n; t++) {
                    int ee = (int)s[t * (C / 128) + cb] - 127;
                    if (ee > emax)
                        emax = ee;
                }
                for (int64_t c = cb * 128; c < cb * 128 + 128; c++)
                    for (int64_t i = 0; i < 128; i++) {
                        uint8_t code = 0;
                        if (i < n) {
                            int ee = (int)s[(t0 + i) * (C / 128) + cb] - 127;
                            double v = ldexp(orc_e4m3_decode(q[(t0 + i) * C + c]), ee);
                            code = orc_e4m3_encode(ldexp(v, -emax));
                        }
                        qt[c * Kc + kc + i] = code;
                    }
                for (int64_t c = cb * 128; c < cb * 128 + 128; c++)
                    st[c * (Kc / 128) + kc / 128] = (uint8_t)(emax + 127);
            }
        }
    }
}

/* Weight-block transpose for Dgrad: W[rows, cols] with 128x128 block      */
/* scales becomes W^T[cols, rows] with transposed block scales; exact.     */
/* ([DSV3] §1: Dgrad multiplies by W, so the NT GEMM needs W^T K-major.)    */
void orc_block_transpose(const uint8_t *q, const uint8_t *s, int64_t rows, int64_t cols,
                         uint8_t *qt, uint8_t *st)
{
    for (int64_t r = 0; r < rows; r++)
        for (int64_t c = 0; c < cols; c++)
            qt[c * rows + r] = q[r * cols + c];
    for (int64_t rb = 0; rb < rows / 128; rb++)
        for (int64_t cb = 0; cb < cols / 128; cb++)
            st[cb * (rows / 128) + rb] = s[rb * (cols / 128) + cb];
}

/* ------------------------------------------------------------------------ */
/* Blockwise-scaled FP8 GEMM, D = A * B^T with A [M,K], B [N,K] (NT,        */
/* K-major, [DSV3] §5.7).  [DSV3] §4 and §5.3: the partial sum over each    */
/* 128-element K group is multiplied by scale_a * scale_b and added into    */
/* the accumulator.  Here every partial sum is exact (a sum of 128 products */
/* of E4M3 values fits in 43 bits of fp64) and the scaled partials are      */
/* summed in fp64.  Scale granularities:                                    */
/*   A: ROW1x128 -> sa[m, K/128], ROW1x32 -> sa[m, K/32]                    */
/*   B: BLOCK128 -> sb[ceil(N/128), K/128], ROW1x128 -> sb[n, K/128],       */
/*      ROW1x32 -> sb[n, K/32]                                              */
/* Optional level-1 factor ([MOSS] §3): b_l1[n, ceil(K/g1)] multiplies the  */
/* contribution of K range [g*g1, (g+1)*g1).                                */
/* ------------------------------------------------------------------------ */
static double g_dec[256], g_dec5[256];
static int g_dec_ready = 0;
static void dec_table(void)
{
    if (!g_dec_ready) {
        for (int c = 0; c < 256; c++) {
            g_dec[c] = orc_e4m3_decode((uint8_t)c);
            g_dec5[c] = orc_e5m2_decode((uint8_t)c);
        }
        g_dec_ready = 1;
    }
}

static int gran_size(int gran) { return gran == ORC_ROW1x32 ? 32 : 128; }

static const double *g_deca = g_dec, *g_decb = g_dec; /* element decoders of A and B */

static double gemm_one(const uint8_t *a, const uint8_t *sa, int a_gran, const uint8_t *b,
                       const uint8_t *sb, int b_gran, const float *b_l1, int64_t g1, int64_t N,
                       int64_t K, int64_t lda, int64_t ldb, int64_t m, int64_t n)
{
    int ga = gran_size(a_gran), gb = gran_size(b_gran);
    int gk = ga < gb ? ga : gb; /* the finer of the two K groups */
    int64_t ng1 = b_l1 ? (K + g1 - 1) / g1 : 1;
    double total = 0.0;
    for (int64_t g = 0; g < ng1; g++) {
        int64_t k0 = b_l1 ? g * g1 : 0, k1 = b_l1 ? (k0 + g1 < K ? k0 + g1 : K) : K;
        double acc = 0.0;
        for (int64_t kb = k0; kb < k1; kb += gk) {
            double part = 0.0; /* exact */
            for (int64_t k = kb; k < kb + gk; k++)
                part += g_deca[a[m * lda + k]] * g_decb[b[n * ldb + k]];
            int ea = (int)sa[m * (K / ga) + kb / ga] - 127;
            int eb = (b_gran == ORC_BLOCK128) ? (int)sb[(n / 128) * (K / 128) + kb / 128] - 127
                                              : (int)sb[n * (K / gb) + kb / gb] - 127;
            acc += ldexp(part, ea + eb);
        }
        total += b_l1 ? (double)b_l1[n * ng1 + g] * acc : acc;
    }
    (void)N;
    return total;
}

void orc_block_gemm(const uint8_t *a, const uint8_t *sa, int a_gran, const uint8_t *b,
                    const uint8_t *sb, int b_gran, const float *b_l1, int64_t g1, int64_t M,
                    int64_t N, int64_t K, int64_t lda, int64_t ldb, double *d)
{
    dec_table();
    for (int64_t m = 0; m < M; m++)
        for (int64_t n = 0; n < N; n++)
            d[m * N + n] = gemm_one(a, sa, a_gran, b, sb, b_gran, b_l1, g1, N, K, lda, ldb, m, n);
}

/* Same result at selected output coordinates only (for full-size checks). */
void orc_block_gemm_sampled(const uint8_t *a, const uint8_t *sa, int a_gran, const uint8_t *b,
                            const uint8_t *sb, int b_gran, const float *b_l1, int64_t g1,
                            int64_t N, int64_t K, int64_t lda, int64_t ldb, const int64_t *mi,
                            const int64_t *ni, int64_t ns, double *out)
{
    dec_table();
    for (int64_t i = 0; i < ns; i++)
        out[i] = gemm_one(a, sa, a_gran, b, sb, b_gran, b_l1, g1, N, K, lda, ldb, mi[i], ni[i]);
}

/* The same GEMM with the element format of each operand chosen (E4M3 or
 * E5M2: [MOSS] §3 gradients in E5M2 meet E4M3 weights and activations in
 * Dgrad and Wgrad).  Sampled outputs. */
void orc_block_gemm_fmt_sampled(const uint8_t *a, const uint8_t *sa, int a_gran, int a_fmt, const uint8_t *b,
                                const uint8_t *sb, int b_gran, int b_fmt, int64_t N, int64_t K,
                                const int64_t *mi, const int64_t *ni, int64_t ns, double *out)
{
    dec_table();
    g_deca = a_fmt == ORC_E5M2 ? g_dec5 : g_dec;
    g_decb = b_fmt == ORC_E5M2 ? g_dec5 : g_dec;
    for (int64_t i = 0; i < ns; i++)
        out[i] = gemm_one(a, sa, a_gran, b, sb, b_gran, NULL, 0, N, K, K, K, mi[i], ni[i]);
    g_deca = g_decb = g_dec;
}

/* K-grouped GEMM for the expert Wgrad ([DSV3] §5.6 grouped GEMMs; each    */
/* expert's weight gradient contracts over its own token segment, the 1D1D  */
/* case of §5.2): D_e = A[:, k0:k1] * B[:, k0:k1]^T, k0 = koff[e],          */
/* k1 = koff[e+1] (multiples of 128).  A [M, Kc], B [N, Kc] codes with      */
/* 1x128 scales [M, Kc/128], [N, Kc/128]; exact 128-term partials scaled    */
/* and summed in fp64.  Sampled outputs (ei, mi, ni).                      */
void orc_kgrouped_gemm_sampled(const uint8_t *a, const uint8_t *sa, const uint8_t *b, const uint8_t *sb,
                               const int32_t *koff, int64_t Kc, const int64_t *ei, const int64_t *mi,
                               const int64_t *ni, int64_t ns, double *out)
{
    dec_table();
    for (int64_t i = 0; i < ns; i++) {
        int64_t e = ei[i], m = mi[i], n = ni[i];
        double acc = 0.0;
        for (int64_t kb = koff[e]; kb < koff[e + 1]; kb += 128) {
            double part = 0.0;
            for (int64_t k = kb; k < kb + 128; k++)
                part += g_dec[a[m * Kc + k]] * g_dec[b[n * Kc + k]];
            acc += ldexp(part, (int)sa[m * (Kc / 128) + kb / 128] + (int)sb[n * (Kc / 128) + kb / 128] - 254);
        }
        out[i] = acc;
    }
}

/* Tolerance helper for a GEMM whose matrix unit sums runs of `run`
 * consecutive K products with each product cut to a fixed number of bits
 * below the run's largest: for each sample returns
 *   runmax[i] = sum over runs of max_{k in run} |scaled product k|,
 *   abssum[i] = sum over k of |scaled product k|
 * (both times |b_l1| when given).  Plain definitions, fp64. */
void orc_gemm_run_bounds_sampled(const uint8_t *a, const uint8_t *sa, int a_gran, const uint8_t *b,
                                 const uint8_t *sb, int b_gran, const float *b_l1, int64_t N,
                                 int64_t K, int64_t lda, int64_t ldb, const int64_t *mi,
                                 const int64_t *ni, int64_t ns, int run, double *runmax,
                                 double *abssum)
{
    dec_table();
    int ga = gran_size(a_gran), gb = gran_size(b_gran);
    for (int64_t i = 0; i < ns; i++) {
        int64_t m = mi[i], n = ni[i];
        double rm = 0.0, as = 0.0;
        for (int64_t k0 = 0; k0 < K; k0 += run) {
            double mx = 0.0;
            for (int64_t k = k0; k < k0 + run && k < K; k++) {
                int ea = (int)sa[m * (K / ga) + k / ga] - 127;
                int eb = (b_gran == ORC_BLOCK128) ? (int)sb[(n / 128) * (K / 128) + k / 128] - 127
                                                  : (int)sb[n * (K / gb) + k / gb] - 127;
                double pr = fabs(ldexp(g_deca[a[m * lda + k]] * g_decb[b[n * ldb + k]], ea + eb));
                as += pr;
                if (pr > mx)
                    mx = pr;
            }
            rm += mx;
        }
        double f = b_l1 ? fabs((double)b_l1[n]) : 1.0;
        runmax[i] = rm * f;
        abssum[i] = as * f;
    }
    (void)N;
}

/* orc_gemm_run_bounds_sampled with the operands' element formats chosen. */
void orc_gemm_run_bounds_fmt_sampled(const uint8_t *a, const uint8_t *sa, int a_gran, int a_fmt,
                                     const uint8_t *b, const uint8_t *sb, int b_gran, int b_fmt, int64_t N,
                                     int64_t K, const int64_t *mi, const int64_t *ni, int64_t ns, int run,
                                     double *runmax, double *abssum)
{
    dec_table();
    g_deca = a_fmt == ORC_E5M2 ? g_dec5 : g_dec;
    g_decb = b_fmt == ORC_E5M2 ? g_dec5 : g_dec;
    orc_gemm_run_bounds_sampled(a, sa, a_gran, b, sb, b_gran, NULL, N, K, K, K, mi, ni, ns, run, runmax, abssum);
    g_deca = g_decb = g_dec;
}

/* M-grouped contiguous GEMM ([DSV3] §5.6): rows [off[g], off[g+1]) of A are */
/* multiplied by expert g's B_g [N, K] with its 128x128 block scales.        */
/* Rows of D outside every segment are not written.  out: [M_rows, N] fp64. */
void orc_grouped_gemm_sampled(const uint8_t *a, const uint8_t *sa, const uint8_t *b,
                              const uint8_t *sb, const int32_t *off, int G, int64_t N, int64_t K,
                              const int64_t *mi, const int64_t *ni, int64_t ns, double *out)
{
    dec_table();
    int64_t nb = (N + 127) / 128;
    for (int64_t i = 0; i < ns; i++) {
        int64_t m = mi[i];
        int g = -1;
        for (int e = 0; e < G; e++)
            if (m >= off[e] && m < off[e + 1])
                g = e;
        if (g < 0) {
            out[i] = NAN;
            continue;
        }
        out[i] = gemm_one(a, sa, ORC_ROW1x128, b + (int64_t)g * N * K,
                          sb + (int64_t)g * nb * (K / 128), ORC_BLOCK128, NULL, 0, N, K, K, K, m,
                          ni[i]);
    }
}

/* ------------------------------------------------------------------------ */
/* Fused permute + pad ([FLOW] "Core method", fused permute+padding: expert */
/* reordering merged with 16-row alignment padding).  Rows are grouped by   */
/* expert id ascending; inside an expert, by (token, slot) ascending; each  */
/* expert segment is padded at its end to a multiple of pad_multiple rows   */
/* with code 0x00 and scale byte 105: exactly what the 1x128 rule gives an  */
/* all-zero tile (e = -22), so a padding row never raises the block-max     */
/* scale of a transposed segment.  A slot whose expert id lies outside      */
/* [0, G) is dropped (row_map = -1).                                        */
/*   xq [T, H], xs [T, H/128], topk_idx [T, topk];                          */
/*   out_q [M_cap, H], out_s [M_cap, H/128], row_map [T, topk], off [G+1].  */
/* Returns the number of rows used (off[G]), or -1 if M_cap is too small.   */
/* ------------------------------------------------------------------------ */
int64_t orc_permute_pad(const uint8_t *xq, const uint8_t *xs, const int32_t *topk_idx, int64_t T,
                        int topk, int G, int64_t H, int pad_multiple, uint8_t *out_q,
                        uint8_t *out_s, int32_t *row_map, int32_t *off, int64_t M_cap)
{
    int64_t *cnt = calloc((size_t)G, sizeof(int64_t));
    int64_t *cur = calloc((size_t)G, sizeof(int64_t));
    for (int64_t i = 0; i < T * topk; i++)
        if (topk_idx[i] >= 0 && topk_idx[i] < G)
            cnt[topk_idx[i]]++;
    off[0] = 0;
    for (int e = 0; e < G; e++)
        off[e + 1] = off[e] + (int32_t)(((cnt[e] + pad_multiple - 1) / pad_multiple) * pad_multiple);
    if (off[G] > M_cap) {
        free(cnt);
        free(cur);
        return -1;
    }
    for (int e = 0; e < G; e++)
        cur[e] = off[e];
    int64_t H128 = H / 128;
    for (int64_t t = 0; t < T; t++)
        for (int k = 0; k < topk; k++) {
            int e = topk_idx[t * topk + k];
            if (e < 0 || e >= G) {
                row_map[t * topk + k] = -1;
                continue;
            }
            int64_t r = cur[e]++;
            memcpy(out_q + r * H, xq + t * H, (size_t)H);
            memcpy(out_s + r * H128, xs + t * H128, (size_t)H128);
            row_map[t * topk + k] = (int32_t)r;
        }
    for (int e = 0; e < G; e++)
        for (int64_t r = off[e] + cnt[e]; r < off[e + 1]; r++) {
            memset(out_q + r * H, 0x00, (size_t)H);
            memset(out_s + r * H128, 105, (size_t)H128);
        }
    free(cnt);
    free(cur);
    return off[G];
}

/* ------------------------------------------------------------------------ */
/* Unpermute + unpad ([FLOW] "Core method", fused unpermute+unpadding):     */
/* out[t][h] = bf16_rne( fold over k = 0..topk-1 of                         */
/*             acc = fmaf(w[t][k], y[row_map[t][k]][h], acc) ), acc0 = 0,   */
/* w = probs or 1, slots with row_map < 0 skipped; padding rows are never  */
/* referenced.  y, out bf16 bits; the fold is fp32 with fused multiply-add. */
/* ------------------------------------------------------------------------ */
void orc_unpermute_unpad(const uint16_t *y, const int32_t *row_map, const float *probs, int64_t T,
                         int topk, int64_t H, uint16_t *out)
{
    for (int64_t t = 0; t < T; t++)
        for (int64_t h = 0; h < H; h++) {
            float acc = 0.0f;
            for (int k = 0; k < topk; k++) {
                int32_t r = row_map[t * topk + k];
                if (r < 0)
                    continue;
                float w = probs ? probs[t * topk + k] : 1.0f;
                acc = fmaf(w, (float)bf16_value(y[(int64_t)r * H + h]), acc);
            }
            out[t * H + h] = bf16_round(acc);
        }
}

/* ------------------------------------------------------------------------ */
/* Backward of unpermute_unpad, for the MoE expert backward ([FLOW] "Core   */
/* method": the fused unpermute; its gradient brings the output gradient   */
/* back into the permuted, padded expert layout).  out[t] = sum_k w[t,k] *  */
/* y[row_map[t,k]] gives dy[row_map[t,k]] = RN_bf16(fp32(w[t,k] * dout[t]))  */
/* (w = 1 without probs); rows no slot maps to (the padding) are zero.      */
/*   dout bf16 [T, H]; row_map, probs [T, topk]; dy bf16 [M_cap, H].         */
/* ------------------------------------------------------------------------ */
void orc_unpermute_backward(const uint16_t *dout, const int32_t *row_map, const float *probs,
                            int64_t T, int topk, int64_t H, int64_t M_cap, uint16_t *dy)
{
    memset(dy, 0, (size_t)(M_cap * H) * sizeof(uint16_t));
    for (int64_t t = 0; t < T; t++)
        for (int k = 0; k < topk; k++) {
            int32_t r = row_map[t * topk + k];
            if (r < 0 || r >= M_cap)
                continue;
            float w = probs ? probs[t * topk + k] : 1.0f;
            for (int64_t h = 0; h < H; h++)
                dy[(int64_t)r * H + h] = bf16_round(w * (float)bf16_value(dout[t * H + h]));
        }
}

/* ------------------------------------------------------------------------ */
/* Exponential used by SwiGLU.  The pages fix no exp; this one is the       */
/* library's own definition so that both implementations round alike:      */
/* Cody-Waite argument reduction x = n ln2 + r (Cody & Waite, "Software     */
/* Manual for the Elementary Functions", 1980) with a two-part ln2, then    */
/* the degree-7 Taylor polynomial of e^r in Horner form, then scaling by    */
/* 2^n in two exact power-of-two steps.  Every step is one fp32 rounding.   */
/* ------------------------------------------------------------------------ */
static float pow2f_exact(int n) /* 2^n for -126 <= n <= 127 */
{
    uint32_t u = (uint32_t)(n + 127) << 23;
    float f;
    memcpy(&f, &u, 4);
    return f;
}

float orc_expf(float x)
{
    if (x > 0x1.62e43p+6f) /* 88.72283935546875 */
        return INFINITY;
    if (x < -0x1.9fe36ap+6f) /* -103.97208404541015625 */
        return 0.0f;
    const float log2e = 0x1.715476p+0f;  /* fp32 nearest to 1/ln2 */
    const float ln2_hi = 0x1.62e4p-1f;   /* ln2 cut to 16 significant bits */
    const float ln2_lo = 0x1.7f7d1cp-20f; /* fp32 nearest to ln2 - ln2_hi */
    float n = rintf(x * log2e);
    float r = fmaf(-n, ln2_hi, x);
    r = fmaf(-n, ln2_lo, r);
    /* Taylor coefficients of e^r: 1/j!, j = 7..0, each the fp32 nearest value */
    float p = 0x1.a01a02p-13f;          /* 1/5040 */
    p = fmaf(p, r, 0x1.6c16c2p-10f);    /* 1/720 */
    p = fmaf(p, r, 0x1.111112p-7f);     /* 1/120 */
    p = fmaf(p, r, 0x1.555556p-5f);     /* 1/24 */
    p = fmaf(p, r, 0x1.555556p-3f);     /* 1/6 */
    p = fmaf(p, r, 0x1p-1f);            /* 1/2 */
    p = fmaf(p, r, 1.0f);
    p = fmaf(p, r, 1.0f);
    int ni = (int)n;
    int n1 = ni / 2, n2 = ni - n1;
    return (p * pow2f_exact(n1)) * pow2f_exact(n2);
}

void orc_expf_bulk(const float *x, int64_t n, float *y)
{
    for (int64_t i = 0; i < n; i++)
        y[i] = orc_expf(x[i]);
}

/* ------------------------------------------------------------------------ */
/* Fused SwiGLU + 1x128 quantization ([FLOW] "Core method": the activation  */
/* emits FP8 directly at the activation boundary; [FLOW] assumption 2: the  */
/* first expert linear's output stays BF16 up to the activation).           */
/*   h: bf16 [M, 2F] (ld ldh), gate = h[:, :F], up = h[:, F:];              */
/*   a = (g / (1 + exp(-g))) * u, each operation one fp32 rounding;          */
/*   then 1x128 quantization of a.  Rows r >= off[G] (when off given) are   */
/*   skipped.                                                               */
/* ------------------------------------------------------------------------ */
void orc_swiglu_quant(const uint16_t *h, int64_t M, int64_t F, int64_t ldh, const int32_t *off,
                      int G, uint8_t *q, uint8_t *s)
{
    int64_t rows = off ? off[G] : M;
    float *a = malloc((size_t)F * sizeof(float));
    for (int64_t r = 0; r < rows; r++) {
        for (int64_t j = 0; j < F; j++) {
            float g = (float)bf16_value(h[r * ldh + j]);
            float u = (float)bf16_value(h[r * ldh + F + j]);
            float e = orc_expf(-g);
            float silu = g / (1.0f + e);
            a[j] = silu * u;
        }
        orc_quant_rowwise(a, ORC_F32, 1, F, F, 128, -22, q + r * F, F, s + r * (F / 128), F / 128);
    }
    free(a);
}

/* ------------------------------------------------------------------------ */
/* Fused SwiGLU backward + 1x128 quantization.  [DSV3] §3 (low-precision    */
/* activations): the MoE SwiGLU input is cached in FP8 and the activation   */
/* is recomputed in the backward pass; [FLOW] "Core method": the activation */
/* boundary emits FP8.  With g, u the dequantized cached input (exact in    */
/* fp32) and da the gradient of a = silu(g) * u, in this order, each        */
/* operation one fp32 rounding:                                             */
/*   e = exp(-g), d = 1 + e, sg = 1 / d, silu = g / d, du = da * silu,      */
/*   dsilu = sg * (1 + g * (1 - sg)), dg = (da * u) * dsilu                 */
/* (dsilu is the derivative of g * sigmoid(g)); then 1x128 quantization of  */
/* the row [dg | du].                                                       */
/*   hq: [M, 2F] codes with hs [M, 2F/128] (1x128 scales); da: bf16 [M, F]; */
/*   dq: [M, 2F], ds: [M, 2F/128].  Rows r >= off[G] (when off given) are   */
/*   skipped.                                                               */
/* ------------------------------------------------------------------------ */
void orc_dswiglu_quant(const uint8_t *hq, const uint8_t *hs, const uint16_t *da, int64_t M,
                       int64_t F, const int32_t *off, int G, uint8_t *dq, uint8_t *ds)
{
    int64_t rows = off ? off[G] : M;
    float *dh = malloc((size_t)(2 * F) * sizeof(float));
    for (int64_t r = 0; r < rows; r++) {
        for (int64_t j = 0; j < F; j++) {
            float g = (float)ldexp(orc_e4m3_decode(hq[r * 2 * F + j]), (int)hs[r * (2 * F / 128) + j / 128] - 127);
            float u = (float)ldexp(orc_e4m3_decode(hq[r * 2 * F + F + j]),
                                   (int)hs[r * (2 * F / 128) + (F + j) / 128] - 127);
            float a = (float)bf16_value(da[r * F + j]);
            float e = orc_expf(-g);
            float d = 1.0f + e;
            float sg = 1.0f / d;
            float silu = g / d;
            float du = a * silu;
            float dsilu = sg * (1.0f + g * (1.0f - sg));
            float dg = (a * u) * dsilu;
            dh[j] = dg;
            dh[F + j] = du;
        }
        orc_quant_rowwise(dh, ORC_F32, 1, 2 * F, 2 * F, 128, -22, dq + r * 2 * F, 2 * F,
                          ds + r * (2 * F / 128), 2 * F / 128);
    }
    free(dh);
}

/* ------------------------------------------------------------------------ */
/* The SwiGLU forward and backward values in fp32, element by element,      */
/* before any quantization: the same operations, in the same order, as     */
/* orc_swiglu_quant and orc_dswiglu_quant above ([FLOW] "Core method";      */
/* [DSV3] §3), for inputs given directly as fp32 (g, u; the gradient a).    */
/* ------------------------------------------------------------------------ */
void orc_swiglu_f32(const float *g, const float *u, int64_t n, float *a)
{
    for (int64_t i = 0; i < n; i++) {
        float e = orc_expf(-g[i]);
        float silu = g[i] / (1.0f + e);
        a[i] = silu * u[i];
    }
}

void orc_dswiglu_f32(const float *g, const float *u, const float *da, int64_t n, float *du, float *dg)
{
    for (int64_t i = 0; i < n; i++) {
        float e = orc_expf(-g[i]);
        float d = 1.0f + e;
        float sg = 1.0f / d;
        float silu = g[i] / d;
        du[i] = da[i] * silu;
        float dsilu = sg * (1.0f + g[i] * (1.0f - sg));
        dg[i] = (da[i] * u[i]) * dsilu;
    }
}

/* ------------------------------------------------------------------------ */
/* MOSS two-level microscaling ([MOSS] §3 "two-level microscaling" and Fig. */
/* 2): level 1 is an FP32 factor alpha1 = max|X| / 448 over a group of about */
/* 10K elements; level 2 is an E8M0 power-of-two scale per 32 elements of   */
/* X / alpha1; elements are E4M3.  Group layout: contiguous g1 elements     */
/* along each row, the last group partial.  alpha1 = fp32(amax / 448), or 1 */
/* for an all-zero group; y = fp32(x / alpha1); level-2 exponent by the     */
/* scale rule above with floor -127.                                        */
/*   x: bf16 [R, C]; q [R, C]; s2 [R, C/32]; s1 [R, ceil(C/g1)].            */
/* ------------------------------------------------------------------------ */
/* rule: the level-2 exponent rule (ORC_SCALE_CEIL as everywhere, or the
 * MX standard's ORC_SCALE_OCP_FLOOR that [MOSS] §3 points to for k2 = 32);
 * codes clip at 448 (the encoder's saturation). */
void orc_mx2_quant_rule(const uint16_t *x, int64_t R, int64_t C, int64_t g1, int rule, uint8_t *q, uint8_t *s2,
                        float *s1)
{
    int64_t ng = (C + g1 - 1) / g1;
    float *y = malloc((size_t)g1 * sizeof(float));
    for (int64_t r = 0; r < R; r++)
        for (int64_t g = 0; g < ng; g++) {
            int64_t c0 = g * g1, c1 = c0 + g1 < C ? c0 + g1 : C;
            float amax = 0.0f;
            for (int64_t c = c0; c < c1; c++) {
                float v = fabsf((float)bf16_value(x[r * C + c]));
                if (v > amax)
                    amax = v;
            }
            float alpha = amax > 0.0f ? amax / 448.0f : 1.0f;
            s1[r * ng + g] = alpha;
            for (int64_t c = c0; c < c1; c++)
                y[c - c0] = (float)bf16_value(x[r * C + c]) / alpha;
            for (int64_t b = c0; b < c1; b += 32) {
                double amax2 = 0.0;
                for (int64_t c = b; c < b + 32; c++)
                    if (fabs((double)y[c - c0]) > amax2)
                        amax2 = fabs((double)y[c - c0]);
                int e = orc_scale_exp_fmt(amax2, ORC_E4M3, rule, -127);
                for (int64_t c = b; c < b + 32; c++)
                    q[r * C + c] = orc_e4m3_encode(ldexp((double)y[c - c0], -e));
                s2[r * (C / 32) + b / 32] = (uint8_t)(e + 127);
            }
        }
    free(y);
}

void orc_mx2_quant(const uint16_t *x, int64_t R, int64_t C, int64_t g1, uint8_t *q, uint8_t *s2, float *s1)
{
    orc_mx2_quant_rule(x, R, C, g1, ORC_SCALE_CEIL, q, s2, s1);
}

/* x_hat = fp32( fp32(decode(q) * 2^e2) * alpha1 ); the first product is    */
/* exact (an E4M3 value times 2^e2, e2 >= -127, stays representable).       */
void orc_mx2_dequant(const uint8_t *q, const uint8_t *s2, const float *s1, int64_t R, int64_t C,
                     int64_t g1, float *out)
{
    int64_t ng = (C + g1 - 1) / g1;
    for (int64_t r = 0; r < R; r++)
        for (int64_t c = 0; c < C; c++) {
            float v = (float)ldexp(orc_e4m3_decode(q[r * C + c]), (int)s2[r * (C / 32) + c / 32] - 127);
            out[r * C + c] = v * s1[r * ng + c / g1];
        }
}

/* Signal-to-noise ratio in dB, 10 log10( sum x^2 / sum (x - x_hat)^2 ), in */
/* fp64.  ([MOSS] §3 prints the ratio upside down; the quantity compared    */
/* there is signal over noise.)                                             */
double orc_snr_db(const float *x, const float *xhat, int64_t n)
{
    double sig = 0.0, noise = 0.0;
    for (int64_t i = 0; i < n; i++) {
        double d = (double)x[i] - (double)xhat[i];
        sig += (double)x[i] * (double)x[i];
        noise += d * d;
    }
    return 10.0 * log10(sig / noise);
}

/* bf16 helpers exposed for tests */
void orc_bf16_to_f32(const uint16_t *h, int64_t n, float *out)
{
    for (int64_t i = 0; i < n; i++)
        out[i] = (float)bf16_value(h[i]);
}
