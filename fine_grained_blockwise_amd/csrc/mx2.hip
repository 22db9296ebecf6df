// mx2.hip -- MOSS two-level microscaling: quantize and dequantize.
//
// xllm-io paper review, "MOSS: Efficient and Accurate FP8 LLM Training with
// Microscaling and Automatic Scaling", §3 two-level microscaling and Fig. 2:
// level 1 is an FP32 factor alpha1 = max|X| / 448 over a group of about 10K
// elements; level 2 is an E8M0 (power-of-two) scale per 32 elements of
// X / alpha1; the elements are E4M3.  Groups are g1 contiguous elements of a
// row (the last one partial); alpha1 = fp32(amax / 448), 1 for an all-zero
// group; y = fp32(x / alpha1) with correctly rounded division; level-2
// exponent = smallest e >= -127 with amax32(y) <= 448 * 2^e.
//
// One workgroup per (row, level-1 group): the group (<= 16384 bf16) is held
// in registers (16-byte loads), amax reduced across the workgroup, then
// divided, scaled per 32 elements (4 lanes) and converted.  HBM-bound.
#include "fgb_internal.h"

namespace fgb {

constexpr int MX_MAXCH = 8; // 16-byte chunks per thread: g1 <= 256 * 8 * 8

// RULE: the level-2 exponent rule -- RULE_CEIL (above) or RULE_OCP_FLOOR, the
// MX standard's floor(log2 amax32) - 8 with the elements clipped at 448.
template <int RULE = RULE_CEIL>
__global__ __launch_bounds__(256) void mx2_quant_kernel(const uint16_t *__restrict__ x, int64_t R,
                                                        int64_t C, int64_t g1, int64_t ng,
                                                        uint8_t *__restrict__ q,
                                                        uint8_t *__restrict__ s2,
                                                        float *__restrict__ s1)
{
    __shared__ uint32_t red[4];
    const int64_t r = blockIdx.x / ng, g = blockIdx.x % ng;
    const int64_t c0 = g * g1;
    const int64_t len = min(g1, C - c0);
    const int64_t nch = len / 8;
    const int t = threadIdx.x;
    const uint16_t *xr = x + r * C + c0;
    uint4 v[MX_MAXCH];
    uint32_t m = 0;
#pragma unroll
    for (int i = 0; i < MX_MAXCH; i++) {
        int64_t c = (int64_t)i * 256 + t;
        v[i] = c < nch ? ld_stream16(xr + c * 8) : make_uint4(0, 0, 0, 0);
        uint32_t w4[4] = {v[i].x, v[i].y, v[i].z, v[i].w};
#pragma unroll
        for (int k = 0; k < 4; k++)
            m = max(m, max((w4[k] << 16) & 0x7FFFFFFFu, w4[k] & 0x7FFF0000u));
    }
    m = group_max_u32<64>(m);
    if (lane_id() == 0)
        red[t >> 6] = m;
    __syncthreads();
    m = max(max(red[0], red[1]), max(red[2], red[3]));
    const float amax = __uint_as_float(m);
    const float alpha = m != 0 ? amax / 448.0f : 1.0f;
    if (t == 0)
        s1[r * ng + g] = alpha;
    // y = RN32(x / alpha) as RN32(RN64(x * RN64(1 / alpha))): the product is
    // within 2^-51.9 relative of x / alpha, while a quotient of a bf16 by an
    // fp32 lies more than 2^-49 relative from every fp32 rounding boundary
    // (the boundary times alpha has at most 49 significant bits and cannot
    // equal x), so both roundings land where the one correct rounding does.
    const double rinv = 1.0 / (double)alpha;
#pragma unroll
    for (int i = 0; i < MX_MAXCH; i++) {
        int64_t c = (int64_t)i * 256 + t;
        if ((int64_t)i * 256 >= nch)
            break; // uniform across the workgroup
        uint32_t w4[4] = {v[i].x, v[i].y, v[i].z, v[i].w};
        float y[8];
        uint32_t m2 = 0;
#pragma unroll
        for (int k = 0; k < 4; k++) {
            y[2 * k] = (float)((double)bf16lo(w4[k]) * rinv);
            y[2 * k + 1] = (float)((double)bf16hi(w4[k]) * rinv);
            m2 = max(m2, __float_as_uint(y[2 * k]) & 0x7FFFFFFFu);
            m2 = max(m2, __float_as_uint(y[2 * k + 1]) & 0x7FFFFFFFu);
        }
        m2 = group_max_u32<4>(m2); // 4 lanes = 32 elements
        int e = scale_exp_fmt<FMT_E4M3, RULE>(m2, -127);
        float sc = pow2f(-e);
        if (c < nch) {
            constexpr bool CLIP = RULE == RULE_OCP_FLOOR;
            uint2 o;
            o.x = cvt4_fmt<FMT_E4M3, CLIP>(y[0] * sc, y[1] * sc, y[2] * sc, y[3] * sc);
            o.y = cvt4_fmt<FMT_E4M3, CLIP>(y[4] * sc, y[5] * sc, y[6] * sc, y[7] * sc);
            st_stream8(q + r * C + c0 + c * 8, o);
            if ((t & 3) == 0)
                s2[r * (C / 32) + (c0 + c * 8) / 32] = (uint8_t)(e + 127);
        }
    }
}

// Workgroup (x, y) decodes row y (and every gridDim.y-th after it), codes
// [2048 x, 2048 x + 2048): each thread takes 2 runs of 4 codes, 256 runs
// apart, so every load and store instruction covers one contiguous span
// (2 runs per thread measured 7-8% faster than 4, and 1 run 4% faster).
__global__ __launch_bounds__(256) void mx2_dequant_kernel(const uint8_t *__restrict__ q,
                                                          const uint8_t *__restrict__ s2,
                                                          const float *__restrict__ s1, int64_t R,
                                                          int64_t C, int64_t g1, int64_t ng,
                                                          float *__restrict__ out)
{
    const int64_t C4 = C / 4;
    for (int64_t r = blockIdx.y; r < R; r += gridDim.y) {
        const uint8_t *qr = q + r * C;
        float *orow = out + r * C;
        uint32_t w[2];
        float al[2];
        int e[2];
#pragma unroll
        for (int u = 0; u < 2; u++) {
            const int64_t j = (int64_t)blockIdx.x * 512 + u * 256 + threadIdx.x; // run index
            if (j < C4) {
                w[u] = __builtin_nontemporal_load(reinterpret_cast<const uint32_t *>(qr + j * 4));
                e[u] = (int)s2[r * (C / 32) + j / 8] - 127;
                al[u] = s1[r * ng + (j * 4) / g1];
            }
        }
#pragma unroll
        for (int u = 0; u < 2; u++) {
            const int64_t j = (int64_t)blockIdx.x * 512 + u * 256 + threadIdx.x;
            if (j < C4) {
                const float2 a = dec2_lo(w[u]), b = dec2_hi(w[u]);
                st_stream16(orow + j * 4,
                            make_uint4(__float_as_uint(ldexpf(a.x, e[u]) * al[u]), __float_as_uint(ldexpf(a.y, e[u]) * al[u]),
                                       __float_as_uint(ldexpf(b.x, e[u]) * al[u]), __float_as_uint(ldexpf(b.y, e[u]) * al[u])));
            }
        }
    }
}

} // namespace fgb

using namespace fgb;

extern "C" int mx2_quant_rule(const void *x, int64_t R, int64_t C, int64_t g1, int rule, uint8_t *q, uint8_t *s2,
                              float *s1, void *stream)
{
    clear_error();
    FGB_REQUIRE(rule == FGB_SCALE_CEIL || rule == FGB_SCALE_OCP_FLOOR, FGB_EUNSUPPORTED,
                "mx2_quant: rule must be FGB_SCALE_CEIL or FGB_SCALE_OCP_FLOOR");
    FGB_REQUIRE(x && q && s2 && s1, FGB_EINVAL, "mx2_quant: null pointer");
    FGB_REQUIRE(R >= 0 && C > 0 && C % 32 == 0, FGB_EINVAL, "mx2_quant: C must be a positive multiple of 32");
    FGB_REQUIRE(g1 > 0 && g1 % 32 == 0 && g1 <= 256 * 8 * MX_MAXCH, FGB_EUNSUPPORTED,
                "mx2_quant: g1 must be a multiple of 32 and at most %d", 256 * 8 * MX_MAXCH);
    FGB_REQUIRE(aligned16(x) && aligned16(q), FGB_EINVAL, "mx2_quant: x and q must be 16-byte aligned");
    if (R == 0)
        return FGB_OK;
    int64_t ng = (C + g1 - 1) / g1;
    FGB_REQUIRE(R * ng < (1ll << 31), FGB_EINVAL, "mx2_quant: too many groups");
    if (rule == FGB_SCALE_OCP_FLOOR)
        mx2_quant_kernel<RULE_OCP_FLOOR><<<(unsigned)(R * ng), 256, 0, (hipStream_t)stream>>>((const uint16_t *)x, R, C, g1,
                                                                                              ng, q, s2, s1);
    else
        mx2_quant_kernel<RULE_CEIL><<<(unsigned)(R * ng), 256, 0, (hipStream_t)stream>>>((const uint16_t *)x, R, C, g1, ng,
                                                                                         q, s2, s1);
    FGB_LAUNCHED("mx2_quant");
    return FGB_OK;
}

extern "C" int mx2_quant(const void *x, int64_t R, int64_t C, int64_t g1, uint8_t *q, uint8_t *s2, float *s1,
                         void *stream)
{
    return mx2_quant_rule(x, R, C, g1, FGB_SCALE_CEIL, q, s2, s1, stream);
}

extern "C" int mx2_dequant(const uint8_t *q, const uint8_t *s2, const float *s1, int64_t R,
                           int64_t C, int64_t g1, float *out, void *stream)
{
    clear_error();
    FGB_REQUIRE(q && s2 && s1 && out, FGB_EINVAL, "mx2_dequant: null pointer");
    FGB_REQUIRE(R >= 0 && C > 0 && C % 32 == 0 && g1 > 0 && g1 % 32 == 0, FGB_EINVAL,
                "mx2_dequant: C and g1 must be positive multiples of 32");
    FGB_REQUIRE(aligned16(q) && aligned16(out), FGB_EINVAL, "mx2_dequant: q and out must be 16-byte aligned");
    if (R == 0)
        return FGB_OK;
    int64_t ng = (C + g1 - 1) / g1;
    const dim3 grid((unsigned)((C / 4 + 511) / 512), (unsigned)(R < 65535 ? R : 65535));
    mx2_dequant_kernel<<<grid, 256, 0, (hipStream_t)stream>>>(q, s2, s1, R, C, g1, ng, out);
    FGB_LAUNCHED("mx2_dequant");
    return FGB_OK;
}
