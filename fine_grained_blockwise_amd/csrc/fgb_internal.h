// fgb_internal.h -- shared host plumbing and gfx950 device helpers of libfgb.
//
// Numeric conventions (llm-infra-atlas, "01 · DeepSeek FP8 and DeepGEMM: Hopper
// software recipe", §3 and §8; "Low precision" chapter index, §2 format table):
//   E4M3 codes are OCP E4M3FN (bias 7, max 448, no Inf); a scale byte b means
//   2^(b-127); the exponent for an amax is the smallest e with amax <= 448*2^e,
//   floored at emin (-22 for 128-element groups, -127 for 32-element groups).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/fgb.h"

namespace fgb {

int set_error(int code, const char *fmt, ...) __attribute__((format(printf, 2, 3)));
void clear_error();

inline bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// ---------------------------------------------------------------------------
// device helpers
// ---------------------------------------------------------------------------

// 2^e as an fp32 for -126 <= e <= 127, built from its bits (exact).
__device__ __forceinline__ float pow2f(int e) { return __uint_as_float((uint32_t)(e + 127) << 23); }

// Scale exponent from the fp32 bit pattern of a non-negative amax.
// 448 = 1.75 * 2^8, so a normal amax = (1 + f/2^23) * 2^Ea needs
// e = Ea - 8 when f <= 0x600000 (1 + f/2^23 <= 1.75) and Ea - 7 above.
// Zero and subnormal amax lie below every floor used here.
__device__ __forceinline__ int scale_exp_from_bits(uint32_t amax_bits, int emin)
{
    int Ea = (int)(amax_bits >> 23) - 127;
    int e = Ea - 8 + ((amax_bits & 0x7FFFFFu) > 0x600000u ? 1 : 0);
    e = amax_bits < 0x00800000u ? emin : e;
    return e < emin ? emin : e;
}

// Pack four fp32 values into four E4M3 bytes (byte i <- value i) with the
// hardware conversion (round to nearest even, OCP E4M3FN on gfx950).
// Callers keep |v| <= 448, so saturation never enters.
__device__ __forceinline__ uint32_t cvt4_e4m3(float a, float b, float c, float d)
{
    int w = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);
    w = __builtin_amdgcn_cvt_pk_fp8_f32(c, d, w, true);
    return (uint32_t)w;
}

// Element formats and scale rules of the format-variant entry points.
enum { FMT_E4M3 = 0, FMT_E5M2 = 1 };
enum { RULE_CEIL = 0, RULE_OCP_FLOOR = 1 };

// Scale exponent for an element format and rule.  CEIL: the smallest e with
// amax <= max * 2^e (max = 1.75 * 2^EMAX, EMAX = 8 for E4M3, 15 for E5M2).
// OCP_FLOOR: the MX standard's floor(log2 amax) - EMAX.  Floored at emin.
template <int FMT, int RULE>
__device__ __forceinline__ int scale_exp_fmt(uint32_t amax_bits, int emin)
{
    constexpr int EMAX = FMT == FMT_E5M2 ? 15 : 8;
    int Ea = (int)(amax_bits >> 23) - 127;
    int e = Ea - EMAX + ((RULE == RULE_CEIL && (amax_bits & 0x7FFFFFu) > 0x600000u) ? 1 : 0);
    e = amax_bits < 0x00800000u ? emin : e;
    return e < emin ? emin : e;
}

// Four fp32 values -> four E5M2 bytes (OCP E5M2, round to nearest even).
// Callers keep |v| <= 57344.
__device__ __forceinline__ uint32_t cvt4_e5m2(float a, float b, float c, float d)
{
    int w = __builtin_amdgcn_cvt_pk_bf8_f32(a, b, 0, false);
    w = __builtin_amdgcn_cvt_pk_bf8_f32(c, d, w, true);
    return (uint32_t)w;
}

// Four fp32 values -> four codes of format FMT; CLIP first limits each value
// to the format's largest finite magnitude (the floor rule can scale a
// group's largest elements past it).
template <int FMT, bool CLIP>
__device__ __forceinline__ uint32_t cvt4_fmt(float a, float b, float c, float d)
{
    if constexpr (CLIP) {
        constexpr float M = FMT == FMT_E5M2 ? 57344.0f : 448.0f;
        a = __builtin_fminf(__builtin_fmaxf(a, -M), M);
        b = __builtin_fminf(__builtin_fmaxf(b, -M), M);
        c = __builtin_fminf(__builtin_fmaxf(c, -M), M);
        d = __builtin_fminf(__builtin_fmaxf(d, -M), M);
    }
    if constexpr (FMT == FMT_E5M2)
        return cvt4_e5m2(a, b, c, d);
    else
        return cvt4_e4m3(a, b, c, d);
}

// Decode bytes (0,1) or (2,3) of a word of E4M3 codes to fp32 (exact).
__device__ __forceinline__ float2 dec2_lo(uint32_t w)
{
    auto v = __builtin_amdgcn_cvt_pk_f32_fp8((int)w, false);
    return make_float2(v[0], v[1]);
}
__device__ __forceinline__ float2 dec2_hi(uint32_t w)
{
    auto v = __builtin_amdgcn_cvt_pk_f32_fp8((int)w, true);
    return make_float2(v[0], v[1]);
}

// The same for E5M2 codes.
__device__ __forceinline__ float2 dec2_lo_e5m2(uint32_t w)
{
    auto v = __builtin_amdgcn_cvt_pk_f32_bf8((int)w, false);
    return make_float2(v[0], v[1]);
}
__device__ __forceinline__ float2 dec2_hi_e5m2(uint32_t w)
{
    auto v = __builtin_amdgcn_cvt_pk_f32_bf8((int)w, true);
    return make_float2(v[0], v[1]);
}

// bf16 halves of a 32-bit word as fp32 (exact).
__device__ __forceinline__ float bf16lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// fp32 -> bf16 bits, round to nearest even (finite values).
__device__ __forceinline__ uint32_t bf16_rne(float f)
{
    uint32_t u = __float_as_uint(f);
    return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

// Two fp32 values -> two bf16 (round to nearest even, v_cvt_pk_bf16_f32), lo in the low half.
typedef __bf16 fgb_bf16x2 __attribute__((ext_vector_type(2)));
typedef float fgb_f32x2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi)
{
    return __builtin_bit_cast(uint32_t, __builtin_convertvector((fgb_f32x2){lo, hi}, fgb_bf16x2));
}

// DPP lane moves (row = 16 lanes).
#define FGB_DPP_QUAD_XOR1 0xB1 // quad_perm [1,0,3,2]
#define FGB_DPP_QUAD_XOR2 0x4E // quad_perm [2,3,0,1]
#define FGB_DPP_HALF_MIRROR 0x141
#define FGB_DPP_ROW_ROR8 0x128

template <int CTRL>
__device__ __forceinline__ uint32_t dpp(uint32_t v)
{
    return (uint32_t)__builtin_amdgcn_mov_dpp((int)v, CTRL, 0xF, 0xF, true);
}

// Unsigned max over aligned groups of L consecutive lanes (L in 4,8,16,32,64);
// every lane of the group receives the result.
template <int L>
__device__ __forceinline__ uint32_t group_max_u32(uint32_t v)
{
    v = max(v, dpp<FGB_DPP_QUAD_XOR1>(v));
    v = max(v, dpp<FGB_DPP_QUAD_XOR2>(v));
    if constexpr (L >= 8)
        v = max(v, dpp<FGB_DPP_HALF_MIRROR>(v));
    if constexpr (L >= 16)
        v = max(v, dpp<FGB_DPP_ROW_ROR8>(v));
    if constexpr (L >= 32)
        v = max(v, (uint32_t)__shfl_xor((int)v, 16));
    if constexpr (L >= 64)
        v = max(v, (uint32_t)__shfl_xor((int)v, 32));
    return v;
}

__device__ __forceinline__ int lane_id() { return (int)(threadIdx.x & 63); }

// Streaming loads and stores (nontemporal: the data is touched once, so it
// should not displace cached lines) of 16, 8 and 4 bytes.
typedef uint32_t fgb_u4v __attribute__((ext_vector_type(4)));
typedef uint32_t fgb_u2v __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint4 ld_stream16(const void *p)
{
    const fgb_u4v v = __builtin_nontemporal_load(reinterpret_cast<const fgb_u4v *>(p));
    return make_uint4(v.x, v.y, v.z, v.w);
}
__device__ __forceinline__ void st_stream16(void *p, uint4 v)
{
    __builtin_nontemporal_store((fgb_u4v){v.x, v.y, v.z, v.w}, reinterpret_cast<fgb_u4v *>(p));
}
__device__ __forceinline__ void st_stream8(void *p, uint2 v)
{
    __builtin_nontemporal_store((fgb_u2v){v.x, v.y}, reinterpret_cast<fgb_u2v *>(p));
}
__device__ __forceinline__ void st_stream4(void *p, uint32_t v)
{
    __builtin_nontemporal_store(v, reinterpret_cast<uint32_t *>(p));
}

// Ordinary (write-back) 16-byte stores, for kernels whose traffic is
// mostly writes: on the MI355X a stream of ordinary 16-byte stores sustained
// ~8% more than nontemporal ones (5.85 against 5.40 TB/s writing 1 GB).
__device__ __forceinline__ void st_plain16(void *p, uint4 v) { *reinterpret_cast<uint4 *>(p) = v; }


} // namespace fgb

#define FGB_REQUIRE(cond, code, ...)                                                              \
    do {                                                                                          \
        if (!(cond))                                                                              \
            return fgb::set_error((code), __VA_ARGS__);                                          \
    } while (0)

#define FGB_LAUNCHED(name)                                                                        \
    do {                                                                                          \
        hipError_t e_ = hipGetLastError();                                                        \
        if (e_ != hipSuccess)                                                                     \
            return fgb::set_error(FGB_EHIP, "%s: launch failed: %s", (name),                      \
                                  hipGetErrorString(e_));                                         \
    } while (0)
