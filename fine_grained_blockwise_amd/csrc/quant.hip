// quant.hip -- 1xg row-wise and 128x128 block-wise E4M3 quantization with
// power-of-two scales, dequantization, and the raw device encoder.
//
// llm-infra-atlas, "01 · DeepSeek FP8 and DeepGEMM: Hopper software recipe":
//   §2 online quantization (amax of each 1x128 activation tile / 128x128 weight
//   block computed when the tensor is produced), §3 tile shapes and scale
//   tensors [T, C/128] and [Cout/128, Cin/128], §8 power-of-two (UE8M0) scales.
// xllm-io review, "MOSS: ...", §3: 32-element E8M0 groups (group = 32 here).
//
// Both quantizers are HBM-bound: each input byte is read once, each code and
// scale byte written once, with 16-byte loads per lane.
#include "fgb_internal.h"

namespace fgb {

typedef unsigned short us2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ uint32_t pkmax_u16(uint32_t a, uint32_t b)
{
    us2 x = __builtin_bit_cast(us2, a), y = __builtin_bit_cast(us2, b);
    return __builtin_bit_cast(uint32_t, __builtin_elementwise_max(x, y));
}

// amax of a 16-byte chunk as fp32 bits (sign dropped).
template <bool BF16>
__device__ __forceinline__ uint32_t chunk_amax_bits(uint4 v)
{
    if constexpr (BF16) {
        uint32_t m = pkmax_u16(pkmax_u16(v.x & 0x7FFF7FFFu, v.y & 0x7FFF7FFFu),
                               pkmax_u16(v.z & 0x7FFF7FFFu, v.w & 0x7FFF7FFFu));
        return max(m << 16, m & 0xFFFF0000u);
    } else {
        return max(max(v.x & 0x7FFFFFFFu, v.y & 0x7FFFFFFFu), max(v.z & 0x7FFFFFFFu, v.w & 0x7FFFFFFFu));
    }
}

// Codes of a 16-byte chunk scaled by sc (= 2^-e, exact products), in
// element format FMT; CLIP limits values to the format's maximum first.
template <int FMT = FMT_E4M3, bool CLIP = false>
__device__ __forceinline__ uint2 chunk_codes_bf16(uint4 v, float sc)
{
    uint2 o;
    o.x = cvt4_fmt<FMT, CLIP>(bf16lo(v.x) * sc, bf16hi(v.x) * sc, bf16lo(v.y) * sc, bf16hi(v.y) * sc);
    o.y = cvt4_fmt<FMT, CLIP>(bf16lo(v.z) * sc, bf16hi(v.z) * sc, bf16lo(v.w) * sc, bf16hi(v.w) * sc);
    return o;
}
template <int FMT = FMT_E4M3, bool CLIP = false>
__device__ __forceinline__ uint32_t chunk_codes_f32(uint4 v, float sc)
{
    return cvt4_fmt<FMT, CLIP>(__uint_as_float(v.x) * sc, __uint_as_float(v.y) * sc,
                               __uint_as_float(v.z) * sc, __uint_as_float(v.w) * sc);
}

// One wave per row (grid-stride over rows); each lane owns a 16-byte chunk,
// LPG consecutive lanes form one group; U chunks per lane are in flight.
// FMT / RULE: element format and scale rule (E4M3 with the ceil rule is the
// path's default; the floor rule clips the values it scales past the maximum).
template <bool BF16, int GROUP, int FMT = FMT_E4M3, int RULE = RULE_CEIL>
__global__ __launch_bounds__(256) void quant_rowwise_kernel(const uint8_t *__restrict__ x,
                                                            int64_t rows, int64_t cpr,
                                                            int64_t ldx_bytes,
                                                            uint8_t *__restrict__ q, int64_t ldq,
                                                            uint8_t *__restrict__ s, int64_t lds,
                                                            int emin)
{
    constexpr int EPC = BF16 ? 8 : 4; // elements per chunk
    constexpr int LPG = GROUP / EPC;  // lanes per group
    constexpr int U = 4;
    const int lane = lane_id();
    const int64_t wave = ((int64_t)blockIdx.x * blockDim.x + threadIdx.x) >> 6;
    const int64_t nwaves = ((int64_t)gridDim.x * blockDim.x) >> 6;
    for (int64_t r = wave; r < rows; r += nwaves) {
        const uint8_t *xr = x + r * ldx_bytes;
        uint8_t *qr = q + r * ldq;
        uint8_t *sr = s + r * lds;
        for (int64_t c0 = 0; c0 < cpr; c0 += 64 * U) {
            uint4 v[U];
#pragma unroll
            for (int u = 0; u < U; u++) {
                int64_t c = c0 + u * 64 + lane;
                v[u] = c < cpr ? ld_stream16(xr + c * 16) : make_uint4(0, 0, 0, 0);
            }
#pragma unroll
            for (int u = 0; u < U; u++) {
                int64_t c = c0 + u * 64 + lane;
                uint32_t m = group_max_u32<LPG>(chunk_amax_bits<BF16>(v[u]));
                int e = scale_exp_fmt<FMT, RULE>(m, emin);
                float sc = pow2f(-e);
                if (c < cpr) {
                    if constexpr (BF16)
                        st_stream8(qr + c * 8, chunk_codes_bf16<FMT, RULE == RULE_OCP_FLOOR>(v[u], sc));
                    else
                        st_stream4(qr + c * 4, chunk_codes_f32<FMT, RULE == RULE_OCP_FLOOR>(v[u], sc));
                    if (lane % LPG == 0)
                        sr[c / LPG] = (uint8_t)(e + 127);
                }
            }
        }
    }
}

// One workgroup (256 threads) per 128x128 block: load the block into
// registers, reduce amax across the workgroup, convert from registers.
template <bool BF16>
__global__ __launch_bounds__(256) void quant_blockwise_kernel(const uint8_t *__restrict__ w,
                                                              int64_t rows, int64_t ldw_bytes,
                                                              uint8_t *__restrict__ q, int64_t ldq,
                                                              uint8_t *__restrict__ s, int64_t lds,
                                                              int64_t nbc)
{
    constexpr int EPC = BF16 ? 8 : 4;
    constexpr int CPB = 128 / EPC;   // chunks per block row
    constexpr int RPP = 256 / CPB;   // rows per pass
    constexpr int NP = 128 / RPP;    // passes
    __shared__ uint32_t red[4];
    const int64_t rb = blockIdx.x / nbc, cb = blockIdx.x % nbc;
    const int t = threadIdx.x;
    const int ch = t % CPB, r0 = t / CPB;
    uint4 v[NP];
    uint32_t m = 0;
#pragma unroll
    for (int i = 0; i < NP; i++) {
        int64_t r = rb * 128 + r0 + i * RPP;
        v[i] = r < rows ? ld_stream16(w + r * ldw_bytes + (cb * 128 + ch * EPC) * (BF16 ? 2 : 4))
                        : make_uint4(0, 0, 0, 0);
        m = max(m, chunk_amax_bits<BF16>(v[i]));
    }
    m = group_max_u32<64>(m);
    if (lane_id() == 0)
        red[t >> 6] = m;
    __syncthreads();
    m = max(max(red[0], red[1]), max(red[2], red[3]));
    int e = scale_exp_from_bits(m, -22);
    float sc = pow2f(-e);
#pragma unroll
    for (int i = 0; i < NP; i++) {
        int64_t r = rb * 128 + r0 + i * RPP;
        if (r < rows) {
            uint8_t *dst = q + r * ldq + cb * 128 + ch * EPC;
            if constexpr (BF16)
                st_stream8(dst, chunk_codes_bf16(v[i], sc));
            else
                st_stream4(dst, chunk_codes_f32(v[i], sc));
        }
    }
    if (t == 0)
        s[rb * lds + cb] = (uint8_t)(e + 127);
}

// 128x128 quantization of bf16 weights that also writes the transposed
// codes (the exact k = 0 byte transpose of each block, whose scale is
// symmetric): one wave per block.  Lane (tsub = lane & 7, csub = lane >> 3)
// owns the 16x16 sub-tile at rows tsub*16.., columns csub*16..: 16 rows of
// 32 bytes in registers (8 lanes cover a 256-byte row segment), the block's
// amax by a wave reduction, codes stored as 16-byte row pieces, then a 16x16
// byte transpose in registers (v_perm_b32) stored as 16-byte column pieces
// (8 lanes cover a 128-byte row of the transposed copy).  Blocks run
// column-block-fastest within a matrix, so the four waves of a workgroup read
// 1 KB of each bf16 row together (measured faster than row-block-fastest,
// which groups the transposed copy's writes instead).
__device__ __forceinline__ void tr4x4b(uint32_t a, uint32_t b, uint32_t c, uint32_t d, uint32_t &o0, uint32_t &o1,
                                       uint32_t &o2, uint32_t &o3)
{
    const uint32_t ab_lo = __builtin_amdgcn_perm(b, a, 0x05010400u);
    const uint32_t ab_hi = __builtin_amdgcn_perm(b, a, 0x07030602u);
    const uint32_t cd_lo = __builtin_amdgcn_perm(d, c, 0x05010400u);
    const uint32_t cd_hi = __builtin_amdgcn_perm(d, c, 0x07030602u);
    o0 = __builtin_amdgcn_perm(cd_lo, ab_lo, 0x05040100u);
    o1 = __builtin_amdgcn_perm(cd_lo, ab_lo, 0x07060302u);
    o2 = __builtin_amdgcn_perm(cd_hi, ab_hi, 0x05040100u);
    o3 = __builtin_amdgcn_perm(cd_hi, ab_hi, 0x07060302u);
}

__global__ __launch_bounds__(256) void quant_blockwise_t_kernel(const uint16_t *__restrict__ w, int64_t rows,
                                                                int64_t cols, int64_t nblocks,
                                                                uint8_t *__restrict__ q, uint8_t *__restrict__ s,
                                                                uint8_t *__restrict__ qt,
                                                                uint8_t *__restrict__ st)
{
    const int lane = lane_id();
    const int64_t blk = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    if (blk >= nblocks)
        return; // uniform per wave
    const int64_t nrb = rows / 128, ncb = cols / 128, per = nrb * ncb;
    const int64_t g = blk / per, bi = blk % per;
    const int64_t rb = bi / ncb, cb = bi % ncb;
    w += g * rows * cols;
    q += g * rows * cols;
    qt += g * rows * cols;
    s += g * per;
    st += g * per;
    const int tsub = lane & 7, csub = lane >> 3;
    const int64_t r0 = rb * 128 + tsub * 16, c0 = cb * 128 + csub * 16;
    uint4 v[16][2];
    uint32_t m = 0;
#pragma unroll
    for (int j = 0; j < 16; j++) {
        const uint16_t *src = w + (r0 + j) * cols + c0;
        v[j][0] = ld_stream16(src);
        v[j][1] = ld_stream16(src + 8);
        m = max(m, max(chunk_amax_bits<true>(v[j][0]), chunk_amax_bits<true>(v[j][1])));
    }
    m = group_max_u32<64>(m);
    const int e = scale_exp_from_bits(m, -22);
    const float sc = pow2f(-e);
    uint32_t c[16][4]; // c[j]: the 16 codes of row r0+j
#pragma unroll
    for (int j = 0; j < 16; j++) {
        const uint2 lo = chunk_codes_bf16(v[j][0], sc), hi = chunk_codes_bf16(v[j][1], sc);
        c[j][0] = lo.x;
        c[j][1] = lo.y;
        c[j][2] = hi.x;
        c[j][3] = hi.y;
        st_stream16(q + (r0 + j) * cols + c0, make_uint4(c[j][0], c[j][1], c[j][2], c[j][3]));
    }
    uint32_t o[16][4]; // o[k][i]: column c0+k, rows r0+4i .. r0+4i+3
#pragma unroll
    for (int i = 0; i < 4; i++)
#pragma unroll
        for (int x = 0; x < 4; x++)
            tr4x4b(c[4 * i + 0][x], c[4 * i + 1][x], c[4 * i + 2][x], c[4 * i + 3][x], o[4 * x + 0][i],
                   o[4 * x + 1][i], o[4 * x + 2][i], o[4 * x + 3][i]);
#pragma unroll
    for (int k = 0; k < 16; k++)
        st_stream16(qt + (c0 + k) * rows + r0, make_uint4(o[k][0], o[k][1], o[k][2], o[k][3]));
    if (lane == 0) {
        s[rb * ncb + cb] = (uint8_t)(e + 127);
        st[cb * nrb + rb] = (uint8_t)(e + 127);
    }
}

// Each thread decodes one 16-byte chunk of codes (16 codes of one scale group).
template <bool OUT_BF16, int FMT = FMT_E4M3>
__global__ __launch_bounds__(256) void dequant_kernel(const uint8_t *__restrict__ q,
                                                      const uint8_t *__restrict__ s, int gran,
                                                      int64_t rows, int64_t cols,
                                                      void *__restrict__ out)
{
    const int64_t nch = rows * (cols / 16);
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < nch;
         i += (int64_t)gridDim.x * blockDim.x) {
        int64_t r = i / (cols / 16), c = (i % (cols / 16)) * 16;
        int sb;
        if (gran == FGB_BLOCK128)
            sb = s[(r / 128) * (cols / 128) + c / 128];
        else if (gran == FGB_ROW1x32)
            sb = s[r * (cols / 32) + c / 32];
        else
            sb = s[r * (cols / 128) + c / 128];
        int e = sb - 127;
        uint4 v = *reinterpret_cast<const uint4 *>(q + r * cols + c);
        uint32_t w[4] = {v.x, v.y, v.z, v.w};
        float f[16];
#pragma unroll
        for (int j = 0; j < 4; j++) {
            float2 a = FMT == FMT_E5M2 ? dec2_lo_e5m2(w[j]) : dec2_lo(w[j]);
            float2 b = FMT == FMT_E5M2 ? dec2_hi_e5m2(w[j]) : dec2_hi(w[j]);
            f[4 * j + 0] = ldexpf(a.x, e);
            f[4 * j + 1] = ldexpf(a.y, e);
            f[4 * j + 2] = ldexpf(b.x, e);
            f[4 * j + 3] = ldexpf(b.y, e);
        }
        if constexpr (OUT_BF16) {
            uint32_t o[8];
#pragma unroll
            for (int j = 0; j < 8; j++)
                o[j] = bf16_rne(f[2 * j]) | (bf16_rne(f[2 * j + 1]) << 16);
            uint4 *dst = reinterpret_cast<uint4 *>((uint16_t *)out + r * cols + c);
            dst[0] = make_uint4(o[0], o[1], o[2], o[3]);
            dst[1] = make_uint4(o[4], o[5], o[6], o[7]);
        } else {
            float4 *dst = reinterpret_cast<float4 *>((float *)out + r * cols + c);
#pragma unroll
            for (int j = 0; j < 4; j++)
                dst[j] = make_float4(f[4 * j], f[4 * j + 1], f[4 * j + 2], f[4 * j + 3]);
        }
    }
}

template <int FMT>
__global__ __launch_bounds__(256) void encode_kernel(const float *__restrict__ x, int64_t n,
                                                     uint8_t *__restrict__ q)
{
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i * 4 < n;
         i += (int64_t)gridDim.x * blockDim.x) {
        float v[4];
#pragma unroll
        for (int j = 0; j < 4; j++) {
            v[j] = i * 4 + j < n ? x[i * 4 + j] : 0.0f;
        }
        uint32_t w = cvt4_fmt<FMT, true>(v[0], v[1], v[2], v[3]);
        if (i * 4 + 3 < n) {
            *reinterpret_cast<uint32_t *>(q + i * 4) = w;
        } else {
            for (int j = 0; j < 4 && i * 4 + j < n; j++)
                q[i * 4 + j] = (uint8_t)(w >> (8 * j));
        }
    }
}

static int grid_for(int64_t work, int64_t per_block, int64_t cap)
{
    int64_t g = (work + per_block - 1) / per_block;
    if (g < 1)
        g = 1;
    return (int)(g < cap ? g : cap);
}

} // namespace fgb

using namespace fgb;

template <int FMT, int RULE>
static void launch_rowwise(const void *x, bool bf16, int group, int64_t rows, int64_t cpr, int64_t ldx_bytes, uint8_t *q,
                           int64_t ldq, uint8_t *s, int64_t lds, int emin, int grid, hipStream_t st)
{
    const uint8_t *xb = (const uint8_t *)x;
    if (bf16 && group == 128)
        quant_rowwise_kernel<true, 128, FMT, RULE><<<grid, 256, 0, st>>>(xb, rows, cpr, ldx_bytes, q, ldq, s, lds, emin);
    else if (bf16)
        quant_rowwise_kernel<true, 32, FMT, RULE><<<grid, 256, 0, st>>>(xb, rows, cpr, ldx_bytes, q, ldq, s, lds, emin);
    else if (group == 128)
        quant_rowwise_kernel<false, 128, FMT, RULE><<<grid, 256, 0, st>>>(xb, rows, cpr, ldx_bytes, q, ldq, s, lds, emin);
    else
        quant_rowwise_kernel<false, 32, FMT, RULE><<<grid, 256, 0, st>>>(xb, rows, cpr, ldx_bytes, q, ldq, s, lds, emin);
}

extern "C" int fp8_quant_rowwise_fmt(const void *x, int x_dtype, int64_t rows, int64_t cols, int64_t ldx, int group,
                                     int fmt, int rule, uint8_t *q, int64_t ldq, uint8_t *s, int64_t lds, void *stream)
{
    clear_error();
    FGB_REQUIRE(x && q && s, FGB_EINVAL, "fp8_quant_rowwise: null pointer");
    FGB_REQUIRE(x_dtype == FGB_F32 || x_dtype == FGB_BF16, FGB_EUNSUPPORTED,
                "fp8_quant_rowwise: x_dtype must be FGB_F32 or FGB_BF16");
    FGB_REQUIRE(group == 128 || group == 32, FGB_EUNSUPPORTED,
                "fp8_quant_rowwise: group must be 128 or 32");
    FGB_REQUIRE(fmt == FGB_E4M3 || fmt == FGB_E5M2, FGB_EUNSUPPORTED,
                "fp8_quant_rowwise: fmt must be FGB_E4M3 or FGB_E5M2");
    FGB_REQUIRE(rule == FGB_SCALE_CEIL || rule == FGB_SCALE_OCP_FLOOR, FGB_EUNSUPPORTED,
                "fp8_quant_rowwise: rule must be FGB_SCALE_CEIL or FGB_SCALE_OCP_FLOOR");
    FGB_REQUIRE(rows >= 0 && cols > 0 && cols % group == 0, FGB_EINVAL,
                "fp8_quant_rowwise: cols must be a positive multiple of group (rows=%lld cols=%lld)",
                (long long)rows, (long long)cols);
    int esz = x_dtype == FGB_F32 ? 4 : 2;
    FGB_REQUIRE(ldx >= cols && (ldx * esz) % 16 == 0, FGB_EINVAL,
                "fp8_quant_rowwise: ldx must be >= cols and ldx*elem_size a multiple of 16");
    FGB_REQUIRE(ldq >= cols && ldq % 16 == 0, FGB_EINVAL,
                "fp8_quant_rowwise: ldq must be >= cols and a multiple of 16");
    FGB_REQUIRE(lds >= cols / group, FGB_EINVAL, "fp8_quant_rowwise: lds must be >= cols/group");
    FGB_REQUIRE(aligned16(x) && aligned16(q), FGB_EINVAL,
                "fp8_quant_rowwise: x and q must be 16-byte aligned");
    if (rows == 0)
        return FGB_OK;
    hipStream_t st = (hipStream_t)stream;
    int64_t cpr = cols * esz / 16;
    // the 1e-4 amax clamp for 128-element groups, the E8M0 range for 32
    int emin = group == 128 ? (fmt == FGB_E5M2 ? -29 : -22) : -127;
    int grid = grid_for(rows, 4, 16384);
    const bool bf16 = x_dtype == FGB_BF16;
    if (fmt == FGB_E4M3 && rule == FGB_SCALE_CEIL)
        launch_rowwise<FMT_E4M3, RULE_CEIL>(x, bf16, group, rows, cpr, ldx * esz, q, ldq, s, lds, emin, grid, st);
    else if (fmt == FGB_E4M3)
        launch_rowwise<FMT_E4M3, RULE_OCP_FLOOR>(x, bf16, group, rows, cpr, ldx * esz, q, ldq, s, lds, emin, grid, st);
    else if (rule == FGB_SCALE_CEIL)
        launch_rowwise<FMT_E5M2, RULE_CEIL>(x, bf16, group, rows, cpr, ldx * esz, q, ldq, s, lds, emin, grid, st);
    else
        launch_rowwise<FMT_E5M2, RULE_OCP_FLOOR>(x, bf16, group, rows, cpr, ldx * esz, q, ldq, s, lds, emin, grid, st);
    FGB_LAUNCHED("fp8_quant_rowwise");
    return FGB_OK;
}

extern "C" int fp8_quant_rowwise(const void *x, int x_dtype, int64_t rows, int64_t cols, int64_t ldx, int group,
                                 uint8_t *q, int64_t ldq, uint8_t *s, int64_t lds, void *stream)
{
    return fp8_quant_rowwise_fmt(x, x_dtype, rows, cols, ldx, group, FGB_E4M3, FGB_SCALE_CEIL, q, ldq, s, lds,
                                 stream);
}

extern "C" int fp8_quant_blockwise(const void *w, int w_dtype, int64_t rows, int64_t cols,
                                   int64_t ldw, uint8_t *q, int64_t ldq, uint8_t *s, int64_t lds,
                                   void *stream)
{
    clear_error();
    FGB_REQUIRE(w && q && s, FGB_EINVAL, "fp8_quant_blockwise: null pointer");
    FGB_REQUIRE(w_dtype == FGB_F32 || w_dtype == FGB_BF16, FGB_EUNSUPPORTED,
                "fp8_quant_blockwise: w_dtype must be FGB_F32 or FGB_BF16");
    FGB_REQUIRE(rows >= 0 && cols > 0 && cols % 128 == 0, FGB_EINVAL,
                "fp8_quant_blockwise: cols must be a positive multiple of 128");
    int esz = w_dtype == FGB_F32 ? 4 : 2;
    FGB_REQUIRE(ldw >= cols && (ldw * esz) % 16 == 0, FGB_EINVAL,
                "fp8_quant_blockwise: ldw must be >= cols and ldw*elem_size a multiple of 16");
    FGB_REQUIRE(ldq >= cols && ldq % 16 == 0, FGB_EINVAL,
                "fp8_quant_blockwise: ldq must be >= cols and a multiple of 16");
    FGB_REQUIRE(lds >= cols / 128, FGB_EINVAL, "fp8_quant_blockwise: lds must be >= cols/128");
    FGB_REQUIRE(aligned16(w) && aligned16(q), FGB_EINVAL,
                "fp8_quant_blockwise: w and q must be 16-byte aligned");
    if (rows == 0)
        return FGB_OK;
    hipStream_t st = (hipStream_t)stream;
    int64_t nbr = (rows + 127) / 128, nbc = cols / 128;
    int64_t nb = nbr * nbc;
    FGB_REQUIRE(nb < (1ll << 31), FGB_EINVAL, "fp8_quant_blockwise: too many blocks");
    if (w_dtype == FGB_BF16)
        quant_blockwise_kernel<true><<<(int)nb, 256, 0, st>>>((const uint8_t *)w, rows, ldw * esz, q, ldq, s, lds, nbc);
    else
        quant_blockwise_kernel<false><<<(int)nb, 256, 0, st>>>((const uint8_t *)w, rows, ldw * esz, q, ldq, s, lds, nbc);
    FGB_LAUNCHED("fp8_quant_blockwise");
    return FGB_OK;
}

extern "C" int fp8_quant_blockwise_t(const void *w, int w_dtype, int G, int64_t rows, int64_t cols, uint8_t *q,
                                     uint8_t *s, uint8_t *qt, uint8_t *st, void *stream)
{
    clear_error();
    FGB_REQUIRE(w && q && s && qt && st, FGB_EINVAL, "fp8_quant_blockwise_t: null pointer");
    FGB_REQUIRE(w_dtype == FGB_BF16, FGB_EUNSUPPORTED, "fp8_quant_blockwise_t: w_dtype must be FGB_BF16");
    FGB_REQUIRE(G >= 1 && rows >= 0 && cols >= 0 && rows % 128 == 0 && cols % 128 == 0, FGB_EINVAL,
                "fp8_quant_blockwise_t: need G >= 1 and rows, cols multiples of 128 (rows=%lld cols=%lld)",
                (long long)rows, (long long)cols);
    FGB_REQUIRE(aligned16(w) && aligned16(q) && aligned16(qt), FGB_EINVAL,
                "fp8_quant_blockwise_t: w, q and qt must be 16-byte aligned");
    const int64_t nb = (int64_t)G * (rows / 128) * (cols / 128);
    if (nb == 0)
        return FGB_OK;
    FGB_REQUIRE((nb + 3) / 4 < (1ll << 31), FGB_EINVAL, "fp8_quant_blockwise_t: too many blocks");
    quant_blockwise_t_kernel<<<(unsigned)((nb + 3) / 4), 256, 0, (hipStream_t)stream>>>((const uint16_t *)w, rows, cols,
                                                                                      nb, q, s, qt, st);
    FGB_LAUNCHED("fp8_quant_blockwise_t");
    return FGB_OK;
}

extern "C" int fp8_dequant_fmt(const uint8_t *q, const uint8_t *s, int gran, int fmt, int64_t rows, int64_t cols,
                               void *out, int out_dtype, void *stream)
{
    clear_error();
    FGB_REQUIRE(fmt == FGB_E4M3 || fmt == FGB_E5M2, FGB_EUNSUPPORTED, "fp8_dequant: fmt must be FGB_E4M3 or FGB_E5M2");
    FGB_REQUIRE(q && s && out, FGB_EINVAL, "fp8_dequant: null pointer");
    FGB_REQUIRE(gran == FGB_ROW1x128 || gran == FGB_ROW1x32 || gran == FGB_BLOCK128,
                FGB_EUNSUPPORTED, "fp8_dequant: unknown granularity");
    FGB_REQUIRE(out_dtype == FGB_F32 || out_dtype == FGB_BF16, FGB_EUNSUPPORTED,
                "fp8_dequant: out_dtype must be FGB_F32 or FGB_BF16");
    int g = gran == FGB_ROW1x32 ? 32 : 128;
    FGB_REQUIRE(rows >= 0 && cols > 0 && cols % g == 0, FGB_EINVAL,
                "fp8_dequant: cols must be a positive multiple of the group");
    FGB_REQUIRE(aligned16(q) && aligned16(out), FGB_EINVAL, "fp8_dequant: q and out must be 16-byte aligned");
    if (rows == 0)
        return FGB_OK;
    hipStream_t st = (hipStream_t)stream;
    int grid = grid_for(rows * (cols / 16), 256, 1 << 16);
    if (out_dtype == FGB_BF16 && fmt == FGB_E5M2)
        dequant_kernel<true, FMT_E5M2><<<grid, 256, 0, st>>>(q, s, gran, rows, cols, out);
    else if (out_dtype == FGB_BF16)
        dequant_kernel<true><<<grid, 256, 0, st>>>(q, s, gran, rows, cols, out);
    else if (fmt == FGB_E5M2)
        dequant_kernel<false, FMT_E5M2><<<grid, 256, 0, st>>>(q, s, gran, rows, cols, out);
    else
        dequant_kernel<false><<<grid, 256, 0, st>>>(q, s, gran, rows, cols, out);
    FGB_LAUNCHED("fp8_dequant");
    return FGB_OK;
}

extern "C" int fp8_dequant(const uint8_t *q, const uint8_t *s, int gran, int64_t rows, int64_t cols, void *out,
                           int out_dtype, void *stream)
{
    return fp8_dequant_fmt(q, s, gran, FGB_E4M3, rows, cols, out, out_dtype, stream);
}

extern "C" int fgb_fp8_encode(const float *x, int64_t n, int fmt, uint8_t *q, void *stream)
{
    clear_error();
    FGB_REQUIRE(x && q, FGB_EINVAL, "fgb_fp8_encode: null pointer");
    FGB_REQUIRE(n >= 0, FGB_EINVAL, "fgb_fp8_encode: negative n");
    FGB_REQUIRE(fmt == FGB_E4M3 || fmt == FGB_E5M2, FGB_EUNSUPPORTED, "fgb_fp8_encode: fmt must be FGB_E4M3 or FGB_E5M2");
    FGB_REQUIRE(((uintptr_t)x & 15) == 0 && ((uintptr_t)q & 3) == 0, FGB_EINVAL,
                "fgb_fp8_encode: x must be 16-byte and q 4-byte aligned");
    if (n == 0)
        return FGB_OK;
    int grid = grid_for((n + 3) / 4, 256, 1 << 16);
    if (fmt == FGB_E5M2)
        encode_kernel<FMT_E5M2><<<grid, 256, 0, (hipStream_t)stream>>>(x, n, q);
    else
        encode_kernel<FMT_E4M3><<<grid, 256, 0, (hipStream_t)stream>>>(x, n, q);
    FGB_LAUNCHED("fgb_fp8_encode");
    return FGB_OK;
}

extern "C" int fgb_e4m3_encode(const float *x, int64_t n, uint8_t *q, void *stream)
{
    return fgb_fp8_encode(x, n, FGB_E4M3, q, stream);
}
