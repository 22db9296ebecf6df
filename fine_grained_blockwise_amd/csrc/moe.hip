// moe.hip -- MoE expert data movement on row-wise FP8, and fused SwiGLU + quant.
//
// awesome-system-papers, "FP8-Flow-MoE: A Casting-Free FP8 Recipe without
// Double Quantization Error", "Core method": fused permute + 16-aligned padding,
// fused unpermute + unpadding, and SwiGLU fused with quantization so the
// activation boundary emits FP8 directly; assumption 2: the expert linears'
// outputs stay BF16 (the fc1 output feeding the activation, the fc2 output
// feeding the combine).
//
// permute_pad runs in four launches, none of which needs a host sync:
//   count   per chunk of tokens, a histogram of expert ids (LDS integer atomics)
//   scan    per expert: total, padded segment size, segment start, and the
//           start of each chunk's run inside the segment
//   rowmap  per chunk, the rank of every (token, slot) among the chunk's slots
//           of the same expert, in (token, slot) order -> row_map
//   copy    one wave per token: the 16-byte chunks of the code row and the
//           scale row are read once (streaming loads) and written to each
//           destination with ordinary stores (the kernel's traffic is ~90%
//           writes; ordinary stores measured 3% faster here); extra
//           waves fill the padding rows (code 0, scale byte 105 -- what
//           the 1x128 rule gives an all-zero tile).
#include "fgb_internal.h"

#include <mutex>

namespace fgb {

constexpr int PP_CHUNK = 256; // tokens per histogram chunk

struct PPWorkspace {
    int32_t *cnt;    // [nchunks][G] slots per chunk per expert
    int32_t *base;   // [nchunks][G] first destination row of the chunk's run
    int32_t *total;  // [G] slots per expert
};

static size_t pp_nchunks(int64_t T) { return (size_t)((T + PP_CHUNK - 1) / PP_CHUNK); }

static PPWorkspace pp_carve(void *ws, int64_t T, int G)
{
    size_t nc = pp_nchunks(T);
    PPWorkspace w;
    w.cnt = (int32_t *)ws;
    w.base = w.cnt + nc * G;
    w.total = w.base + nc * G;
    return w;
}

__global__ __launch_bounds__(256) void pp_count_kernel(const int32_t *__restrict__ idx, int64_t T,
                                                       int topk, int G, int32_t *__restrict__ cnt)
{
    extern __shared__ int32_t hist[];
    for (int e = threadIdx.x; e < G; e += blockDim.x)
        hist[e] = 0;
    __syncthreads();
    int64_t t0 = (int64_t)blockIdx.x * PP_CHUNK;
    int64_t t1 = min(t0 + PP_CHUNK, T);
    for (int64_t i = t0 * topk + threadIdx.x; i < t1 * topk; i += blockDim.x) {
        int e = idx[i];
        if (e >= 0 && e < G)
            atomicAdd(&hist[e], 1);
    }
    __syncthreads();
    for (int e = threadIdx.x; e < G; e += blockDim.x)
        cnt[(int64_t)blockIdx.x * G + e] = hist[e];
}

__global__ __launch_bounds__(256) void pp_scan_kernel(const int32_t *__restrict__ cnt, int nchunks,
                                                      int G, int pad, int32_t *__restrict__ base,
                                                      int32_t *__restrict__ total,
                                                      int32_t *__restrict__ offs)
{
    extern __shared__ int32_t sh[]; // [G] padded sizes, [G+1] offsets, [256] slice sums
    int32_t *padded = sh, *off = sh + G, *part = sh + 2 * G + 1;
    // S threads per expert (G <= 128), each summing a slice of the chunks;
    // with more experts one thread per expert walks all chunks.
    const int S = G <= 128 ? 256 / G : 1;
    const int per = (nchunks + S - 1) / S;
    if (S > 1) {
        const int e = threadIdx.x / S, j = threadIdx.x % S;
        const bool act = e < G;
        const int c0 = min(nchunks, j * per), c1 = min(nchunks, c0 + per);
        int32_t sum = 0;
        if (act)
            for (int c = c0; c < c1; c++)
                sum += cnt[(int64_t)c * G + e];
        part[threadIdx.x] = sum;
        __syncthreads();
        if (act && j == 0) {
            int32_t t = 0;
            for (int k = 0; k < S; k++)
                t += part[threadIdx.x + k];
            total[e] = t;
            padded[e] = (t + pad - 1) / pad * pad;
        }
    } else {
        for (int e = threadIdx.x; e < G; e += blockDim.x) {
            int32_t t = 0;
            for (int c = 0; c < nchunks; c++)
                t += cnt[(int64_t)c * G + e];
            total[e] = t;
            padded[e] = (t + pad - 1) / pad * pad;
        }
    }
    __syncthreads();
    if (threadIdx.x == 0) {
        int32_t acc = 0;
        for (int e = 0; e < G; e++) {
            off[e] = acc;
            acc += padded[e];
        }
        off[G] = acc;
    }
    __syncthreads();
    for (int e = threadIdx.x; e <= G; e += blockDim.x)
        offs[e] = off[e];
    if (S > 1) {
        const int e = threadIdx.x / S, j = threadIdx.x % S;
        if (e < G) {
            int32_t run = off[e];
            for (int k = 0; k < j; k++)
                run += part[e * S + k]; // the expert's slots in earlier slices
            const int c0 = min(nchunks, j * per), c1 = min(nchunks, c0 + per);
            for (int c = c0; c < c1; c++) {
                base[(int64_t)c * G + e] = run;
                run += cnt[(int64_t)c * G + e];
            }
        }
    } else {
        for (int e = threadIdx.x; e < G; e += blockDim.x) {
            int32_t run = off[e];
            for (int c = 0; c < nchunks; c++) {
                base[(int64_t)c * G + e] = run;
                run += cnt[(int64_t)c * G + e];
            }
        }
    }
}

// Ranks inside a chunk: slots are taken 256 at a time in (token, slot) order;
// a slot's rank = running count of its expert + slots of the same expert in
// earlier waves of this pass + same-expert lanes below it in its wave.
__global__ __launch_bounds__(256) void pp_rowmap_kernel(const int32_t *__restrict__ idx, int64_t T,
                                                        int topk, int G,
                                                        const int32_t *__restrict__ base,
                                                        int32_t *__restrict__ row_map)
{
    extern __shared__ int32_t sm[]; // running[G], wcnt[4][G]
    int32_t *running = sm, *wcnt = sm + G;
    const int lane = lane_id(), wave = threadIdx.x >> 6;
    for (int e = threadIdx.x; e < G; e += blockDim.x)
        running[e] = base[(int64_t)blockIdx.x * G + e];
    int nbits = 0;
    while ((1 << nbits) < G + 1)
        nbits++;
    int64_t s0 = (int64_t)blockIdx.x * PP_CHUNK * topk;
    int64_t s1 = min((int64_t)(blockIdx.x + 1) * PP_CHUNK, T) * topk;
    for (int64_t p = s0; p < s1; p += 256) {
        for (int e = threadIdx.x; e < 4 * G; e += blockDim.x)
            wcnt[e] = 0;
        __syncthreads();
        int64_t i = p + threadIdx.x;
        int e = i < s1 ? idx[i] : -1;
        int key = (e >= 0 && e < G) ? e : G; // G = dropped / out of range
        uint64_t peers = __ballot(i < s1);
        for (int b = 0; b < nbits; b++) {
            uint64_t m = __ballot((key >> b) & 1);
            peers &= ((key >> b) & 1) ? m : ~m;
        }
        uint64_t below = lane == 0 ? 0ull : (~0ull >> (64 - lane));
        int rank_w = __popcll(peers & below);
        bool leader = (peers & below) == 0;
        if (i < s1 && key < G && leader)
            wcnt[wave * G + key] = __popcll(peers);
        __syncthreads();
        if (i < s1) {
            if (key < G) {
                int r = running[key] + rank_w;
                for (int w = 0; w < wave; w++)
                    r += wcnt[w * G + key];
                row_map[i] = r;
            } else {
                row_map[i] = -1;
            }
        }
        __syncthreads();
        for (int ee = threadIdx.x; ee < G; ee += blockDim.x)
            running[ee] += wcnt[ee] + wcnt[G + ee] + wcnt[2 * G + ee] + wcnt[3 * G + ee];
        __syncthreads();
    }
}

// One wave per token (blocks [0, tok_blocks)), then one wave per potential
// padding row (pad-1 per expert).
__global__ __launch_bounds__(256) void pp_copy_kernel(const uint8_t *__restrict__ xq,
                                                      const uint8_t *__restrict__ xs,
                                                      const int32_t *__restrict__ row_map,
                                                      int64_t T, int topk, int G, int64_t H,
                                                      int pad, const int32_t *__restrict__ total,
                                                      const int32_t *__restrict__ offs,
                                                      uint8_t *__restrict__ out_q,
                                                      uint8_t *__restrict__ out_s, int64_t tok_blocks,
                                                      int64_t M_cap)
{
    const int lane = lane_id(), wave = threadIdx.x >> 6;
    const int64_t H16 = H / 16, H128 = H / 128;
    if ((int64_t)blockIdx.x < tok_blocks) {
        int64_t t = (int64_t)blockIdx.x * 4 + wave;
        if (t >= T)
            return;
        int32_t my_row = lane < topk ? row_map[t * topk + lane] : -1;
        my_row = my_row < M_cap ? my_row : -1; // defensive: never write past the buffer
        const uint8_t *src = xq + t * H;
        for (int64_t c0 = 0; c0 < H16; c0 += 64 * 8) {
            uint4 v[8];
#pragma unroll
            for (int u = 0; u < 8; u++) {
                int64_t c = c0 + u * 64 + lane;
                v[u] = c < H16 ? ld_stream16(src + c * 16) : make_uint4(0, 0, 0, 0);
            }
            for (int k = 0; k < topk; k++) {
                int32_t r = __shfl(my_row, k);
                if (r < 0)
                    continue;
                uint8_t *dst = out_q + (int64_t)r * H;
#pragma unroll
                for (int u = 0; u < 8; u++) {
                    int64_t c = c0 + u * 64 + lane;
                    if (c < H16)
                        st_plain16(dst + c * 16, v[u]);
                }
            }
        }
        for (int64_t c0 = 0; c0 < H128; c0 += 64) {
            int64_t c = c0 + lane;
            uint8_t sv = c < H128 ? xs[t * H128 + c] : 0;
            for (int k = 0; k < topk; k++) {
                int32_t r = __shfl(my_row, k);
                if (r >= 0 && c < H128)
                    out_s[(int64_t)r * H128 + c] = sv;
            }
        }
    } else {
        int64_t pidx = ((int64_t)blockIdx.x - tok_blocks) * 4 + wave;
        if (pad <= 1 || pidx >= (int64_t)(pad - 1) * G)
            return;
        int e = (int)(pidx / (pad - 1)), j = (int)(pidx % (pad - 1));
        int64_t r = (int64_t)offs[e] + total[e] + j;
        if (r >= offs[e + 1])
            return;
        uint8_t *dst = out_q + r * H;
        for (int64_t c = lane; c < H16; c += 64)
            st_plain16(dst + c * 16, make_uint4(0, 0, 0, 0));
        for (int64_t c = lane; c < H128; c += 64)
            out_s[r * H128 + c] = 105;
    }
}

// ---------------------------------------------------------------------------
// unpermute + unpad: one wave per token; each lane owns 16-byte chunks (8 bf16)
// of the output row, four per pass (2-6% faster than two); the topk source
// rows are gathered 8 at a time with all their loads in flight, then folded
// in slot order with fused multiply-adds.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void unpermute_kernel(const uint16_t *__restrict__ y,
                                                        const int32_t *__restrict__ row_map,
                                                        const float *__restrict__ probs, int64_t T,
                                                        int topk, int64_t H,
                                                        uint16_t *__restrict__ out)
{
    const int lane = lane_id();
    const int64_t H8 = H / 8;
    const int64_t wave = ((int64_t)blockIdx.x * blockDim.x + threadIdx.x) >> 6;
    const int64_t nwaves = ((int64_t)gridDim.x * blockDim.x) >> 6;
    for (int64_t t = wave; t < T; t += nwaves) {
        int32_t my_row = lane < topk ? row_map[t * topk + lane] : -1;
        float my_w = lane < topk ? (probs ? probs[t * topk + lane] : 1.0f) : 0.0f;
        for (int64_t c0 = 0; c0 < H8; c0 += 64 * 4) {
            float acc[4][8];
#pragma unroll
            for (int u = 0; u < 4; u++)
#pragma unroll
                for (int x = 0; x < 8; x++)
                    acc[u][x] = 0.0f;
            for (int k0 = 0; k0 < topk; k0 += 8) {
                uint4 v[8][4];
                int32_t rr[8];
                float ww[8];
#pragma unroll
                for (int kk = 0; kk < 8; kk++) {
                    int k = k0 + kk;
                    rr[kk] = __shfl(my_row, k < topk ? k : 63);
                    ww[kk] = __shfl(my_w, k < topk ? k : 63);
                    if (k >= topk)
                        rr[kk] = -1;
#pragma unroll
                    for (int u = 0; u < 4; u++) {
                        int64_t c = c0 + u * 64 + lane;
                        v[kk][u] = (rr[kk] >= 0 && c < H8)
                                       ? ld_stream16(y + (int64_t)rr[kk] * H + c * 8)
                                       : make_uint4(0, 0, 0, 0);
                    }
                }
#pragma unroll
                for (int kk = 0; kk < 8; kk++) {
                    if (rr[kk] < 0)
                        continue;
#pragma unroll
                    for (int u = 0; u < 4; u++) {
                        uint32_t w4[4] = {v[kk][u].x, v[kk][u].y, v[kk][u].z, v[kk][u].w};
#pragma unroll
                        for (int x = 0; x < 4; x++) {
                            acc[u][2 * x] = __builtin_fmaf(ww[kk], bf16lo(w4[x]), acc[u][2 * x]);
                            acc[u][2 * x + 1] = __builtin_fmaf(ww[kk], bf16hi(w4[x]), acc[u][2 * x + 1]);
                        }
                    }
                }
            }
#pragma unroll
            for (int u = 0; u < 4; u++) {
                int64_t c = c0 + u * 64 + lane;
                if (c < H8) {
                    uint4 o;
                    o.x = bf16_rne(acc[u][0]) | (bf16_rne(acc[u][1]) << 16);
                    o.y = bf16_rne(acc[u][2]) | (bf16_rne(acc[u][3]) << 16);
                    o.z = bf16_rne(acc[u][4]) | (bf16_rne(acc[u][5]) << 16);
                    o.w = bf16_rne(acc[u][6]) | (bf16_rne(acc[u][7]) << 16);
                    st_stream16(out + t * H + c * 8, o);
                }
            }
        }
    }
}

// ---------------------------------------------------------------------------
// SwiGLU + 1x128 quant.
// The exponential is the library's own fp32 function: Cody-Waite reduction
// x = n*ln2 + r with ln2 split in two (Cody & Waite 1980), the degree-7 Taylor
// polynomial of e^r (coefficients 1/j! rounded to fp32) in Horner form with
// fused multiply-adds, and scaling by 2^n.  The definition scales in two
// power-of-two steps, p * 2^(n/2) (exact: p is near 1 and |n/2| <= 75 keeps
// it normal in the range that is not clamped) and then * 2^(n - n/2), which
// rounds once; v_ldexp_f32 rounds p * 2^n once, so it gives the same value.
// Every step rounds once in fp32, so the result is reproducible bit for bit.
// ---------------------------------------------------------------------------
__device__ __forceinline__ float fgb_expf(float x)
{
    float n = __builtin_rintf(x * 0x1.715476p+0f);
    float r = __builtin_fmaf(-n, 0x1.62e4p-1f, x);
    r = __builtin_fmaf(-n, 0x1.7f7d1cp-20f, r);
    float p = 0x1.a01a02p-13f;
    p = __builtin_fmaf(p, r, 0x1.6c16c2p-10f);
    p = __builtin_fmaf(p, r, 0x1.111112p-7f);
    p = __builtin_fmaf(p, r, 0x1.555556p-5f);
    p = __builtin_fmaf(p, r, 0x1.555556p-3f);
    p = __builtin_fmaf(p, r, 0x1p-1f);
    p = __builtin_fmaf(p, r, 1.0f);
    p = __builtin_fmaf(p, r, 1.0f);
    float res = __builtin_amdgcn_ldexpf(p, (int)n);
    res = x > 0x1.62e43p+6f ? __builtin_inff() : res;
    res = x < -0x1.9fe36ap+6f ? 0.0f : res;
    return res;
}

// Correctly rounded 1/d for d in [1, 2^126): the hardware reciprocal
// (within 1 ulp) refined by two Newton steps with fused multiply-adds, whose
// remainders 1 - d*y are exact.
__device__ __forceinline__ float recip_rn(float d)
{
    float y = __builtin_amdgcn_rcpf(d);
    float r = __builtin_fmaf(-d, y, 1.0f);
    y = __builtin_fmaf(r, y, y);
    r = __builtin_fmaf(-d, y, 1.0f);
    return __builtin_fmaf(r, y, y);
}

// Correctly rounded g/d from y = RN(1/d): q = g*y is within an ulp of the
// quotient, its remainder g - q*d is exact, and one correction q + r*y rounds
// to RN(g/d) (Markstein's theorem); an exact q (r = 0, also a signed zero) is
// kept as it is.
__device__ __forceinline__ float div_rn(float g, float d, float y)
{
    const float q = g * y;
    const float r = __builtin_fmaf(-q, d, g);
    return r == 0.0f ? q : __builtin_fmaf(r, y, q);
}

// The SwiGLU forward and backward values of one element in fp32, each
// operation one rounding, in the order the C ABI declares; shared by the
// quantizing kernels and the fp32 diagnostic entry points.  The divisions
// by d = 1 + e are IEEE-exact: recip_rn / div_rn where d < 2^126 (1/d normal),
// the compiler's division otherwise (g < -87, rare; the branch is skipped
// when no lane of the wave needs it).  Both sides are checked bit for bit
// against the oracle's divisions for every input the kernels can see.
__device__ __forceinline__ float swiglu_elem(float g, float u)
{
    const float e = fgb_expf(-g);
    const float d = 1.0f + e;
    float s;
    if (d < 0x1p126f)
        s = div_rn(g, d, recip_rn(d));
    else
        s = g / d;
    return s * u;
}

__device__ __forceinline__ void dswiglu_elem(float g, float u, float a, float &du, float &dg)
{
    const float e = fgb_expf(-g);
    const float d = 1.0f + e;
    float sg, silu;
    if (d < 0x1p126f) {
        sg = recip_rn(d);
        silu = div_rn(g, d, sg);
    } else {
        sg = 1.0f / d;
        silu = g / d;
    }
    du = a * silu;
    const float dsilu = sg * (1.0f + g * (1.0f - sg));
    dg = (a * u) * dsilu;
}

// 1x128 quantization of the 8 values a lane holds, 16 lanes forming one
// group: returns the codes and the group's scale exponent.
__device__ __forceinline__ uint2 quant8_group16(const float (&v)[8], int &e)
{
    uint32_t m = 0;
#pragma unroll
    for (int k = 0; k < 8; k++)
        m = max(m, __float_as_uint(v[k]) & 0x7FFFFFFFu);
    m = group_max_u32<16>(m);
    e = scale_exp_from_bits(m, -22);
    const float sc = pow2f(-e);
    return make_uint2(cvt4_e4m3(v[0] * sc, v[1] * sc, v[2] * sc, v[3] * sc),
                      cvt4_e4m3(v[4] * sc, v[5] * sc, v[6] * sc, v[7] * sc));
}

// One wave per row; lane owns 8 gate and the matching 8 up values (16-byte
// loads); 16 lanes form one 128-element output group.  CACHE: the same pass
// also writes the 1x128 quantization of the input row [g | u] (the FP8 copy
// the backward recomputes the activation from).
constexpr int SW_U = 2; // 16-byte chunks of gate and of up in flight per lane (5% faster than 4)
template <bool CACHE>
__global__ __launch_bounds__(256) void swiglu_quant_kernel(const uint8_t *__restrict__ h, int64_t M,
                                                           int64_t F, int64_t ldh_bytes,
                                                           const int32_t *__restrict__ offs, int G,
                                                           uint8_t *__restrict__ q,
                                                           uint8_t *__restrict__ s,
                                                           uint8_t *__restrict__ hq,
                                                           uint8_t *__restrict__ hs)
{
    const int lane = lane_id();
    const int64_t rows = offs ? (int64_t)offs[G] : M;
    const int64_t F8 = F / 8;
    const int64_t wave = ((int64_t)blockIdx.x * blockDim.x + threadIdx.x) >> 6;
    const int64_t nwaves = ((int64_t)gridDim.x * blockDim.x) >> 6;
    for (int64_t r = wave; r < rows && r < M; r += nwaves) {
        const uint8_t *hr = h + r * ldh_bytes;
        for (int64_t c0 = 0; c0 < F8; c0 += 64 * SW_U) {
            uint4 gv[SW_U], uv[SW_U];
#pragma unroll
            for (int u = 0; u < SW_U; u++) {
                int64_t c = c0 + u * 64 + lane;
                gv[u] = c < F8 ? ld_stream16(hr + c * 16) : make_uint4(0, 0, 0, 0);
                uv[u] = c < F8 ? ld_stream16(hr + F * 2 + c * 16) : make_uint4(0, 0, 0, 0);
            }
#pragma unroll
            for (int u = 0; u < SW_U; u++) {
                int64_t c = c0 + u * 64 + lane;
                uint32_t gw[4] = {gv[u].x, gv[u].y, gv[u].z, gv[u].w};
                uint32_t uw[4] = {uv[u].x, uv[u].y, uv[u].z, uv[u].w};
                float a[8];
                uint32_t m = 0;
#pragma unroll
                for (int x = 0; x < 4; x++) {
                    a[2 * x] = swiglu_elem(bf16lo(gw[x]), bf16lo(uw[x]));
                    a[2 * x + 1] = swiglu_elem(bf16hi(gw[x]), bf16hi(uw[x]));
                    m = max(m, __float_as_uint(a[2 * x]) & 0x7FFFFFFFu);
                    m = max(m, __float_as_uint(a[2 * x + 1]) & 0x7FFFFFFFu);
                }
                m = group_max_u32<16>(m);
                int e = scale_exp_from_bits(m, -22);
                float sc = pow2f(-e);
                if (c < F8) {
                    uint2 o;
                    o.x = cvt4_e4m3(a[0] * sc, a[1] * sc, a[2] * sc, a[3] * sc);
                    o.y = cvt4_e4m3(a[4] * sc, a[5] * sc, a[6] * sc, a[7] * sc);
                    st_stream8(q + r * F + c * 8, o);
                    if ((lane & 15) == 0)
                        s[r * (F / 128) + c / 16] = (uint8_t)(e + 127);
                }
                if constexpr (CACHE) {
                    float gf[8], uf[8];
#pragma unroll
                    for (int x = 0; x < 4; x++) {
                        gf[2 * x] = bf16lo(gw[x]);
                        gf[2 * x + 1] = bf16hi(gw[x]);
                        uf[2 * x] = bf16lo(uw[x]);
                        uf[2 * x + 1] = bf16hi(uw[x]);
                    }
                    int eg, eu;
                    const uint2 og = quant8_group16(gf, eg), ou = quant8_group16(uf, eu);
                    if (c < F8) {
                        st_stream8(hq + r * 2 * F + c * 8, og);
                        st_stream8(hq + r * 2 * F + F + c * 8, ou);
                        if ((lane & 15) == 0) {
                            hs[r * (F / 64) + c / 16] = (uint8_t)(eg + 127);
                            hs[r * (F / 64) + F / 128 + c / 16] = (uint8_t)(eu + 127);
                        }
                    }
                }
            }
        }
    }
}

// SwiGLU backward + 1x128 quantization from the FP8-cached input.  One wave
// per row; lane owns 8 consecutive columns of g and u (8 code bytes each, one
// scale byte each) and of da (16 bytes of bf16); 16 lanes form one
// 128-element group of dg and of du.  The fp32 operations follow the
// definition in include/fgb.h one by one (no contraction).
constexpr int DS_U = 1; // column chunks per lane and pass (6% faster than 2)
__global__ __launch_bounds__(256) void dswiglu_quant_kernel(const uint8_t *__restrict__ hq,
                                                            const uint8_t *__restrict__ hs,
                                                            const uint16_t *__restrict__ da, int64_t M,
                                                            int64_t F, const int32_t *__restrict__ offs,
                                                            int G, uint8_t *__restrict__ dq,
                                                            uint8_t *__restrict__ ds)
{
    const int lane = lane_id();
    const int64_t rows = offs ? (int64_t)offs[G] : M;
    const int64_t F8 = F / 8, S = F / 64; // chunks of 8 per half-row, scale bytes per row
    const int64_t wave = ((int64_t)blockIdx.x * blockDim.x + threadIdx.x) >> 6;
    const int64_t nwaves = ((int64_t)gridDim.x * blockDim.x) >> 6;
    for (int64_t r = wave; r < rows && r < M; r += nwaves) {
        const uint8_t *hr = hq + r * 2 * F;
        for (int64_t c0 = 0; c0 < F8; c0 += 64 * DS_U) {
            uint2 gq[DS_U], uq[DS_U];
            uint4 av[DS_U];
            int eg[DS_U], eu[DS_U];
#pragma unroll
            for (int u = 0; u < DS_U; u++) {
                const int64_t c = c0 + u * 64 + lane;
                if (c < F8) {
                    gq[u] = *reinterpret_cast<const uint2 *>(hr + c * 8);
                    uq[u] = *reinterpret_cast<const uint2 *>(hr + F + c * 8);
                    av[u] = ld_stream16(da + r * F + c * 8);
                    eg[u] = (int)hs[r * S + c / 16] - 127;
                    eu[u] = (int)hs[r * S + F / 128 + c / 16] - 127;
                } else {
                    gq[u] = make_uint2(0, 0);
                    uq[u] = make_uint2(0, 0);
                    av[u] = make_uint4(0, 0, 0, 0);
                    eg[u] = eu[u] = 0;
                }
            }
#pragma unroll
            for (int u = 0; u < DS_U; u++) {
                const int64_t c = c0 + u * 64 + lane;
                const float fg = pow2f(eg[u]), fu = pow2f(eu[u]);
                const uint32_t gw[2] = {gq[u].x, gq[u].y}, uw[2] = {uq[u].x, uq[u].y};
                const uint32_t aw[4] = {av[u].x, av[u].y, av[u].z, av[u].w};
                float g[8], uu[8], a[8], dg[8], du[8];
                // decode x scale in one conversion per two codes (the scale
                // operand's exponent field is the power of two; exact)
#pragma unroll
                for (int k = 0; k < 2; k++) {
                    const fgb_f32x2 g0 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8((int)gw[k], fg, false);
                    const fgb_f32x2 g1 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8((int)gw[k], fg, true);
                    const fgb_f32x2 u0 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8((int)uw[k], fu, false);
                    const fgb_f32x2 u1 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8((int)uw[k], fu, true);
                    g[4 * k + 0] = g0.x; g[4 * k + 1] = g0.y; g[4 * k + 2] = g1.x; g[4 * k + 3] = g1.y;
                    uu[4 * k + 0] = u0.x; uu[4 * k + 1] = u0.y; uu[4 * k + 2] = u1.x; uu[4 * k + 3] = u1.y;
                }
#pragma unroll
                for (int k = 0; k < 4; k++) {
                    a[2 * k] = bf16lo(aw[k]);
                    a[2 * k + 1] = bf16hi(aw[k]);
                }
                uint32_t mg = 0, mu = 0;
#pragma unroll
                for (int k = 0; k < 8; k++) {
                    dswiglu_elem(g[k], uu[k], a[k], du[k], dg[k]);
                    mg = max(mg, __float_as_uint(dg[k]) & 0x7FFFFFFFu);
                    mu = max(mu, __float_as_uint(du[k]) & 0x7FFFFFFFu);
                }
                mg = group_max_u32<16>(mg);
                mu = group_max_u32<16>(mu);
                const int sgx = scale_exp_from_bits(mg, -22), sux = scale_exp_from_bits(mu, -22);
                const float scg = pow2f(-sgx), scu = pow2f(-sux);
                if (c < F8) {
                    st_stream8(dq + r * 2 * F + c * 8,
                               make_uint2(cvt4_e4m3(dg[0] * scg, dg[1] * scg, dg[2] * scg, dg[3] * scg),
                                          cvt4_e4m3(dg[4] * scg, dg[5] * scg, dg[6] * scg, dg[7] * scg)));
                    st_stream8(dq + r * 2 * F + F + c * 8,
                               make_uint2(cvt4_e4m3(du[0] * scu, du[1] * scu, du[2] * scu, du[3] * scu),
                                          cvt4_e4m3(du[4] * scu, du[5] * scu, du[6] * scu, du[7] * scu)));
                    if ((lane & 15) == 0) {
                        ds[r * S + c / 16] = (uint8_t)(sgx + 127);
                        ds[r * S + F / 128 + c / 16] = (uint8_t)(sux + 127);
                    }
                }
            }
        }
    }
}

// fp32 diagnostic forms: the element functions alone, one thread per element.
__global__ __launch_bounds__(256) void swiglu_f32_kernel(const float *__restrict__ g, const float *__restrict__ u,
                                                         int64_t n, float *__restrict__ a)
{
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x)
        a[i] = swiglu_elem(g[i], u[i]);
}

__global__ __launch_bounds__(256) void dswiglu_f32_kernel(const float *__restrict__ g, const float *__restrict__ u,
                                                          const float *__restrict__ da, int64_t n,
                                                          float *__restrict__ du, float *__restrict__ dg)
{
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x) {
        float x, y;
        dswiglu_elem(g[i], u[i], da[i], x, y);
        du[i] = x;
        dg[i] = y;
    }
}

// ---- backward of unpermute_unpad ------------------------------------------------
// dy[row_map[t,k]] = bf16(w[t,k] * dout[t]); rows no slot maps to are zero.
// Three passes: inverse map filled with -1, slot index scattered into it,
// then one wave per destination row gathers (or zeroes) its row.
__global__ __launch_bounds__(256) void ub_fill_kernel(int32_t *__restrict__ inv, int64_t n)
{
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x)
        inv[i] = -1;
}

__global__ __launch_bounds__(256) void ub_scatter_kernel(const int32_t *__restrict__ row_map, int64_t n,
                                                         int64_t M_cap, int32_t *__restrict__ inv)
{
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x) {
        const int32_t r = row_map[i];
        if (r >= 0 && r < M_cap)
            inv[r] = (int32_t)i;
    }
}

__global__ __launch_bounds__(256) void ub_gather_kernel(const uint16_t *__restrict__ dout,
                                                        const int32_t *__restrict__ inv,
                                                        const float *__restrict__ probs, int topk, int64_t H,
                                                        int64_t M_cap, uint16_t *__restrict__ dy)
{
    const int lane = lane_id();
    const int64_t H8 = H / 8;
    const int64_t wave = ((int64_t)blockIdx.x * blockDim.x + threadIdx.x) >> 6;
    const int64_t nwaves = ((int64_t)gridDim.x * blockDim.x) >> 6;
    for (int64_t r = wave; r < M_cap; r += nwaves) {
        const int32_t si = inv[r];
        uint16_t *dst = dy + r * H;
        if (si < 0) {
            for (int64_t c = lane; c < H8; c += 64)
                st_stream16(dst + c * 8, make_uint4(0, 0, 0, 0));
            continue;
        }
        const float w = probs ? probs[si] : 1.0f;
        const uint16_t *src = dout + (int64_t)(si / topk) * H;
        for (int64_t c0 = 0; c0 < H8; c0 += 64 * 4) {
            uint4 v[4];
#pragma unroll
            for (int u = 0; u < 4; u++) {
                const int64_t c = c0 + u * 64 + lane;
                v[u] = c < H8 ? *reinterpret_cast<const uint4 *>(src + c * 8) : make_uint4(0, 0, 0, 0);
            }
#pragma unroll
            for (int u = 0; u < 4; u++) {
                const int64_t c = c0 + u * 64 + lane;
                if (c < H8) {
                    const uint32_t x4[4] = {v[u].x, v[u].y, v[u].z, v[u].w};
                    uint32_t o[4];
#pragma unroll
                    for (int k = 0; k < 4; k++)
                        o[k] = bf16_rne(w * bf16lo(x4[k])) | (bf16_rne(w * bf16hi(x4[k])) << 16);
                    st_stream16(dst + c * 8, make_uint4(o[0], o[1], o[2], o[3]));
                }
            }
        }
    }
}

// unpermute_backward fused with 1x128 quantization, token-major: a wave takes token t, keeps its dO row
// chunks in registers (the row is read once, not once per slot) and, for
// each of the token's slots, writes the probs-weighted, bf16-rounded,
// 1x128-quantized copy into the slot's row of the padded layout.  Work
// items past the T tokens are rows; those no slot references (inv < 0) get
// code 0 / scale 105, as a zero row quantizes.  Per slot: the product w * x
// rounded to bf16 (v_cvt_pk_bf16_f32, round to nearest even: the value the
// unfused unpermute_backward writes), then quantized.
typedef __bf16 fgb_bf2 __attribute__((ext_vector_type(2)));
typedef float fgb_f2 __attribute__((ext_vector_type(2)));
constexpr int UBT_U = 2;
__global__ __launch_bounds__(256) void ub_token_quant_kernel(const uint16_t *__restrict__ dout,
                                                             const int32_t *__restrict__ row_map,
                                                             const float *__restrict__ probs,
                                                             const int32_t *__restrict__ inv, int64_t T, int topk,
                                                             int64_t H, int64_t M_cap, uint8_t *__restrict__ q,
                                                             uint8_t *__restrict__ s)
{
    const int lane = lane_id();
    const int64_t H8 = H / 8;
    const int64_t wave = ((int64_t)blockIdx.x * blockDim.x + threadIdx.x) >> 6;
    const int64_t nwaves = ((int64_t)gridDim.x * blockDim.x) >> 6;
    for (int64_t it = wave; it < T + M_cap; it += nwaves) {
        if (it >= T) {
            const int64_t r = it - T;
            if (inv[r] >= 0)
                continue;
            uint8_t *dq = q + r * H;
            for (int64_t c = lane; c < H / 16; c += 64)
                st_stream16(dq + c * 16, make_uint4(0, 0, 0, 0));
            for (int64_t c = lane; c < H / 128; c += 64)
                s[r * (H / 128) + c] = 105;
            continue;
        }
        const int64_t t = it;
        // lane k < topk holds slot k's row and weight
        int32_t rv = -1;
        float wv = 0.0f;
        if (lane < topk) {
            rv = row_map[t * topk + lane];
            wv = probs ? probs[t * topk + lane] : 1.0f;
        }
        const uint16_t *src = dout + t * H;
        for (int64_t c0 = 0; c0 < H8; c0 += 64 * UBT_U) {
            float x[UBT_U][8];
            uint32_t ax[UBT_U]; // |x| maximum of each 128-group (bits), over the group's 16 lanes
#pragma unroll
            for (int u = 0; u < UBT_U; u++) {
                const int64_t c = c0 + u * 64 + lane;
                const uint4 v = c < H8 ? ld_stream16(src + c * 8) : make_uint4(0, 0, 0, 0);
                const uint32_t x4[4] = {v.x, v.y, v.z, v.w};
                uint32_t m = 0;
#pragma unroll
                for (int k = 0; k < 4; k++) {
                    x[u][2 * k] = bf16lo(x4[k]);
                    x[u][2 * k + 1] = bf16hi(x4[k]);
                    m = max(m, max(__float_as_uint(x[u][2 * k]) & 0x7FFFFFFFu,
                                   __float_as_uint(x[u][2 * k + 1]) & 0x7FFFFFFFu));
                }
                ax[u] = group_max_u32<16>(m);
            }
            for (int k = 0; k < topk; k++) {
                const int32_t r = __builtin_amdgcn_readlane(rv, k);
                if (r < 0 || r >= M_cap)
                    continue; // dropped slot (uniform)
                const float w = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, wv), k));
                uint8_t *dq = q + (int64_t)r * H;
                uint8_t *dsc = s + (int64_t)r * (H / 128);
#pragma unroll
                for (int u = 0; u < UBT_U; u++) {
                    const int64_t c = c0 + u * 64 + lane;
                    float y[8];
#pragma unroll
                    for (int j = 0; j < 4; j++) {
                        const fgb_f2 pr = {w * x[u][2 * j], w * x[u][2 * j + 1]};
                        const uint32_t b = __builtin_bit_cast(uint32_t, __builtin_convertvector(pr, fgb_bf2));
                        y[2 * j] = bf16lo(b);
                        y[2 * j + 1] = bf16hi(b);
                    }
                    // The group's amax of y = bf16(w * x) is bf16(|w| * amax|x|): the fp32
                    // product and the bf16 rounding are monotonic in |x|, so the
                    // per-slot group reduction is not needed.
                    const float am = bf16lo(pack_bf16x2(fabsf(w) * __uint_as_float(ax[u]), 0.0f));
                    const int e = scale_exp_from_bits(__float_as_uint(am), -22);
                    const float sc = pow2f(-e);
                    const uint2 o = make_uint2(cvt4_e4m3(y[0] * sc, y[1] * sc, y[2] * sc, y[3] * sc),
                                               cvt4_e4m3(y[4] * sc, y[5] * sc, y[6] * sc, y[7] * sc));
                    if (c < H8) {
                        st_stream8(dq + c * 8, o);
                        if ((lane & 15) == 0)
                            dsc[c / 16] = (uint8_t)(e + 127);
                    }
                }
            }
        }
    }
}

// Validation and launches of permute_pad, with the workspace already chosen
// (the caller's, or the no-allocation variant's scratch array).
static int permute_pad_check(const char *name, const uint8_t *xq, const uint8_t *xs, const int32_t *topk_idx,
                             int64_t T, int topk, int G, int64_t H, int pad_multiple, const uint8_t *out_q,
                             const uint8_t *out_s, const int32_t *row_map, const int32_t *group_offsets,
                             int64_t M_cap)
{
    FGB_REQUIRE(xq && xs && topk_idx && out_q && out_s && row_map && group_offsets, FGB_EINVAL,
                "%s: null pointer", name);
    FGB_REQUIRE(T >= 0 && topk >= 1 && topk <= 64 && G >= 1 && G <= 1024, FGB_EINVAL,
                "%s: need T >= 0, 1 <= topk <= 64, 1 <= G <= 1024", name);
    FGB_REQUIRE(H > 0 && H % 128 == 0, FGB_EINVAL, "%s: H must be a positive multiple of 128", name);
    FGB_REQUIRE(pad_multiple >= 1 && pad_multiple <= 256, FGB_EINVAL, "%s: pad_multiple must be in [1, 256]", name);
    FGB_REQUIRE(M_cap >= T * topk + (int64_t)(pad_multiple - 1) * G, FGB_EINVAL,
                "%s: M_cap must be >= T*topk + (pad_multiple-1)*G", name);
    FGB_REQUIRE(M_cap < (1ll << 31), FGB_EINVAL, "%s: M_cap must fit in int32", name);
    FGB_REQUIRE(aligned16(xq) && aligned16(out_q), FGB_EINVAL, "%s: xq and out_q must be 16-byte aligned", name);
    return FGB_OK;
}

static int permute_pad_launch(const uint8_t *xq, const uint8_t *xs, const int32_t *topk_idx, int64_t T, int topk,
                              int G, int64_t H, int pad_multiple, uint8_t *out_q, uint8_t *out_s, int32_t *row_map,
                              int32_t *group_offsets, int64_t M_cap, void *workspace, hipStream_t st)
{
    PPWorkspace w = pp_carve(workspace, T, G);
    int nchunks = (int)pp_nchunks(T);
    if (nchunks > 0) {
        pp_count_kernel<<<nchunks, 256, G * sizeof(int32_t), st>>>(topk_idx, T, topk, G, w.cnt);
        FGB_LAUNCHED("permute_pad/count");
    }
    pp_scan_kernel<<<1, 256, (2 * G + 1 + 256) * sizeof(int32_t), st>>>(w.cnt, nchunks, G, pad_multiple,
                                                                 w.base, w.total, group_offsets);
    FGB_LAUNCHED("permute_pad/scan");
    if (nchunks > 0) {
        pp_rowmap_kernel<<<nchunks, 256, 5 * G * sizeof(int32_t), st>>>(topk_idx, T, topk, G, w.base, row_map);
        FGB_LAUNCHED("permute_pad/rowmap");
    }
    int64_t tok_blocks = (T + 3) / 4;
    int64_t pad_blocks = ((int64_t)(pad_multiple - 1) * G + 3) / 4;
    int64_t grid = tok_blocks + pad_blocks;
    if (grid > 0) {
        pp_copy_kernel<<<(unsigned)grid, 256, 0, st>>>(xq, xs, row_map, T, topk, G, H, pad_multiple,
                                                      w.total, group_offsets, out_q, out_s, tok_blocks, M_cap);
        FGB_LAUNCHED("permute_pad/copy");
    }
    return FGB_OK;
}

// ---- the no-allocation variant's scratch array ------------------------------
// One copy per GPU, alive until the process ends.  The host never passes the
// array's name to a kernel (in host code it is only a stand-in for the
// symbol): the device address of each GPU's copy is looked up once per
// device with hipGetSymbolAddress, with that device current, and kept here.
static __device__ __align__(256) int32_t scratch[FGB_PERMUTE_PAD_NOALLOC_SCRATCH_BYTES / sizeof(int32_t)];

constexpr int PP_MAX_DEVICES = 64;
static std::mutex g_scratch_mu;
static void *g_scratch_ptr[PP_MAX_DEVICES];

// The current device's copy of `scratch` (looked up on the first call made
// with that device current).
static int scratch_for_current_device(void **out)
{
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess)
        return set_error(FGB_EHIP, "permute_pad_noalloc: hipGetDevice failed: %s", hipGetErrorString(e));
    if (dev < 0 || dev >= PP_MAX_DEVICES)
        return set_error(FGB_EUNSUPPORTED, "permute_pad_noalloc: device %d beyond the %d supported", dev,
                         PP_MAX_DEVICES);
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void *p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess || !p)
            return set_error(FGB_EHIP, "permute_pad_noalloc: hipGetSymbolAddress failed: %s", hipGetErrorString(e));
        g_scratch_ptr[dev] = p;
    }
    *out = g_scratch_ptr[dev];
    return FGB_OK;
}

} // namespace fgb

using namespace fgb;

extern "C" int permute_pad(const uint8_t *xq, const uint8_t *xs, const int32_t *topk_idx,
                           int64_t T, int topk, int G, int64_t H, int pad_multiple,
                           uint8_t *out_q, uint8_t *out_s, int32_t *row_map,
                           int32_t *group_offsets, int64_t M_cap, void *workspace,
                           size_t ws_bytes, void *stream)
{
    clear_error();
    int rc = permute_pad_check("permute_pad", xq, xs, topk_idx, T, topk, G, H, pad_multiple, out_q, out_s, row_map,
                               group_offsets, M_cap);
    if (rc != FGB_OK)
        return rc;
    size_t need = permute_pad_workspace_size(T, topk, G);
    FGB_REQUIRE(workspace && ws_bytes >= need, FGB_EWORKSPACE,
                "permute_pad: workspace of %zu bytes required", need);
    return permute_pad_launch(xq, xs, topk_idx, T, topk, G, H, pad_multiple, out_q, out_s, row_map, group_offsets,
                              M_cap, workspace, (hipStream_t)stream);
}

extern "C" int permute_pad_noalloc(const uint8_t *xq, const uint8_t *xs, const int32_t *topk_idx, int64_t T,
                                   int topk, int G, int64_t H, int pad_multiple, uint8_t *out_q, uint8_t *out_s,
                                   int32_t *row_map, int32_t *group_offsets, int64_t M_cap, void *stream)
{
    clear_error();
    int rc = permute_pad_check("permute_pad_noalloc", xq, xs, topk_idx, T, topk, G, H, pad_multiple, out_q, out_s,
                               row_map, group_offsets, M_cap);
    if (rc != FGB_OK)
        return rc;
    const size_t need = permute_pad_workspace_size(T, topk, G);
    FGB_REQUIRE(need <= (size_t)FGB_PERMUTE_PAD_NOALLOC_SCRATCH_BYTES, FGB_EWORKSPACE,
                "permute_pad_noalloc: these sizes need %zu bytes of scratch, more than the %d bytes it holds "
                "(2*ceil(T/256)*G + G int32 words); call permute_pad with a workspace instead",
                need, (int)FGB_PERMUTE_PAD_NOALLOC_SCRATCH_BYTES);
    void *ws = nullptr;
    rc = scratch_for_current_device(&ws);
    if (rc != FGB_OK)
        return rc;
    return permute_pad_launch(xq, xs, topk_idx, T, topk, G, H, pad_multiple, out_q, out_s, row_map, group_offsets,
                              M_cap, ws, (hipStream_t)stream);
}

extern "C" size_t permute_pad_workspace_size(int64_t T, int topk, int G)
{
    (void)topk;
    if (T < 0 || G < 1)
        return 0;
    return (2 * pp_nchunks(T) * (size_t)G + (size_t)G) * sizeof(int32_t);
}

extern "C" int unpermute_unpad(const void *y, const int32_t *row_map, const float *probs,
                               int64_t T, int topk, int64_t H, void *out, void *stream)
{
    clear_error();
    FGB_REQUIRE(y && row_map && out, FGB_EINVAL, "unpermute_unpad: null pointer");
    FGB_REQUIRE(T >= 0 && topk >= 1 && topk <= 64, FGB_EINVAL, "unpermute_unpad: need 1 <= topk <= 64");
    FGB_REQUIRE(H > 0 && H % 8 == 0, FGB_EINVAL, "unpermute_unpad: H must be a positive multiple of 8");
    FGB_REQUIRE(aligned16(y) && aligned16(out), FGB_EINVAL, "unpermute_unpad: y and out must be 16-byte aligned");
    if (T == 0)
        return FGB_OK;
    int64_t grid = (T + 3) / 4;
    grid = grid < 8192 ? grid : 8192;
    unpermute_kernel<<<(unsigned)grid, 256, 0, (hipStream_t)stream>>>((const uint16_t *)y, row_map, probs,
                                                                      T, topk, H, (uint16_t *)out);
    FGB_LAUNCHED("unpermute_unpad");
    return FGB_OK;
}

extern "C" int swiglu_quant(const void *h, int64_t M, int64_t F, int64_t ldh,
                            const int32_t *group_offsets, int G, uint8_t *q, uint8_t *s,
                            void *stream)
{
    clear_error();
    FGB_REQUIRE(h && q && s, FGB_EINVAL, "swiglu_quant: null pointer");
    FGB_REQUIRE(M >= 0 && F > 0 && F % 128 == 0, FGB_EINVAL, "swiglu_quant: F must be a positive multiple of 128");
    FGB_REQUIRE(ldh >= 2 * F && ldh % 8 == 0, FGB_EINVAL, "swiglu_quant: ldh must be >= 2F and a multiple of 8");
    FGB_REQUIRE(!group_offsets || G >= 1, FGB_EINVAL, "swiglu_quant: G must be >= 1 with group_offsets");
    FGB_REQUIRE(aligned16(h) && aligned16(q), FGB_EINVAL, "swiglu_quant: h and q must be 16-byte aligned");
    if (M == 0)
        return FGB_OK;
    int64_t grid = (M + 3) / 4;
    grid = grid < 16384 ? grid : 16384;
    swiglu_quant_kernel<false><<<(unsigned)grid, 256, 0, (hipStream_t)stream>>>((const uint8_t *)h, M, F, ldh * 2,
                                                                                group_offsets, G, q, s, nullptr,
                                                                                nullptr);
    FGB_LAUNCHED("swiglu_quant");
    return FGB_OK;
}

extern "C" int swiglu_quant_cache(const void *h, int64_t M, int64_t F, int64_t ldh,
                                  const int32_t *group_offsets, int G, uint8_t *q, uint8_t *s,
                                  uint8_t *hq, uint8_t *hs, void *stream)
{
    clear_error();
    FGB_REQUIRE(h && q && s && hq && hs, FGB_EINVAL, "swiglu_quant_cache: null pointer");
    FGB_REQUIRE(M >= 0 && F > 0 && F % 128 == 0, FGB_EINVAL,
                "swiglu_quant_cache: F must be a positive multiple of 128");
    FGB_REQUIRE(ldh >= 2 * F && ldh % 8 == 0, FGB_EINVAL,
                "swiglu_quant_cache: ldh must be >= 2F and a multiple of 8");
    FGB_REQUIRE(!group_offsets || G >= 1, FGB_EINVAL, "swiglu_quant_cache: G must be >= 1 with group_offsets");
    FGB_REQUIRE(aligned16(h) && aligned16(q) && aligned16(hq), FGB_EINVAL,
                "swiglu_quant_cache: h, q and hq must be 16-byte aligned");
    if (M == 0)
        return FGB_OK;
    int64_t grid = (M + 3) / 4;
    grid = grid < 16384 ? grid : 16384;
    swiglu_quant_kernel<true><<<(unsigned)grid, 256, 0, (hipStream_t)stream>>>((const uint8_t *)h, M, F, ldh * 2,
                                                                               group_offsets, G, q, s, hq, hs);
    FGB_LAUNCHED("swiglu_quant_cache");
    return FGB_OK;
}

extern "C" int dswiglu_quant(const uint8_t *hq, const uint8_t *hs, const void *da, int64_t M, int64_t F,
                             const int32_t *group_offsets, int G, uint8_t *dq, uint8_t *ds, void *stream)
{
    clear_error();
    FGB_REQUIRE(hq && hs && da && dq && ds, FGB_EINVAL, "dswiglu_quant: null pointer");
    FGB_REQUIRE(M >= 0 && F > 0 && F % 128 == 0, FGB_EINVAL, "dswiglu_quant: F must be a positive multiple of 128");
    FGB_REQUIRE(!group_offsets || G >= 1, FGB_EINVAL, "dswiglu_quant: G must be >= 1 with group_offsets");
    FGB_REQUIRE(aligned16(da) && ((uintptr_t)hq & 7) == 0 && ((uintptr_t)dq & 7) == 0, FGB_EINVAL,
                "dswiglu_quant: da must be 16-byte and hq, dq 8-byte aligned");
    if (M == 0)
        return FGB_OK;
    int64_t grid = (M + 3) / 4;
    grid = grid < 16384 ? grid : 16384;
    dswiglu_quant_kernel<<<(unsigned)grid, 256, 0, (hipStream_t)stream>>>(hq, hs, (const uint16_t *)da, M, F,
                                                                          group_offsets, G, dq, ds);
    FGB_LAUNCHED("dswiglu_quant");
    return FGB_OK;
}

extern "C" size_t unpermute_backward_workspace_size(int64_t M_cap)
{
    return M_cap > 0 ? (size_t)(4 * M_cap) : 0;
}

extern "C" int unpermute_backward(const void *dout, const int32_t *row_map, const float *probs, int64_t T,
                                  int topk, int64_t H, int64_t M_cap, void *dy, void *workspace, size_t ws_bytes,
                                  void *stream)
{
    clear_error();
    FGB_REQUIRE(dout && row_map && dy, FGB_EINVAL, "unpermute_backward: null pointer");
    FGB_REQUIRE(T >= 0 && topk >= 1 && topk <= 64 && H > 0 && H % 8 == 0 && M_cap >= 0, FGB_EINVAL,
                "unpermute_backward: need topk in [1, 64] and H a positive multiple of 8");
    FGB_REQUIRE(T * topk < (1ll << 31) && M_cap < (1ll << 31), FGB_EINVAL, "unpermute_backward: too many rows");
    FGB_REQUIRE(aligned16(dout) && aligned16(dy), FGB_EINVAL, "unpermute_backward: dout and dy must be 16-byte aligned");
    if (M_cap == 0)
        return FGB_OK;
    FGB_REQUIRE(workspace && ws_bytes >= unpermute_backward_workspace_size(M_cap), FGB_EWORKSPACE,
                "unpermute_backward: workspace must hold %zu bytes", unpermute_backward_workspace_size(M_cap));
    hipStream_t st = (hipStream_t)stream;
    int32_t *inv = (int32_t *)workspace;
    int64_t g1 = (M_cap + 255) / 256;
    ub_fill_kernel<<<(unsigned)(g1 < 4096 ? g1 : 4096), 256, 0, st>>>(inv, M_cap);
    FGB_LAUNCHED("unpermute_backward");
    if (T > 0) {
        int64_t g2 = (T * topk + 255) / 256;
        ub_scatter_kernel<<<(unsigned)(g2 < 4096 ? g2 : 4096), 256, 0, st>>>(row_map, T * topk, M_cap, inv);
        FGB_LAUNCHED("unpermute_backward");
    }
    int64_t g3 = (M_cap + 3) / 4;
    ub_gather_kernel<<<(unsigned)(g3 < 16384 ? g3 : 16384), 256, 0, st>>>((const uint16_t *)dout, inv, probs, topk,
                                                                           H, M_cap, (uint16_t *)dy);
    FGB_LAUNCHED("unpermute_backward");
    return FGB_OK;
}

extern "C" int unpermute_backward_quant(const void *dout, const int32_t *row_map, const float *probs, int64_t T,
                                        int topk, int64_t H, int64_t M_cap, uint8_t *q, uint8_t *s,
                                        void *workspace, size_t ws_bytes, void *stream)
{
    clear_error();
    FGB_REQUIRE(dout && row_map && q && s, FGB_EINVAL, "unpermute_backward_quant: null pointer");
    FGB_REQUIRE(T >= 0 && topk >= 1 && topk <= 64 && H > 0 && H % 128 == 0 && M_cap >= 0, FGB_EINVAL,
                "unpermute_backward_quant: need topk in [1, 64] and H a positive multiple of 128");
    FGB_REQUIRE(T * topk < (1ll << 31) && M_cap < (1ll << 31), FGB_EINVAL,
                "unpermute_backward_quant: too many rows");
    FGB_REQUIRE(aligned16(dout) && aligned16(q), FGB_EINVAL,
                "unpermute_backward_quant: dout and q must be 16-byte aligned");
    if (M_cap == 0)
        return FGB_OK;
    FGB_REQUIRE(workspace && ws_bytes >= unpermute_backward_workspace_size(M_cap), FGB_EWORKSPACE,
                "unpermute_backward_quant: workspace must hold %zu bytes",
                unpermute_backward_workspace_size(M_cap));
    hipStream_t st = (hipStream_t)stream;
    int32_t *inv = (int32_t *)workspace;
    int64_t g1 = (M_cap + 255) / 256;
    ub_fill_kernel<<<(unsigned)(g1 < 4096 ? g1 : 4096), 256, 0, st>>>(inv, M_cap);
    FGB_LAUNCHED("unpermute_backward_quant");
    if (T > 0) {
        int64_t g2 = (T * topk + 255) / 256;
        ub_scatter_kernel<<<(unsigned)(g2 < 4096 ? g2 : 4096), 256, 0, st>>>(row_map, T * topk, M_cap, inv);
        FGB_LAUNCHED("unpermute_backward_quant");
    }
    int64_t g3 = (T + M_cap + 3) / 4;
    ub_token_quant_kernel<<<(unsigned)(g3 < 16384 ? g3 : 16384), 256, 0, st>>>(
        (const uint16_t *)dout, row_map, probs, inv, T, topk, H, M_cap, q, s);
    FGB_LAUNCHED("unpermute_backward_quant");
    return FGB_OK;
}

extern "C" int swiglu_f32(const float *g, const float *u, int64_t n, float *a, void *stream)
{
    clear_error();
    FGB_REQUIRE(n >= 0, FGB_EINVAL, "swiglu_f32: n must be >= 0");
    if (n == 0)
        return FGB_OK;
    FGB_REQUIRE(g && u && a, FGB_EINVAL, "swiglu_f32: null pointer");
    const int64_t grid = min((n + 255) / 256, (int64_t)65536);
    swiglu_f32_kernel<<<(unsigned)grid, 256, 0, (hipStream_t)stream>>>(g, u, n, a);
    FGB_LAUNCHED("swiglu_f32");
    return FGB_OK;
}

extern "C" int dswiglu_f32(const float *g, const float *u, const float *da, int64_t n, float *du, float *dg,
                           void *stream)
{
    clear_error();
    FGB_REQUIRE(n >= 0, FGB_EINVAL, "dswiglu_f32: n must be >= 0");
    if (n == 0)
        return FGB_OK;
    FGB_REQUIRE(g && u && da && du && dg, FGB_EINVAL, "dswiglu_f32: null pointer");
    const int64_t grid = min((n + 255) / 256, (int64_t)65536);
    dswiglu_f32_kernel<<<(unsigned)grid, 256, 0, (hipStream_t)stream>>>(g, u, da, n, du, dg);
    FGB_LAUNCHED("dswiglu_f32");
    return FGB_OK;
}
