// probe.hip -- reference access patterns on plain bytes, for calibrating the
// bandwidth of the data-movement kernels (no part of the method's arithmetic).
//
// Each pattern moves bytes with the same 16-byte nontemporal loads and stores
// the library's kernels use, one 16-byte chunk per lane, with nothing but the
// copy in between:
//   COPY           dst = src, both sides contiguous;
//   READ           16 bytes per 4 KB of src written (the XOR of the 4 KB);
//   FILL           dst = 0;
//   STRIDED_READ   [rows, cols] read by 128x128 blocks as the transposes read
//                  them (8 lanes per 128-byte row piece, 16 rows per lane),
//                  each block written as 16 contiguous KB (block b at b*16 KB);
//   STRIDED_WRITE  the reverse: contiguous 16 KB blocks read, written into
//                  the [rows, cols] layout by 128-byte row pieces.
// A kernel whose bytes follow one of these patterns cannot beat it; the
// bench reports them beside the kernels' rates.
#include "fgb_internal.h"

namespace fgb {

__global__ __launch_bounds__(256) void probe_copy_kernel(const uint8_t *__restrict__ s, uint8_t *__restrict__ d,
                                                         int64_t n16)
{
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i < n16)
        st_stream16(d + i * 16, ld_stream16(s + i * 16));
}

__global__ __launch_bounds__(256) void probe_fill_kernel(uint8_t *__restrict__ d, int64_t n16)
{
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i < n16)
        st_stream16(d + i * 16, make_uint4(0, 0, 0, 0));
}

// One wave per 4 KB: four 16-byte loads per lane, XOR-reduced over the wave.
__global__ __launch_bounds__(256) void probe_read_kernel(const uint8_t *__restrict__ s, uint8_t *__restrict__ d,
                                                         int64_t nblk)
{
    const int lane = lane_id();
    const int64_t b = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    if (b >= nblk)
        return;
    uint4 x = make_uint4(0, 0, 0, 0);
#pragma unroll
    for (int k = 0; k < 4; k++) {
        const uint4 v = ld_stream16(s + b * 4096 + k * 1024 + lane * 16);
        x.x ^= v.x;
        x.y ^= v.y;
        x.z ^= v.z;
        x.w ^= v.w;
    }
#pragma unroll
    for (int m = 1; m < 64; m <<= 1) {
        x.x ^= __shfl_xor(x.x, m);
        x.y ^= __shfl_xor(x.y, m);
        x.z ^= __shfl_xor(x.z, m);
        x.w ^= __shfl_xor(x.w, m);
    }
    if (lane == 0)
        st_stream16(d + b * 16, x);
}

// One wave per 128x128 block b = tb + ntb * cb (row blocks fastest).
template <bool STRIDED_IN>
__global__ __launch_bounds__(256) void probe_strided_kernel(const uint8_t *__restrict__ s, uint8_t *__restrict__ d,
                                                            int64_t rows, int64_t cols, int64_t nblk)
{
    const int lane = lane_id();
    const int64_t b = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    if (b >= nblk)
        return;
    const int64_t ntb = rows / 128, tb = b % ntb, cb = b / ntb;
    const int tsub = lane & 7, csub = lane >> 3;
    const int64_t piece = (tb * 128 + tsub * 16) * cols + cb * 128 + csub * 16; // row j adds j * cols
    const int64_t flat = b * 16384 + lane * 16;                                  // row j adds j * 1024
    uint4 v[16];
#pragma unroll
    for (int j = 0; j < 16; j++)
        v[j] = ld_stream16(s + (STRIDED_IN ? piece + j * cols : flat + j * 1024));
#pragma unroll
    for (int j = 0; j < 16; j++)
        st_stream16(d + (STRIDED_IN ? flat + j * 1024 : piece + j * cols), v[j]);
}

} // namespace fgb

using namespace fgb;

extern "C" int fgb_hbm_probe(const void *src, void *dst, int64_t rows, int64_t cols, int pattern, void *stream)
{
    clear_error();
    FGB_REQUIRE(pattern >= FGB_PROBE_COPY && pattern <= FGB_PROBE_STRIDED_WRITE, FGB_EUNSUPPORTED,
                "fgb_hbm_probe: unknown pattern %d", pattern);
    FGB_REQUIRE(dst && (src || pattern == FGB_PROBE_FILL), FGB_EINVAL, "fgb_hbm_probe: null pointer");
    FGB_REQUIRE(aligned16(dst) && (!src || aligned16(src)), FGB_EINVAL,
                "fgb_hbm_probe: src and dst must be 16-byte aligned");
    FGB_REQUIRE(rows >= 0 && cols >= 0 && rows % 128 == 0 && cols % 128 == 0, FGB_EINVAL,
                "fgb_hbm_probe: rows and cols must be multiples of 128 (rows=%lld cols=%lld)", (long long)rows,
                (long long)cols);
    const int64_t n = rows * cols;
    if (n == 0)
        return FGB_OK;
    hipStream_t stm = (hipStream_t)stream;
    const char *name = "fgb_hbm_probe";
    switch (pattern) {
    case FGB_PROBE_COPY:
    case FGB_PROBE_FILL: {
        const int64_t n16 = n / 16, grid = (n16 + 255) / 256;
        FGB_REQUIRE(grid < (1ll << 31), FGB_EINVAL, "fgb_hbm_probe: too large");
        if (pattern == FGB_PROBE_COPY)
            probe_copy_kernel<<<(unsigned)grid, 256, 0, stm>>>((const uint8_t *)src, (uint8_t *)dst, n16);
        else
            probe_fill_kernel<<<(unsigned)grid, 256, 0, stm>>>((uint8_t *)dst, n16);
        break;
    }
    case FGB_PROBE_READ: {
        const int64_t nblk = n / 4096, grid = (nblk + 3) / 4;
        FGB_REQUIRE(grid < (1ll << 31), FGB_EINVAL, "fgb_hbm_probe: too large");
        probe_read_kernel<<<(unsigned)grid, 256, 0, stm>>>((const uint8_t *)src, (uint8_t *)dst, nblk);
        break;
    }
    default: {
        const int64_t nblk = n / 16384, grid = (nblk + 3) / 4;
        FGB_REQUIRE(grid < (1ll << 31), FGB_EINVAL, "fgb_hbm_probe: too large");
        if (pattern == FGB_PROBE_STRIDED_READ)
            probe_strided_kernel<true><<<(unsigned)grid, 256, 0, stm>>>((const uint8_t *)src, (uint8_t *)dst, rows,
                                                                        cols, nblk);
        else
            probe_strided_kernel<false><<<(unsigned)grid, 256, 0, stm>>>((const uint8_t *)src, (uint8_t *)dst, rows,
                                                                         cols, nblk);
    }
    }
    FGB_LAUNCHED(name);
    return FGB_OK;
}
