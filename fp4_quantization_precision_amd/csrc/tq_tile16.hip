// tq_tile16.hip - 16x16-tile scaling: quantize and exact transpose (gfx950).
//
// [TML] "싱킹 머신스 랩, 4비트 학습 기법 공개", forward/backward-mismatch
// paragraph: the alternative to requantizing after a transpose gives one scale
// to a 16 x 16 tile (256 values), so a transpose moves codes and scales without
// changing any value; its cost is that one large value can zero the rest of
// its tile.  Arithmetic as the block-16 quantizer with the block maximum taken
// over the tile; layouts in include/tq.h.
//
// Quantize: a wave covers four horizontally adjacent tiles (64 columns x 16
// rows).  Lane 16 t + j loads row j of tile t (16 values; the four lanes of one
// row read 128 contiguous bytes of bf16), takes its row maximum, and the 16
// lanes of a tile reduce it with cross-lane exchanges; each lane then writes
// its row's 8 code bytes and lane 0 the tile's scale byte.
//
// Transpose: a workgroup moves a 64 x 64 region (4 x 4 tiles) through LDS: 32
// code bytes per input row in, 32 per output row out, and the 16 tile scales.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "tq_device.hpp"
#include "tq_kernels.hpp"

namespace tq {

constexpr int kT16Threads = 256;

template <bool BF16>
__device__ __forceinline__ void load_row16(const void* __restrict__ x, int64_t elem, float v[16])
{
    if (BF16) {
        const uint4* p = reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(x) + elem);
        const uint4 a = p[0], b = p[1];
        const uint32_t w[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            v[2 * i] = bf16_lo(w[i]);
            v[2 * i + 1] = bf16_hi(w[i]);
        }
    } else {
        const float4* p = reinterpret_cast<const float4*>(static_cast<const float*>(x) + elem);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const float4 q = p[i];
            v[4 * i] = q.x;
            v[4 * i + 1] = q.y;
            v[4 * i + 2] = q.z;
            v[4 * i + 3] = q.w;
        }
    }
}

template <bool BF16>
__global__ __launch_bounds__(kT16Threads) void quantize_tile16_kernel(
    const void* __restrict__ x, int64_t batch, int64_t rows, int64_t cols,
    const float* __restrict__ tensor_amax, uint2* __restrict__ codes, uint8_t* __restrict__ scales,
    float* __restrict__ tensor_scale, int64_t units)
{
    const int lane = threadIdx.x & 63, t = lane >> 4, j = lane & 15;
    const int64_t tr = rows / 16, tc = cols / 16, groups = (tc + 3) / 4;
    const int64_t waves_total = (int64_t)gridDim.x * (kT16Threads / 64);
    const int64_t wave_id = (int64_t)blockIdx.x * (kT16Threads / 64) + (threadIdx.x >> 6);
    for (int64_t u = wave_id; u < units; u += waves_total) {
        // unit = (tensor b, tile row ti, group of four tile columns g)
        const int64_t b = u / (tr * groups);
        const int64_t rem = u - b * tr * groups;
        const int64_t ti = rem / groups, g = rem - ti * groups;
        const int64_t tj = 4 * g + t;
        const bool live = tj < tc;  // the last group of a row may hold fewer tiles
        const float A_T = tensor_amax[b];
        const float s_t = (A_T == 0.0f) ? 0.0f : A_T / 2688.0f;
        if (ti == 0 && g == 0 && lane == 0)
            tensor_scale[b] = s_t;
        const int64_t elem = (b * rows + 16 * ti + j) * cols + 16 * tj;
        float v[16];
        float A = 0.0f;
        if (live) {
            load_row16<BF16>(x, elem, v);
#pragma unroll
            for (int i = 0; i < 16; ++i)
                A = fmaxf(A, fabsf(v[i]));
        }
        // tile maximum over the 16 lanes of the tile
#pragma unroll
        for (int off = 1; off < 16; off <<= 1)
            A = fmaxf(A, __shfl_xor(A, off, 64));
        if (!live)
            continue;
        uint32_t e = 0;
        if (s_t != 0.0f)
            e = e4m3_encode((A / 6.0f) / s_t);
        const float dec = e4m3_decode(e);
        uint32_t lo = 0, hi = 0;
        if (dec != 0.0f) {
            const float r = 1.0f / (dec * s_t);
            float y[16];
#pragma unroll
            for (int i = 0; i < 16; ++i)
                y[i] = v[i] * r;
            lo = pack8_nearest(y);
            hi = pack8_nearest(y + 8);
        }
        codes[elem / 16] = make_uint2(lo, hi);
        if (j == 0)
            scales[(b * tr + ti) * tc + tj] = (uint8_t)e;
    }
}

// Region of 64 x 64 values (4 x 4 tiles) per workgroup iteration.
__global__ __launch_bounds__(kT16Threads) void transpose_tile16_kernel(
    const uint8_t* __restrict__ codes, const uint8_t* __restrict__ scales,
    const float* __restrict__ tensor_scale, int64_t batch, int64_t rows, int64_t cols,
    uint8_t* __restrict__ codes_t, uint8_t* __restrict__ scales_t,
    float* __restrict__ tensor_scale_t, int64_t regions_r, int64_t regions_c)
{
    __shared__ uint2 tile_s[64][4];  // 64 input rows x 32 code bytes
    const int tid = threadIdx.x;
    const int64_t tr = rows / 16, tc = cols / 16;
    const int64_t per_tensor = regions_r * regions_c, total = per_tensor * batch;
    for (int64_t reg = blockIdx.x; reg < total; reg += gridDim.x) {
        const int64_t b = reg / per_tensor;
        const int64_t rem = reg - b * per_tensor;
        const int64_t rr = rem / regions_c, rc = rem - rr * regions_c;
        const int64_t r0 = 64 * rr, c0 = 64 * rc;
        const int rows_valid = (int)(rows - r0 < 64 ? rows - r0 : 64);  // multiples of 16
        const int cols_valid = (int)(cols - c0 < 64 ? cols - c0 : 64);
        if (rr == 0 && rc == 0 && tid == 0)
            tensor_scale_t[b] = tensor_scale[b];
        // load: thread -> input row tid / 4, 8-byte chunk tid % 4 (16 columns)
        {
            const int r = tid >> 2, q = tid & 3;
            uint2 w = make_uint2(0, 0);
            if (r < rows_valid && 16 * q < cols_valid)
                w = *reinterpret_cast<const uint2*>(codes + ((b * rows + r0 + r) * cols + c0 + 16 * q) / 2);
            tile_s[r][q] = w;
        }
        // tile scales: 16 threads, one tile each
        if (tid < 16) {
            const int a = tid >> 2, c = tid & 3;  // tile row / column inside the region
            if (16 * a < rows_valid && 16 * c < cols_valid) {
                const int64_t ti = r0 / 16 + a, tj = c0 / 16 + c;
                scales_t[(b * tc + tj) * tr + ti] = scales[(b * tr + ti) * tc + tj];
            }
        }
        __syncthreads();
        // transpose: thread -> output row c0 + c (input column), input rows 16 q .. 16 q + 15
        {
            const int c = tid >> 2, q = tid & 3;
            if (c < cols_valid && 16 * q < rows_valid) {
                const int shift = 4 * (c & 7);
                const int half = (c & 15) >> 3;  // which dword of the 8-byte chunk
                const int chunk = c >> 4;
                uint32_t out[2] = {0, 0};
#pragma unroll
                for (int m = 0; m < 16; ++m) {
                    const uint2 w = tile_s[16 * q + m][chunk];
                    const uint32_t nib = ((half ? w.y : w.x) >> shift) & 15u;
                    out[m >> 3] |= nib << (4 * (m & 7));
                }
                *reinterpret_cast<uint2*>(codes_t + ((b * cols + c0 + c) * rows + r0 + 16 * q) / 2) =
                    make_uint2(out[0], out[1]);
            }
        }
        __syncthreads();
    }
}

__global__ void copy_tensor_scales_kernel(const float* __restrict__ src, float* __restrict__ dst,
                                          int64_t n)
{
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n;
         i += (int64_t)gridDim.x * blockDim.x)
        dst[i] = src[i];
}

void launch_quantize_tile16(const void* x, bool bf16, int64_t batch, int64_t rows, int64_t cols,
                            const float* tensor_amax, uint8_t* codes, uint8_t* scales,
                            float* tensor_scale, hipStream_t s)
{
    const int64_t groups = (cols / 16 + 3) / 4;
    const int64_t units = batch * (rows / 16) * groups;  // one wave each
    if (units == 0)
        return;
    int64_t blocks = (units + 3) / 4;
    blocks = blocks < (1 << 30) ? blocks : (1 << 30);  // one unit per wave
    uint2* c2 = reinterpret_cast<uint2*>(codes);
    if (bf16)
        hipLaunchKernelGGL(quantize_tile16_kernel<true>, dim3((unsigned)blocks), dim3(kT16Threads), 0,
                           s, x, batch, rows, cols, tensor_amax, c2, scales, tensor_scale, units);
    else
        hipLaunchKernelGGL(quantize_tile16_kernel<false>, dim3((unsigned)blocks), dim3(kT16Threads),
                           0, s, x, batch, rows, cols, tensor_amax, c2, scales, tensor_scale, units);
}

void launch_transpose_tile16(const uint8_t* codes, const uint8_t* scales, const float* tensor_scale,
                             int64_t batch, int64_t rows, int64_t cols, uint8_t* codes_t,
                             uint8_t* scales_t, float* tensor_scale_t, hipStream_t s)
{
    const int64_t regions_r = (rows + 63) / 64, regions_c = (cols + 63) / 64;
    const int64_t total = regions_r * regions_c * batch;
    if (total == 0) {
        if (batch > 0)
            hipLaunchKernelGGL(copy_tensor_scales_kernel, dim3(1), dim3(256), 0, s, tensor_scale,
                               tensor_scale_t, batch);
        return;
    }
    const int64_t g = total < (1 << 20) ? total : (1 << 20);
    hipLaunchKernelGGL(transpose_tile16_kernel, dim3((unsigned)g), dim3(kT16Threads), 0, s, codes,
                       scales, tensor_scale, batch, rows, cols, codes_t, scales_t, tensor_scale_t,
                       regions_r, regions_c);
}

}  // namespace tq
