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
// Transpose: a workgroup moves a 128 x 256 region (8 x 16 tiles): 8 x 8 nibble
// blocks are transposed in registers and regrouped through LDS, so that input
// rows are read 128 contiguous bytes at a time and output rows written 64 bytes
// at a time; the 128 tile scales move one byte each.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

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

// Maximum over the 16 lanes of a DPP row (one tile): quad exchanges (lane ^ 1,
// lane ^ 2), then the half-row and row mirrors, which pair the quads.
__device__ __forceinline__ uint32_t row16_max(uint32_t v)
{
    v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0xB1, 0xF, 0xF, false));   // quad_perm 1,0,3,2
    v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x4E, 0xF, 0xF, false));   // quad_perm 2,3,0,1
    v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x141, 0xF, 0xF, false));  // row_half_mirror
    v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x140, 0xF, 0xF, false));  // row_mirror
    return v;
}

// WIDE: unit indices need 64 bits; otherwise they are split with 32-bit
// arithmetic.  The unit index is wave-uniform, so the split runs on the scalar
// unit.
template <bool BF16, bool WIDE>
__global__ __launch_bounds__(kT16Threads) void quantize_tile16_kernel(
    const void* __restrict__ x, int64_t rows, int64_t cols, const float* __restrict__ tensor_amax,
    uint2* __restrict__ codes, uint8_t* __restrict__ scales, float* __restrict__ tensor_scale,
    int64_t units)
{
    typedef typename std::conditional<WIDE, uint64_t, uint32_t>::type I;
    const int lane = threadIdx.x & 63, t = lane >> 4, j = lane & 15;
    const I tr = (I)(rows / 16), tc = (I)(cols / 16), groups = (tc + 3) / 4;
    const I per_tensor = tr * groups;
    const I waves_total = (I)gridDim.x * (kT16Threads / 64);
    // Consecutive workgroups are dealt to the 8 XCDs in turn; the remap gives
    // each XCD a contiguous run of units (6% over the plain order).
    const I per_xcd = ((I)gridDim.x + 7) / 8;
    const I bx = (I)blockIdx.x;
    const I blk = (bx & 7) * per_xcd + (bx >> 3);
    const I wave_id = blk * (kT16Threads / 64) + (I)__builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    for (I u = wave_id; u < (I)units; u += waves_total) {
        // unit = (tensor b, tile row ti, group of four tile columns g)
        const I b = u / per_tensor;
        const I rem = u - b * per_tensor;
        const I ti = rem / groups, g = rem - ti * groups;
        const I tj = 4 * g + (I)t;
        const bool live = tj < tc;  // the last group of a row may hold fewer tiles
        const float A_T = tensor_amax[b];
        const float s_t = (A_T == 0.0f) ? 0.0f : A_T / 2688.0f;
        if (ti == 0 && g == 0 && lane == 0)
            tensor_scale[b] = s_t;
        const int64_t elem = ((int64_t)b * rows + 16 * (int64_t)ti + j) * cols + 16 * (int64_t)tj;
        float v[16];
        uint32_t Ab = 0;  // |x| bits: integer order = value order
        if (live) {
            load_row16<BF16>(x, elem, v);
#pragma unroll
            for (int i = 0; i < 16; ++i)
                Ab = max(Ab, __float_as_uint(v[i]) & 0x7FFFFFFFu);
        }
        const float A = __uint_as_float(row16_max(Ab));  // tile maximum
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
            scales[((int64_t)b * tr + ti) * tc + tj] = (uint8_t)e;
    }
}

// Transpose of an 8 x 8 block of nibbles held as eight dwords (row r in r[r],
// column k in nibble k): three rounds of swapping the off-diagonal halves of
// 2 x 2 arrangements of 4 x 4, 2 x 2 and 1 x 1 sub-blocks.
__device__ __forceinline__ void swap_blocks(uint32_t& a, uint32_t& b, int s, uint32_t lo_mask)
{
    const uint32_t na = (a & lo_mask) | ((b << s) & ~lo_mask);
    const uint32_t nb = ((a >> s) & lo_mask) | (b & ~lo_mask);
    a = na;
    b = nb;
}
__device__ __forceinline__ void transpose8x8_nibbles(uint32_t r[8])
{
#pragma unroll
    for (int i = 0; i < 4; ++i)
        swap_blocks(r[i], r[i + 4], 16, 0x0000FFFFu);
#pragma unroll
    for (int i = 0; i < 8; i += (i & 1) ? 3 : 1)  // 0, 1, 4, 5
        swap_blocks(r[i], r[i + 2], 8, 0x00FF00FFu);
#pragma unroll
    for (int i = 0; i < 8; i += 2)
        swap_blocks(r[i], r[i + 1], 4, 0x0F0F0F0Fu);
}

// Region of kRR x kRC = 128 x 256 values (8 x 16 tiles) per workgroup iteration.
// Load: a thread takes two 8 x 8 nibble blocks (one dword from each of 8 input
// rows; the 32 lanes of a half-wave read 128 contiguous bytes of a row) and
// transposes them in registers; the transposed dwords go to LDS, where an
// output row (input column) is an LDS row of 16 dwords.  Store: four lanes
// write one output row's 64 bytes, 16 bytes each.
constexpr int kRR = 128, kRC = 256, kTPitch = 17;  // LDS dwords per output row (16 + 1 pad)

__global__ __launch_bounds__(kT16Threads) void transpose_tile16_kernel(
    const uint8_t* __restrict__ codes, const uint8_t* __restrict__ scales,
    const float* __restrict__ tensor_scale, int64_t batch, int64_t rows, int64_t cols,
    uint8_t* __restrict__ codes_t, uint8_t* __restrict__ scales_t,
    float* __restrict__ tensor_scale_t, int64_t regions_r, int64_t regions_c)
{
    __shared__ uint32_t t_s[kRC * kTPitch];
    const int tid = threadIdx.x;
    const int64_t tr = rows / 16, tc = cols / 16;
    const int64_t per_tensor = regions_r * regions_c, total = per_tensor * batch;
    const bool vec16 = (rows % 32) == 0;
    for (int64_t reg = blockIdx.x; reg < total; reg += gridDim.x) {
        const int64_t b = reg / per_tensor;
        const int64_t rem = reg - b * per_tensor;
        const int64_t rr = rem / regions_c, rc = rem - rr * regions_c;
        const int64_t r0 = kRR * rr, c0 = kRC * rc;
        const int rows_valid = (int)(rows - r0 < kRR ? rows - r0 : kRR);  // multiples of 16
        const int cols_valid = (int)(cols - c0 < kRC ? cols - c0 : kRC);
        if (rr == 0 && rc == 0 && tid == 0)
            tensor_scale_t[b] = tensor_scale[b];
        // tile scales: one thread per tile of the region
        if (tid < (kRR / 16) * (kRC / 16)) {
            const int ta = tid / (kRC / 16), tb = tid % (kRC / 16);  // tile row / column in the region
            if (16 * ta < rows_valid && 16 * tb < cols_valid) {
                const int64_t ti = r0 / 16 + ta, tj = c0 / 16 + tb;
                scales_t[(b * tc + tj) * tr + ti] = scales[(b * tr + ti) * tc + tj];
            }
        }
        // load and transpose 8 x 8 blocks: block (i, j) = input rows 8 i .., columns 8 j ..
#pragma unroll
        for (int s2 = 0; s2 < 2; ++s2) {
            const int blk = tid + kT16Threads * s2;
            const int i = blk / (kRC / 8), j = blk % (kRC / 8);
            uint32_t v[8] = {0, 0, 0, 0, 0, 0, 0, 0};
            if (8 * i < rows_valid && 8 * j < cols_valid) {
                const uint32_t* src = reinterpret_cast<const uint32_t*>(
                    codes + ((b * rows + r0 + 8 * i) * cols + c0 + 8 * j) / 2);
#pragma unroll
                for (int q = 0; q < 8; ++q)
                    v[q] = src[q * (cols / 8)];
            }
            transpose8x8_nibbles(v);
#pragma unroll
            for (int q = 0; q < 8; ++q)
                t_s[(8 * j + q) * kTPitch + i] = v[q];
        }
        __syncthreads();
        // store: four lanes per output row (input column c0 + c), each 16 bytes = 32
        // input rows, so that one store instruction writes 16 rows' 64-byte runs
#pragma unroll
        for (int pass = 0; pass < kRC / (kT16Threads / 4); ++pass) {
            const int c = (kT16Threads / 4) * pass + (tid >> 2), p = tid & 3;
            if (c < cols_valid && 32 * p < rows_valid) {
                const uint32_t* row = t_s + c * kTPitch + 4 * p;
                uint8_t* dst = codes_t + ((b * cols + c0 + c) * rows + r0) / 2 + 16 * p;
                if (vec16 && 32 * p + 32 <= rows_valid) {
                    *reinterpret_cast<uint4*>(dst) = make_uint4(row[0], row[1], row[2], row[3]);
                } else {
                    reinterpret_cast<uint2*>(dst)[0] = make_uint2(row[0], row[1]);
                    if (32 * p + 16 < rows_valid)
                        reinterpret_cast<uint2*>(dst)[1] = make_uint2(row[2], row[3]);
                }
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
    blocks = (blocks + 7) / 8 * 8;  // the XCD remap is a permutation only of a multiple of 8
    uint2* c2 = reinterpret_cast<uint2*>(codes);
    // 32-bit unit arithmetic when every index it forms fits
    const bool wide = units + 4 * blocks >= (int64_t(1) << 32) || batch * (rows / 16) * (cols / 16) >= (int64_t(1) << 32);
#define TQ_T16_LAUNCH(B, W)                                                                        \
    hipLaunchKernelGGL((quantize_tile16_kernel<B, W>), dim3((unsigned)blocks), dim3(kT16Threads), 0, s, \
                       x, rows, cols, tensor_amax, c2, scales, tensor_scale, units)
    if (bf16) {
        if (wide)
            TQ_T16_LAUNCH(true, true);
        else
            TQ_T16_LAUNCH(true, false);
    } else {
        if (wide)
            TQ_T16_LAUNCH(false, true);
        else
            TQ_T16_LAUNCH(false, false);
    }
#undef TQ_T16_LAUNCH
}

void launch_transpose_tile16(const uint8_t* codes, const uint8_t* scales, const float* tensor_scale,
                             int64_t batch, int64_t rows, int64_t cols, uint8_t* codes_t,
                             uint8_t* scales_t, float* tensor_scale_t, hipStream_t s)
{
    const int64_t regions_r = (rows + kRR - 1) / kRR, regions_c = (cols + kRC - 1) / kRC;
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
