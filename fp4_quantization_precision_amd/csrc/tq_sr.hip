// tq_sr.hip - dequantize -> transpose -> stochastic-rounding requantize (gfx950).
//
// [TML] "싱킹 머신스 랩, 4비트 학습 기법 공개", forward/backward-mismatch
// paragraph: a transpose changes which 16 values share a scale, so the stored
// tensor is taken back to higher precision, transposed and quantized again with
// stochastic rounding.  Arithmetic and random-byte layout are those of
// include/tq.h.
//
// One workgroup owns a tile of kTR input rows x kTC input columns.  Each thread
// loads two input rows of one 32-column half of the tile (codes + block scales),
// dequantizes them exactly (u = +-G[m] * dec(e) has at most 6 significant bits,
// so bf16 holds it) and writes them transposed into LDS, so every output row of
// the tile is contiguous there.  Then each lane owns one output row and four new
// 16-element blocks: block amax, E4M3 scale, one Philox4x32-10 call for the
// block's 16 random bytes, 16 stochastic roundings and one packed store.  A
// wave's 64 lanes cover 64 output rows, and the four waves of a workgroup cover
// 4 x 64 = 256 consecutive input rows, so every output row receives one full
// 128-byte run of codes per tile.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "tq_device.hpp"
#include "tq_kernels.hpp"

namespace tq {

constexpr int kTR = 256;  // input rows per tile (= output elements per row)
constexpr int kTC = 64;   // input columns per tile (= output rows)
constexpr int kSThreads = 256;
// LDS row = one output row of the tile: kTR bf16 values as kTR/2 dwords, padded
// so that lanes reading 16-byte runs of consecutive rows hit distinct banks.
constexpr int kLdsStride = kTR / 2 + 4;

__global__ __launch_bounds__(kSThreads) void requant_transpose_sr_kernel(
    const uint8_t* __restrict__ codes, const uint8_t* __restrict__ scales,
    const float* __restrict__ tensor_scale, int64_t batch, int64_t rows, int64_t cols,
    uint32_t seed_lo, uint32_t seed_hi, uint8_t* __restrict__ codes_t,
    uint8_t* __restrict__ scales_t, float* __restrict__ tensor_scale_t, int64_t tiles_r,
    int64_t tiles_c)
{
    __shared__ uint32_t u_s[kTC * kLdsStride];
    const int64_t tiles_per_tensor = tiles_r * tiles_c;
    const int64_t total_tiles = tiles_per_tensor * batch;
    const int tid = threadIdx.x;

    for (int64_t tile = blockIdx.x; tile < total_tiles; tile += gridDim.x) {
        const int64_t b = tile / tiles_per_tensor;
        const int64_t rem = tile - b * tiles_per_tensor;
        const int64_t tr = rem / tiles_c, tc = rem - tr * tiles_c;
        const int64_t r0 = tr * kTR, c0 = tc * kTC;
        if (tr == 0 && tc == 0 && tid == 0)
            tensor_scale_t[b] = tensor_scale[b];

        // ---- load + exact dequant: thread owns input rows (2p, 2p+1) of the tile
        //      and one 32-column half; it writes both rows' values of a column as
        //      one dword, so a wave writes 64 consecutive dwords per column ----
        {
            const int p = tid & 127, half = tid >> 7;
            const int64_t cols_valid = cols - c0 < kTC ? cols - c0 : kTC;  // multiple of 16
#pragma unroll
            for (int blk = 0; blk < 2; ++blk) {
                const int cl = 32 * half + 16 * blk;  // first tile column of this block
                uint2 q[2] = {make_uint2(0, 0), make_uint2(0, 0)};
                float d[2] = {0.0f, 0.0f};
                if (cl < cols_valid) {
#pragma unroll
                    for (int rr = 0; rr < 2; ++rr) {
                        const int64_t gr = r0 + 2 * p + rr;
                        if (gr < rows) {
                            q[rr] = *reinterpret_cast<const uint2*>(
                                codes + ((b * rows + gr) * cols + c0 + cl) / 2);
                            d[rr] = e4m3_decode(scales[(b * rows + gr) * (cols / 16) + (c0 + cl) / 16]);
                        }
                    }
                }
                // u = +-G[m] * dec(e), exact; the two rows' values of column cl+i share one dword
                uint32_t* dst = u_s + cl * kLdsStride + p;
#pragma unroll
                for (int half8 = 0; half8 < 2; ++half8) {
                    const uint32_t w0 = half8 ? q[0].y : q[0].x;
                    const uint32_t w1 = half8 ? q[1].y : q[1].x;
                    tq_f32x2 a0[4], a1[4];
                    a0[0] = fp4x2_to_f32<0>(w0); a0[1] = fp4x2_to_f32<1>(w0);
                    a0[2] = fp4x2_to_f32<2>(w0); a0[3] = fp4x2_to_f32<3>(w0);
                    a1[0] = fp4x2_to_f32<0>(w1); a1[1] = fp4x2_to_f32<1>(w1);
                    a1[2] = fp4x2_to_f32<2>(w1); a1[3] = fp4x2_to_f32<3>(w1);
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
#pragma unroll
                        for (int t = 0; t < 2; ++t) {
                            const int i = 8 * half8 + 2 * j + t;
                            dst[i * kLdsStride] = pack_hi16(a0[j][t] * d[0], a1[j][t] * d[1]);
                        }
                    }
                }
            }
        }
        __syncthreads();

        // ---- requantize: lane -> output row c0 + lane, wave -> 4 new blocks ----
        {
            const int lane = tid & 63, wave = tid >> 6;
            const int64_t oc = c0 + lane;  // output row (input column)
            if (oc < cols) {
                const uint32_t* urow = u_s + lane * kLdsStride;
                uint32_t words[8];
                uint32_t sc = 0;
                int nvalid = 0;
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const int local = 64 * wave + 16 * q;  // first input row of the block
                    words[2 * q] = words[2 * q + 1] = 0;
                    if (r0 + local >= rows)
                        continue;
                    ++nvalid;
                    const uint4 w0 = *reinterpret_cast<const uint4*>(urow + local / 2);
                    const uint4 w1 = *reinterpret_cast<const uint4*>(urow + local / 2 + 4);
                    const uint32_t pk[8] = {w0.x, w0.y, w0.z, w0.w, w1.x, w1.y, w1.z, w1.w};
                    float u[16];
#pragma unroll
                    for (int i = 0; i < 8; ++i) {
                        u[2 * i] = bf16_lo(pk[i]);
                        u[2 * i + 1] = bf16_hi(pk[i]);
                    }
                    float A = 0.0f;
#pragma unroll
                    for (int i = 0; i < 16; ++i)
                        A = fmaxf(A, fabsf(u[i]));
                    const uint32_t e = e4m3_encode(A / 6.0f);
                    sc |= e << (8 * q);
                    const float dec = e4m3_decode(e);
                    if (dec == 0.0f)
                        continue;
                    const float rr = 1.0f / dec;
                    const uint64_t beta = (uint64_t)(((b * cols + oc) * rows + r0 + local) / 16);
                    const u32x4 rnd = philox4x32_10((uint32_t)beta, (uint32_t)(beta >> 32), 0u, 0u,
                                                    seed_lo, seed_hi);
                    const uint32_t rw[4] = {rnd.x, rnd.y, rnd.z, rnd.w};
                    uint32_t lo = 0, hi = 0;
#pragma unroll
                    for (int i = 0; i < 16; ++i) {
                        const float y = u[i] * rr;
                        const float k = (float)((rw[i >> 2] >> (8 * (i & 3))) & 0xFFu);
                        const uint32_t c = e2m1_code(y, e2m1_sr_bits(fabsf(y), k));
                        if (i < 8)
                            lo |= c << (4 * i);
                        else
                            hi |= c << (4 * (i - 8));
                    }
                    words[2 * q] = lo;
                    words[2 * q + 1] = hi;
                }
                // output row oc, input rows r0 + 64*wave ... + 16*nvalid
                uint8_t* orow = codes_t + ((b * cols + oc) * rows + r0 + 64 * wave) / 2;
                uint8_t* srow = scales_t + (b * cols + oc) * (rows / 16) + (r0 + 64 * wave) / 16;
                if (nvalid == 4 && ((uintptr_t)orow & 15u) == 0) {
                    reinterpret_cast<uint4*>(orow)[0] = make_uint4(words[0], words[1], words[2], words[3]);
                    reinterpret_cast<uint4*>(orow)[1] = make_uint4(words[4], words[5], words[6], words[7]);
                } else {
                    for (int q = 0; q < nvalid; ++q)
                        reinterpret_cast<uint2*>(orow)[q] = make_uint2(words[2 * q], words[2 * q + 1]);
                }
                if (nvalid == 4 && ((uintptr_t)srow & 3u) == 0) {
                    *reinterpret_cast<uint32_t*>(srow) = sc;
                } else {
                    for (int q = 0; q < nvalid; ++q)
                        srow[q] = (uint8_t)(sc >> (8 * q));
                }
            }
        }
        __syncthreads();
    }
}

__global__ void copy_scalars_kernel(const float* __restrict__ src, float* __restrict__ dst, int64_t n)
{
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n;
         i += (int64_t)gridDim.x * blockDim.x)
        dst[i] = src[i];
}

void launch_requant_transpose_sr(const uint8_t* codes, const uint8_t* scales,
                                 const float* tensor_scale, int64_t batch, int64_t rows,
                                 int64_t cols, uint64_t seed, uint8_t* codes_t, uint8_t* scales_t,
                                 float* tensor_scale_t, hipStream_t s)
{
    const int64_t tiles_r = (rows + kTR - 1) / kTR, tiles_c = (cols + kTC - 1) / kTC;
    const int64_t total = tiles_r * tiles_c * batch;
    if (total == 0) {
        // empty tensors: only the tensor scales are defined (copied)
        if (batch > 0)
            hipLaunchKernelGGL(copy_scalars_kernel, dim3(1), dim3(256), 0, s, tensor_scale,
                               tensor_scale_t, batch);
        return;
    }
    const int64_t g = total < (1 << 20) ? total : (1 << 20);
    hipLaunchKernelGGL(requant_transpose_sr_kernel, dim3((unsigned)g), dim3(kSThreads), 0, s, codes,
                       scales, tensor_scale, batch, rows, cols, (uint32_t)seed,
                       (uint32_t)(seed >> 32), codes_t, scales_t, tensor_scale_t, tiles_r, tiles_c);
}

}  // namespace tq
