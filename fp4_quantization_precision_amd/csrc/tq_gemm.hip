// tq_gemm.hip - grouped GEMM with NVFP4 expert weights and bf16 activations (gfx950).
//
// [TML] "싱킹 머신스 랩, 4비트 학습 기법 공개", summary box and the paragraph on
// where 4-bit compute is used: the MoE layers' forward runs with NVFP4 operands.
// Here the weights are NVFP4 and the activations bf16: each weight tile is
// dequantized exactly into LDS (G[m] * dec(e) has at most 6 significant bits, so
// bf16 holds it), the products go through bf16 MFMA with fp32 accumulation, and
// the per-expert fp32 tensor scale is applied once in the epilogue before the
// round-to-nearest-even conversion to bf16.
//
// Work decomposition: one workgroup computes a kBM x kBN output tile of one
// group (expert); the tile list is derived on the device from the group offsets
// (no host synchronisation).  Four waves in a 2 x 2 arrangement each own a
// 64 x 64 sub-tile = 2 x 2 MFMA 32x32x16 tiles.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "tq_device.hpp"
#include "tq_kernels.hpp"

namespace tq {

constexpr int kBM = 128, kBN = 128, kBK = 64, kGThreads = 256;
constexpr int kPad = 8;  // bf16 elements of padding per LDS row

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));

// Two E2M1 codes (one byte, low nibble first) times the block scale d, as two
// bf16 values in one dword (exact).
__device__ __forceinline__ uint32_t dequant_pair_bf16(uint32_t byte, float d)
{
    const uint32_t c0 = byte & 15u, c1 = (byte >> 4) & 15u;
    const uint32_t v0 = (__float_as_uint(e2m1_value(c0 & 7u) * d) >> 16) | ((c0 & 8u) << 12);
    const uint32_t v1 = (__float_as_uint(e2m1_value(c1 & 7u) * d) >> 16) | ((c1 & 8u) << 12);
    return v0 | (v1 << 16);
}

__device__ __forceinline__ uint32_t f32_to_bf16_rne(float f)
{
    uint32_t u = __float_as_uint(f);
    u += 0x7FFFu + ((u >> 16) & 1u);
    return u >> 16;
}

__global__ __launch_bounds__(kGThreads) void grouped_gemm_nvfp4_kernel(
    const uint16_t* __restrict__ a, const int32_t* __restrict__ group_offsets, int num_groups,
    int64_t n, int64_t k, const uint8_t* __restrict__ w_codes, const uint8_t* __restrict__ w_scales,
    const float* __restrict__ w_tensor_scale, uint16_t* __restrict__ out, int n_tiles)
{
    __shared__ __attribute__((aligned(16))) uint16_t As[kBM * (kBK + kPad)];
    __shared__ __attribute__((aligned(16))) uint16_t Ws[kBN * (kBK + kPad)];
    __shared__ int64_t s_info[3];

    const int tid = threadIdx.x;
    if (tid == 0) {
        const int64_t t = blockIdx.x / n_tiles;
        int64_t acc = 0, e = -1, mt = 0;
        for (int g = 0; g < num_groups; ++g) {
            const int64_t me = (int64_t)group_offsets[g + 1] - group_offsets[g];
            const int64_t tiles = me > 0 ? (me + kBM - 1) / kBM : 0;
            if (t < acc + tiles) {
                e = g;
                mt = t - acc;
                break;
            }
            acc += tiles;
        }
        s_info[0] = e;
        s_info[1] = mt;
    }
    __syncthreads();
    const int64_t e = s_info[0];
    if (e < 0)
        return;
    const int64_t nt = blockIdx.x % n_tiles;
    const int64_t row0 = (int64_t)group_offsets[e] + s_info[1] * kBM;
    const int64_t row_end = group_offsets[e + 1];
    const int64_t col0 = nt * kBN;
    const int64_t kb = k / 16;  // scale blocks per weight row

    const int lane = tid & 63, wave = tid >> 6;
    const int wm = wave >> 1, wn = wave & 1;

    f32x16_t acc[2][2];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r)
                acc[i][j][r] = 0.0f;

    for (int64_t k0 = 0; k0 < k; k0 += kBK) {
        // ---- A tile: kBM rows x kBK bf16 -> LDS (zero outside the group / k) ----
#pragma unroll
        for (int it = 0; it < (kBM * kBK / 8) / kGThreads; ++it) {
            const int idx = tid + it * kGThreads;
            const int r = idx / (kBK / 8), c8 = idx % (kBK / 8);
            const int64_t gr = row0 + r, gk = k0 + 8 * c8;
            uint4 q = make_uint4(0, 0, 0, 0);
            if (gr < row_end && gk < k)
                q = *reinterpret_cast<const uint4*>(a + gr * k + gk);
            *reinterpret_cast<uint4*>(As + r * (kBK + kPad) + 8 * c8) = q;
        }
        // ---- W tile: kBN weight rows x kBK, dequantized exactly to bf16 ----
        {
            const int nn = tid >> 1, h = tid & 1;
            const int64_t gn = col0 + nn;
            const int64_t gk = k0 + 32 * h;
            uint32_t pk[16];
#pragma unroll
            for (int j = 0; j < 16; ++j)
                pk[j] = 0;
            if (gn < n) {
                const int64_t wrow = (e * n + gn);
#pragma unroll
                for (int blk = 0; blk < 2; ++blk) {
                    const int64_t gkb = gk + 16 * blk;
                    if (gkb < k) {
                        const uint2 q = *reinterpret_cast<const uint2*>(w_codes + (wrow * k + gkb) / 2);
                        const float d = e4m3_decode(w_scales[wrow * kb + gkb / 16]);
#pragma unroll
                        for (int j = 0; j < 4; ++j) {
                            pk[8 * blk + j] = dequant_pair_bf16((q.x >> (8 * j)) & 0xFFu, d);
                            pk[8 * blk + 4 + j] = dequant_pair_bf16((q.y >> (8 * j)) & 0xFFu, d);
                        }
                    }
                }
            }
            uint4* dst = reinterpret_cast<uint4*>(Ws + nn * (kBK + kPad) + 32 * h);
#pragma unroll
            for (int j = 0; j < 4; ++j)
                dst[j] = make_uint4(pk[4 * j], pk[4 * j + 1], pk[4 * j + 2], pk[4 * j + 3]);
        }
        __syncthreads();

        // ---- MFMA over the four 16-deep k slices of the tile ----
#pragma unroll
        for (int kk = 0; kk < kBK / 16; ++kk) {
            bf16x8_t af[2], bfr[2];
#pragma unroll
            for (int i = 0; i < 2; ++i) {
                const uint4 q = *reinterpret_cast<const uint4*>(
                    As + (64 * wm + 32 * i + (lane & 31)) * (kBK + kPad) + 16 * kk + 8 * (lane >> 5));
                af[i] = __builtin_bit_cast(bf16x8_t, q);
            }
#pragma unroll
            for (int j = 0; j < 2; ++j) {
                const uint4 q = *reinterpret_cast<const uint4*>(
                    Ws + (64 * wn + 32 * j + (lane & 31)) * (kBK + kPad) + 16 * kk + 8 * (lane >> 5));
                bfr[j] = __builtin_bit_cast(bf16x8_t, q);
            }
#pragma unroll
            for (int i = 0; i < 2; ++i)
#pragma unroll
                for (int j = 0; j < 2; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[i], bfr[j], acc[i][j], 0, 0, 0);
        }
        __syncthreads();
    }

    // ---- epilogue: scale by the expert's tensor scale, RNE to bf16 ----
    const float s_e = w_tensor_scale[e];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int64_t gr = row0 + 64 * wm + 32 * i + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
                const int64_t gc = col0 + 64 * wn + 32 * j + (lane & 31);
                if (gr < row_end && gc < n)
                    out[gr * n + gc] = (uint16_t)f32_to_bf16_rne(acc[i][j][r] * s_e);
            }
}

void launch_grouped_gemm_nvfp4(const uint16_t* a, const int32_t* group_offsets, int num_groups,
                               int64_t m_total, int64_t n, int64_t k, const uint8_t* w_codes,
                               const uint8_t* w_scales, const float* w_tensor_scale, uint16_t* out,
                               hipStream_t s)
{
    const int n_tiles = (int)((n + kBN - 1) / kBN);
    const int64_t m_tiles_max = (m_total + kBM - 1) / kBM + num_groups;
    const int64_t grid = m_tiles_max * n_tiles;
    if (grid == 0)
        return;
    hipLaunchKernelGGL(grouped_gemm_nvfp4_kernel, dim3((unsigned)grid), dim3(kGThreads), 0, s, a,
                       group_offsets, num_groups, n, k, w_codes, w_scales, w_tensor_scale, out,
                       n_tiles);
}

}  // namespace tq
