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
// Work decomposition.  One workgroup (4 waves) computes a kBM x kBN output tile
// of one group (expert); each wave owns a 64 x 64 sub-tile = 2 x 2 MFMA
// 32x32x16 tiles.  The tile list is derived on the device from the group
// offsets (a wave-wide prefix sum of per-group tile counts), so no host
// synchronisation is needed.  Consecutive workgroup ids are dealt round-robin
// to the 8 XCDs; the id -> tile map undoes that, so each XCD walks a contiguous
// run of tiles in (M-tile, N-tile) order and the N-tiles of one M-tile share
// their activation rows through that XCD's L2.
//
// Pipeline.  The K loop is software-pipelined through registers: the global
// loads of K-slice s+1 (activations, weight codes, block scales) are issued
// before the MFMAs of slice s and only written to LDS (activations as is,
// weights dequantized with gfx950's packed FP4 -> f32 conversion) after them.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "tq_device.hpp"
#include "tq_kernels.hpp"

namespace tq {

constexpr int kBM = 128, kBN = 128, kBK = 64, kGThreads = 256;
constexpr int kLd = kBK + 8;            // bf16 per LDS row of an A or W tile
constexpr int kCLd = kBN + 8;           // bf16 per LDS row of the output tile
constexpr int kSmemHalves = 2 * kBM * kLd;  // A tile + W tile (kBM == kBN)
static_assert(kBM == kBN, "A and W tiles share one LDS layout");
static_assert(kBM * kCLd <= kSmemHalves, "output tile must fit in the operand tiles' LDS");

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));

__device__ __forceinline__ uint32_t f32_to_bf16_rne(float f)
{
    uint32_t u = __float_as_uint(f);
    u += 0x7FFFu + ((u >> 16) & 1u);
    return u >> 16;
}

// Eight codes (one dword, element 2j in the low nibble of byte j) times the
// block scale d as four dwords of bf16 pairs.  Exact.
__device__ __forceinline__ uint4 dequant8_bf16(uint32_t w, float d)
{
    const tq_f32x2 p0 = fp4x2_to_f32<0>(w), p1 = fp4x2_to_f32<1>(w);
    const tq_f32x2 p2 = fp4x2_to_f32<2>(w), p3 = fp4x2_to_f32<3>(w);
    return make_uint4(pack_hi16(p0[0] * d, p0[1] * d), pack_hi16(p1[0] * d, p1[1] * d),
                      pack_hi16(p2[0] * d, p2[1] * d), pack_hi16(p3[0] * d, p3[1] * d));
}

struct TileRegs {
    uint4 a[4];   // 4 x 8 bf16 of the A tile
    uint4 w;      // 32 weight codes (one row, 32 consecutive k)
    float d[2];   // their two block scales
};

__global__ __launch_bounds__(kGThreads, 3) void grouped_gemm_nvfp4_kernel(
    const uint16_t* __restrict__ a, const int32_t* __restrict__ group_offsets, int num_groups,
    int64_t n, int64_t k, const uint8_t* __restrict__ w_codes, const uint8_t* __restrict__ w_scales,
    const float* __restrict__ w_tensor_scale, uint16_t* __restrict__ out, int n_tiles)
{
    __shared__ __attribute__((aligned(16))) uint16_t smem[kSmemHalves];
    __shared__ int64_t s_tile[3];
    uint16_t* As = smem;
    uint16_t* Ws = smem + kBM * kLd;

    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;

    // ---- tile id: prefix sum of per-group M-tile counts (wave 0), XCD-aware order ----
    if (wave == 0) {
        int64_t carry = 0;
        int64_t found_e = -1, found_mt = 0;
        const int64_t b = blockIdx.x;
        // total tiles first (needed for the XCD split), then locate this tile
        int64_t total_m = 0;
        for (int g0 = 0; g0 < num_groups; g0 += 64) {
            const int g = g0 + lane;
            int64_t cnt = 0;
            if (g < num_groups) {
                const int64_t me = (int64_t)group_offsets[g + 1] - group_offsets[g];
                cnt = me > 0 ? (me + kBM - 1) / kBM : 0;
            }
#pragma unroll
            for (int off = 32; off >= 1; off >>= 1)
                cnt += __shfl_xor(cnt, off, 64);
            total_m += cnt;
        }
        const int64_t total = total_m * n_tiles;
        const int64_t per_xcd = (total + 7) / 8;
        const int64_t L = (b & 7) * per_xcd + (b >> 3);
        const bool live = (b >> 3) < per_xcd && L < total;
        const int64_t t = live ? L / n_tiles : -1;
        for (int g0 = 0; g0 < num_groups && live; g0 += 64) {
            const int g = g0 + lane;
            int64_t cnt = 0;
            if (g < num_groups) {
                const int64_t me = (int64_t)group_offsets[g + 1] - group_offsets[g];
                cnt = me > 0 ? (me + kBM - 1) / kBM : 0;
            }
            int64_t incl = cnt;  // inclusive prefix over the 64 lanes
#pragma unroll
            for (int off = 1; off < 64; off <<= 1) {
                const int64_t v = __shfl_up(incl, off, 64);
                if (lane >= off)
                    incl += v;
            }
            const int64_t lo = carry + incl - cnt;
            if (cnt > 0 && t >= lo && t < lo + cnt) {
                found_e = g;
                found_mt = t - lo;
            }
            carry += __shfl(incl, 63, 64);
        }
        // exactly one lane (or none) found the group
#pragma unroll
        for (int off = 32; off >= 1; off >>= 1) {
            const int64_t oe = __shfl_xor(found_e, off, 64);
            const int64_t om = __shfl_xor(found_mt, off, 64);
            if (oe > found_e) {
                found_e = oe;
                found_mt = om;
            }
        }
        if (lane == 0) {
            s_tile[0] = live ? found_e : -1;
            s_tile[1] = found_mt;
            s_tile[2] = live ? L % n_tiles : 0;
        }
    }
    __syncthreads();
    const int64_t e = s_tile[0];
    if (e < 0)
        return;
    const int64_t row0 = (int64_t)group_offsets[e] + s_tile[1] * kBM;
    const int64_t row_end = group_offsets[e + 1];
    const int64_t col0 = s_tile[2] * kBN;
    const int64_t kb = k / 16;  // scale blocks per weight row

    // per-thread load coordinates
    const int wn_row = tid >> 1, wk_half = tid & 1;  // weight row in tile, 32-k half
    const int64_t w_row = e * n + col0 + wn_row;
    const bool w_row_ok = col0 + wn_row < n;

    auto load = [&](int64_t k0, TileRegs& R) {
#pragma unroll
        for (int it = 0; it < 4; ++it) {
            const int idx = tid + it * kGThreads;
            const int r = idx >> 3, c8 = idx & 7;
            const int64_t gr = row0 + r, gk = k0 + 8 * c8;
            R.a[it] = (gr < row_end && gk < k) ? *reinterpret_cast<const uint4*>(a + gr * k + gk)
                                               : make_uint4(0, 0, 0, 0);
        }
        const int64_t gk = k0 + 32 * wk_half;
        R.w = make_uint4(0, 0, 0, 0);
        R.d[0] = R.d[1] = 0.0f;
        if (w_row_ok) {
            const uint8_t* wp = w_codes + (w_row * k + gk) / 2;
            if (gk + 32 <= k) {
                const uint2 lo = *reinterpret_cast<const uint2*>(wp);
                const uint2 hi = *reinterpret_cast<const uint2*>(wp + 8);
                R.w = make_uint4(lo.x, lo.y, hi.x, hi.y);
                R.d[0] = e4m3_decode(w_scales[w_row * kb + gk / 16]);
                R.d[1] = e4m3_decode(w_scales[w_row * kb + gk / 16 + 1]);
            } else if (gk + 16 <= k) {
                const uint2 lo = *reinterpret_cast<const uint2*>(wp);
                R.w = make_uint4(lo.x, lo.y, 0, 0);
                R.d[0] = e4m3_decode(w_scales[w_row * kb + gk / 16]);
            }
        }
    };
    auto store = [&](const TileRegs& R) {
#pragma unroll
        for (int it = 0; it < 4; ++it) {
            const int idx = tid + it * kGThreads;
            const int r = idx >> 3, c8 = idx & 7;
            *reinterpret_cast<uint4*>(As + r * kLd + 8 * c8) = R.a[it];
        }
        uint4* dst = reinterpret_cast<uint4*>(Ws + wn_row * kLd + 32 * wk_half);
        dst[0] = dequant8_bf16(R.w.x, R.d[0]);
        dst[1] = dequant8_bf16(R.w.y, R.d[0]);
        dst[2] = dequant8_bf16(R.w.z, R.d[1]);
        dst[3] = dequant8_bf16(R.w.w, R.d[1]);
    };

    const int wm = wave >> 1, wn = wave & 1;
    f32x16_t acc[2][2];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r)
                acc[i][j][r] = 0.0f;

    TileRegs R;
    if (k > 0) {
        load(0, R);
        store(R);
    }
    __syncthreads();
    for (int64_t k0 = 0; k0 < k; k0 += kBK) {
        const bool more = k0 + kBK < k;
        if (more)
            load(k0 + kBK, R);
#pragma unroll
        for (int kk = 0; kk < kBK / 16; ++kk) {
            bf16x8_t af[2], bfr[2];
#pragma unroll
            for (int i = 0; i < 2; ++i)
                af[i] = __builtin_bit_cast(bf16x8_t, *reinterpret_cast<const uint4*>(
                    As + (64 * wm + 32 * i + (lane & 31)) * kLd + 16 * kk + 8 * (lane >> 5)));
#pragma unroll
            for (int j = 0; j < 2; ++j)
                bfr[j] = __builtin_bit_cast(bf16x8_t, *reinterpret_cast<const uint4*>(
                    Ws + (64 * wn + 32 * j + (lane & 31)) * kLd + 16 * kk + 8 * (lane >> 5)));
#pragma unroll
            for (int i = 0; i < 2; ++i)
#pragma unroll
                for (int j = 0; j < 2; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[i], bfr[j], acc[i][j], 0, 0, 0);
        }
        __syncthreads();
        if (more) {
            store(R);
            __syncthreads();
        }
    }

    // ---- epilogue: scale, RNE to bf16, stage the tile in LDS, coalesced stores ----
    const float s_e = w_tensor_scale[e];
    uint16_t* Cs = smem;
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int row = 64 * wm + 32 * i + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
                const int col = 64 * wn + 32 * j + (lane & 31);
                Cs[row * kCLd + col] = (uint16_t)f32_to_bf16_rne(acc[i][j][r] * s_e);
            }
    __syncthreads();
    const bool vec_ok = (n % 8) == 0;
#pragma unroll
    for (int it = 0; it < (kBM * kBN / 8) / kGThreads; ++it) {
        const int idx = tid + it * kGThreads;
        const int r = idx / (kBN / 8), c8 = idx % (kBN / 8);
        const int64_t gr = row0 + r, gc = col0 + 8 * c8;
        if (gr >= row_end || gc >= n)
            continue;
        const uint4 v = *reinterpret_cast<const uint4*>(Cs + r * kCLd + 8 * c8);
        uint16_t* dst = out + gr * n + gc;
        if (vec_ok && gc + 8 <= n) {
            *reinterpret_cast<uint4*>(dst) = v;
        } else {
            const uint32_t w[4] = {v.x, v.y, v.z, v.w};
            for (int t = 0; t < 8 && gc + t < n; ++t)
                dst[t] = (uint16_t)(w[t >> 1] >> (16 * (t & 1)));
        }
    }
}

void launch_grouped_gemm_nvfp4(const uint16_t* a, const int32_t* group_offsets, int num_groups,
                               int64_t m_total, int64_t n, int64_t k, const uint8_t* w_codes,
                               const uint8_t* w_scales, const float* w_tensor_scale, uint16_t* out,
                               hipStream_t s)
{
    const int n_tiles = (int)((n + kBN - 1) / kBN);
    const int64_t m_tiles_max = (m_total + kBM - 1) / kBM + num_groups;
    int64_t grid = m_tiles_max * n_tiles;
    if (grid == 0)
        return;
    // a multiple of 8 with at least ceil(total/8) groups per XCD slot
    grid = ((grid + 7) / 8) * 8;
    hipLaunchKernelGGL(grouped_gemm_nvfp4_kernel, dim3((unsigned)grid), dim3(kGThreads), 0, s, a,
                       group_offsets, num_groups, n, k, w_codes, w_scales, w_tensor_scale, out,
                       n_tiles);
}

}  // namespace tq
