// tq_sr.hip - dequantize -> transpose -> stochastic-rounding requantize (gfx950).
//
// [TML] "싱킹 머신스 랩, 4비트 학습 기법 공개", forward/backward-mismatch
// paragraph: a transpose changes which 16 values share a scale, so the stored
// tensor is taken back to higher precision, transposed and quantized again with
// stochastic rounding.  Arithmetic and random-byte layout are those of
// include/tq.h.
//
// One workgroup owns a tile of kTR = 128 input rows x kTC = 256 input columns,
// so every input row is read as one 128-byte run of codes (plus 16 scale
// bytes) and every output row of the tile is written as one 64-byte run.  The
// grid is persistent: each workgroup walks a strided list of tiles and loads
// the next tile's codes and scales into registers while it requantizes the
// current one.
//
// Load phase: a thread takes a pair of input rows and one 32-column chunk,
// dequantizes them exactly in binary16 (u = +-G[m] * dec(e) has at most 6
// significant bits and lies in [2^-10, 2688] or is zero, so the packed FP4 ->
// f16 conversion and one packed f16 multiply by the E4M3 scale, itself an f16
// value, are exact) and stores each column's two values as one dword into LDS,
// where tile column c (= output row) is an LDS row.  The row-pair index is
// XOR-swizzled with four times the column's chunk so that each half-wave's
// stores hit 32 distinct banks, and the LDS row pitch is 68 dwords so that the
// 16-byte reads of the next phase are conflict-free as well (their two halves
// swap places for odd chunks).
//
// Requantize phase: a thread owns one output row and four new 16-element
// blocks: block amax (on the f16 magnitude patterns, whose integer order is the
// value order), E4M3 scale, one Philox4x32-10 call for the block's 16 random
// bytes, y = u * r' (one mixed-precision FMA per value, f16 u, with a -0 addend
// so that it is the rounded product, sign of zero included), then the
// stochastic rounding.  The floor grid point of each value comes from
// v_cvt_scalef32_sr_pk_fp4_f32 with a zero seed (which truncates to the grid
// toward zero, sign kept), its value from the packed decode; the step up is
// taken iff G[lo] + k * D / 256 < |y| with D the grid spacing above G[lo] (all
// terms exact).  Values above 6 in magnitude (the E4M3 block scale may round
// down) truncate to the top code, whose step up is masked off, so saturation
// needs no per-value clamp.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "tq_device.hpp"
#include "tq_kernels.hpp"

namespace tq {

constexpr int kTR = 128;          // input rows per tile (= output elements per row)
constexpr int kTC = 256;          // input columns per tile (= output rows)
constexpr int kSThreads = 512;
constexpr int kLdsStride = 68;    // dwords per LDS row: 64 row pairs + 4 pad

typedef _Float16 sr_h2 __attribute__((ext_vector_type(2)));
typedef unsigned short sr_u16x2 __attribute__((ext_vector_type(2)));

// the two E2M1 codes of byte S of w as f16 (exact: every E2M1 value is an f16 value)
template <int S>
__device__ __forceinline__ sr_h2 fp4x2_to_h2(uint32_t w)
{
    return __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, S);
}

// LDS dword of tile column c, input row pair p.  LDS stores are served 32 lanes at a
// time over 32 four-byte banks.  A store instruction of the load phase has one
// column offset within each lane's 32-column chunk, so c * 68 is the same bank for
// every lane, and the row pair XOR 4 * chunk puts the 32 lanes of each half-wave
// (four row pairs x eight chunks) on 32 distinct banks.
__device__ __forceinline__ int lds_slot(int c, int p) { return c * kLdsStride + (p ^ (4 * (c >> 5))); }

// New block scale from the block maximum A (0, or at least 2^-10: a nonzero |u| is
// G[m] * dec(e) >= 0.5 * 2^-9).  The three steps give the bits of the plain forms
// e4m3_encode(A / 6), e4m3_decode and 1 / dec, each checked on the device over its whole
// domain here: A / 6 as A * RN(1/6) with one FMA correction equals the correctly rounded
// quotient for every finite A >= 2^-125 (and 0); the packed f32 -> E4M3 conversion
// equals the nearest rule for 0 <= d <= 464 and gives NaN above (the minimum with 448
// gives the rule's saturation); v_rcp_f32 with one Newton step equals the correctly
// rounded reciprocal of
// all 126 nonzero finite E4M3 values.  d = 0 gives rcp = 0: every y of the block is then
// +-0, which the stochastic rounding below maps to code 0 whatever the random bytes, so
// zero-scale blocks need no branch.
struct BlockScale { uint32_t e; float dec, rcp; };
__device__ __forceinline__ BlockScale block_scale(float A)
{
    typedef short s16x2 __attribute__((ext_vector_type(2)));
    constexpr float kSixth = 1.0f / 6.0f;
    const float q0 = A * kSixth;
    const float d = __builtin_fmaf(__builtin_fmaf(-q0, 6.0f, A), kSixth, q0);
    s16x2 r = {0, 0};
    r = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(r, fminf(d, 448.0f), 0.0f, 1.0f, false);
    const uint32_t e = __builtin_bit_cast(uint32_t, r) & 0xFFu;
    const float dec = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(e, 1.0f, false)[0];
    const float dd = dec == 0.0f ? 1.0f : dec;
    const float r0 = __builtin_amdgcn_rcpf(dd);
    const float r1 = __builtin_fmaf(__builtin_fmaf(-dd, r0, 1.0f), r0, r0);
    return {e, dec, dec == 0.0f ? 0.0f : r1};
}

// Stochastic rounding of eight values with their random bytes k[0..7]: floor
// codes from the hardware truncation (saturating at 6), plus one where the
// random byte falls below the distance to the floor point, except from the top
// code.  The grid spacing D
// above the floor point, divided by 256, is 2^-9 below 2, 2^-8 for 2 and 3 and
// 2^-7 for 4 and 6; it is decoded from the floor code itself: the magnitude
// with bit 0 cleared is the code of 0, 1, 2 or 4 (0 for the first two grid
// points, which is then replaced by the code of 1), and the conversion's
// power-of-two scale 2^-9 makes that D / 256 exactly.
__device__ __forceinline__ uint32_t sr_pack8(const float yc[8], const float k[8])
{
    uint32_t P = 0;
    P = floor_pk_fp4<0>(P, yc[0], yc[1]);
    P = floor_pk_fp4<1>(P, yc[2], yc[3]);
    P = floor_pk_fp4<2>(P, yc[4], yc[5]);
    P = floor_pk_fp4<3>(P, yc[6], yc[7]);
    const tq_f32x2 g0 = fp4x2_to_f32<0>(P), g1 = fp4x2_to_f32<1>(P);
    const tq_f32x2 g2 = fp4x2_to_f32<2>(P), g3 = fp4x2_to_f32<3>(P);
    const float g[8] = {g0[0], g0[1], g1[0], g1[1], g2[0], g2[1], g3[0], g3[1]};
    const uint32_t x = P & 0x66666666u;                                    // m & 6 per nibble
    const uint32_t nz = (x | (x >> 1)) & 0x22222222u;                      // bit 1: m & 6 != 0
    const uint32_t Q = x | (nz ^ 0x22222222u);                             // 0 -> code of 1
    const tq_f32x2 d0 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(Q, 0x1p-9f, 0);
    const tq_f32x2 d1 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(Q, 0x1p-9f, 1);
    const tq_f32x2 d2 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(Q, 0x1p-9f, 2);
    const tq_f32x2 d3 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(Q, 0x1p-9f, 3);
    const float step[8] = {d0[0], d0[1], d1[0], d1[1], d2[0], d2[1], d3[0], d3[1]};
    // Step up iff t = |g| + k * step < |y|, i.e. iff t - |y| is negative: the
    // sum t is exact and a rounded difference keeps the sign of the exact one
    // (an exact zero is +0, not a step).  Each difference's top nibble is
    // shifted into an accumulator, last value first, so that value i's sign bit
    // lands on bit 3 of nibble i.
    uint32_t acc = 0;
#pragma unroll
    for (int i = 7; i >= 0; --i) {
        const float t = __builtin_fmaf(k[i], step[i], fabsf(g[i]));  // exact: no rounding occurs
        acc = __builtin_amdgcn_alignbit(acc, __float_as_uint(t - fabsf(yc[i])), 28);
    }
    uint32_t U = (acc >> 3) & 0x11111111u;
    // |y| may exceed 6 (the block scale is rounded to E4M3); its floor is then
    // the top code 7, which never steps up: clear the step of magnitude-7 nibbles
    U &= ~(P & (P >> 1) & (P >> 2));
    return clear_negative_zero(P + U);
}

// WIDE: tile indices need 64 bits; otherwise the per-tile index arithmetic is
// done in 32 bits (64-bit division is a long instruction sequence).
template <bool WIDE>
__global__ __launch_bounds__(kSThreads, 2) void requant_transpose_sr_kernel(
    const uint8_t* __restrict__ codes, const uint8_t* __restrict__ scales,
    const float* __restrict__ tensor_scale, int64_t batch, int64_t rows, int64_t cols,
    uint32_t seed_lo, uint32_t seed_hi, uint8_t* __restrict__ codes_t,
    uint8_t* __restrict__ scales_t, float* __restrict__ tensor_scale_t, int64_t tiles_r,
    int64_t tiles_c, int vec_in, int vec_scale_in, int vec_out, int vec_scale_out)
{
    __shared__ __attribute__((aligned(16))) uint32_t u_s[kTC * kLdsStride];
    const int64_t tiles_per_tensor = tiles_r * tiles_c;
    const int64_t total_tiles = tiles_per_tensor * batch;
    const int64_t paired = total_tiles & ~(int64_t)15;
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int64_t sc_pitch = cols / 16, sct_pitch = rows / 16;

    // tile coordinates of work item idx; workgroups idx and idx + 8 run on the
    // same XCD: give them the two tiles that write the two halves of the same
    // 128-byte output runs
    struct Tile { int64_t b, r0, c0; int rows_valid, cols_valid; bool first; };
    using I = typename std::conditional<WIDE, uint64_t, uint32_t>::type;
    auto tile_of = [&](int64_t idx) -> Tile {
        const I tile = (I)(idx < paired ? (idx & ~(int64_t)15) + 2 * (idx & 7) + ((idx >> 3) & 1) : idx);
        const I b = tile / (I)tiles_per_tensor;
        const I rem = tile - b * (I)tiles_per_tensor;
        const I tc = rem / (I)tiles_r, tr = rem - tc * (I)tiles_r;
        const int64_t r0 = (int64_t)tr * kTR, c0 = (int64_t)tc * kTC;
        return {(int64_t)b, r0, c0, (int)(rows - r0 < kTR ? rows - r0 : kTR), (int)(cols - c0 < kTC ? cols - c0 : kTC),
                tr == 0 && tc == 0};
    };
    // load phase operands: input rows (2p, 2p+1), columns [32h, 32h + 32)
    const int lp = 8 * wave + (lane >> 3), lh = lane & 7, lcl = 32 * lh;
    struct LRegs { uint32_t w[2][4]; uint32_t s[2]; };
    auto load = [&](int64_t idx, LRegs& R) {
#pragma unroll
        for (int rr = 0; rr < 2; ++rr) {
            R.w[rr][0] = R.w[rr][1] = R.w[rr][2] = R.w[rr][3] = 0;
            R.s[rr] = 0;
        }
        if (idx >= total_tiles)
            return;
        const Tile T = tile_of(idx);
        int nb = (T.cols_valid - lcl) / 16;
        nb = nb < 0 ? 0 : (nb > 2 ? 2 : nb);
        if (2 * lp < T.rows_valid && nb > 0) {
#pragma unroll
            for (int rr = 0; rr < 2; ++rr) {
                const int64_t grow = T.b * rows + T.r0 + 2 * lp + rr;
                const uint8_t* src = codes + (grow * cols + T.c0 + lcl) / 2;
                if (vec_in && nb == 2) {
                    const uint4 q = *reinterpret_cast<const uint4*>(src);
                    R.w[rr][0] = q.x; R.w[rr][1] = q.y; R.w[rr][2] = q.z; R.w[rr][3] = q.w;
                } else {
                    const uint2 q0 = *reinterpret_cast<const uint2*>(src);
                    R.w[rr][0] = q0.x; R.w[rr][1] = q0.y;
                    if (nb == 2) {
                        const uint2 q1 = reinterpret_cast<const uint2*>(src)[1];
                        R.w[rr][2] = q1.x; R.w[rr][3] = q1.y;
                    }
                }
                const uint8_t* sp = scales + grow * sc_pitch + (T.c0 + lcl) / 16;
                if (vec_scale_in && nb == 2) {
                    R.s[rr] = *reinterpret_cast<const uint16_t*>(sp);
                } else {
                    R.s[rr] = sp[0];
                    if (nb == 2)
                        R.s[rr] |= (uint32_t)sp[1] << 8;
                }
            }
        }
    };
    // -0, hidden from constant folding so that u * r' + (-0) stays one mixed-precision FMA
    // (its rounded value is that of the product u * r', sign of zero included)
    float neg_zero = -0.0f;
    asm("" : "+v"(neg_zero));
    LRegs R;
    load(blockIdx.x, R);
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): the first tile is needed at once, and no load
                                         // is then pending where the loop begins
    for (int64_t idx = blockIdx.x; idx < total_tiles; idx += gridDim.x) {
        const Tile T = tile_of(idx);
        const int64_t b = T.b, r0 = T.r0, c0 = T.c0;
        const int rows_valid = T.rows_valid, cols_valid = T.cols_valid;
        if (T.first && tid == 0)
            tensor_scale_t[b] = tensor_scale[b];

        // ---- exact dequant of the prefetched codes into LDS ----
        {
            const int p = lp, cl = lcl;
            sr_h2 d[2];
#pragma unroll
            for (int rr = 0; rr < 2; ++rr)  // both scale bytes by the exact E4M3 -> f16 decode
                d[rr] = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(R.s[rr], 1.0f, false);
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const sr_h2 da = {d[0][j >> 1], d[0][j >> 1]}, db = {d[1][j >> 1], d[1][j >> 1]};
                auto stage = [&](auto T) __attribute__((always_inline)) {  // columns 8j + 2t, 8j + 2t + 1
                    constexpr int t = decltype(T)::value;
                    const uint32_t wa = __builtin_bit_cast(uint32_t, fp4x2_to_h2<t>(R.w[0][j]) * da);
                    const uint32_t wb = __builtin_bit_cast(uint32_t, fp4x2_to_h2<t>(R.w[1][j]) * db);
                    u_s[lds_slot(cl + 8 * j + 2 * t, p)] = __builtin_amdgcn_perm(wb, wa, 0x05040100u);
                    u_s[lds_slot(cl + 8 * j + 2 * t + 1, p)] = __builtin_amdgcn_perm(wb, wa, 0x07060302u);
                };
                stage(std::integral_constant<int, 0>{});
                stage(std::integral_constant<int, 1>{});
                stage(std::integral_constant<int, 2>{});
                stage(std::integral_constant<int, 3>{});
            }
        }
        // the next tile's codes are in flight during this tile's requantization
        load(idx + gridDim.x, R);
        __syncthreads();

        // ---- requantize: thread -> output row c0 + c, input rows [64 half, 64 half + 64) ----
        {
            const int c = tid & (kTC - 1), half = tid >> 8, h = c >> 5;
            const int64_t oc = c0 + c;
            // Lanes past the tile's columns compute on the zeros staged there and store
            // nothing; no branch encloses the computation, so the wait below is on
            // every path.
            const bool active = c < cols_valid;
            uint32_t out[8] = {0, 0, 0, 0, 0, 0, 0, 0};
            uint32_t sc = 0;
            int nvalid = 0;
            // linear index / 16 of the output row's first element in this tile: the
            // Philox counter of block q is beta0 + q (rows is a multiple of 16)
            const uint64_t orow_first = ((uint64_t)b * (uint64_t)cols + (uint64_t)oc) * (uint64_t)rows +
                                        (uint64_t)(r0 + 64 * half);
            const uint64_t beta0 = orow_first / 16;
            {
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const int lr = 64 * half + 16 * q;  // first local input row of the block
                    out[2 * q] = out[2 * q + 1] = 0;
                    if (lr >= rows_valid)
                        continue;
                    ++nvalid;
                    // row pairs 8X .. 8X+7 of the block sit at 8 (X ^ (h >> 1)) + (t ^ 4 (h & 1))
                    const uint32_t* blk = u_s + c * kLdsStride + 8 * ((4 * half + q) ^ (h >> 1));
                    const uint4 v0 = *reinterpret_cast<const uint4*>(blk + 4 * (h & 1));
                    const uint4 v1 = *reinterpret_cast<const uint4*>(blk + 4 * ((h & 1) ^ 1));
                    const uint32_t pk[8] = {v0.x, v0.y, v0.z, v0.w, v1.x, v1.y, v1.z, v1.w};
                    sr_u16x2 am = {0, 0};
#pragma unroll
                    for (int i = 0; i < 8; ++i)
                        am = __builtin_elementwise_max(am, __builtin_bit_cast(sr_u16x2, pk[i] & 0x7FFF7FFFu));
                    const float A = (float)__builtin_bit_cast(_Float16, am[0] > am[1] ? am[0] : am[1]);
                    const BlockScale bs = block_scale(A);
                    sc |= bs.e << (8 * q);
                    const float rcp = bs.rcp;
                    const uint64_t beta = beta0 + (uint64_t)q;
                    const u32x4 rnd = philox4x32_10((uint32_t)beta, (uint32_t)(beta >> 32), 0u, 0u,
                                                    seed_lo, seed_hi);
                    const uint32_t rw[4] = {rnd.x, rnd.y, rnd.z, rnd.w};
                    float yc[16], k[16];
#pragma unroll
                    for (int i = 0; i < 16; ++i) {
                        const sr_h2 hv = __builtin_bit_cast(sr_h2, pk[i >> 1]);
                        yc[i] = __builtin_fmaf((float)hv[i & 1], rcp, neg_zero);
                        k[i] = (float)((rw[i >> 2] >> (8 * (i & 3))) & 0xFFu);
                    }
                    out[2 * q] = sr_pack8(yc, k);
                    out[2 * q + 1] = sr_pack8(yc + 8, k + 8);
                }
            }
            // The next tile's codes were loaded before this phase and have landed.  Waiting
            // for them here, on every path and before the stores, keeps the next dequant
            // from waiting on this tile's stores: the vector memory counter covers both.
            __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
            if (active) {
                uint8_t* orow = codes_t + orow_first / 2;
                uint8_t* srow = scales_t + (b * cols + oc) * sct_pitch + (r0 + 64 * half) / 16;
                if (nvalid == 4 && vec_out) {
                    reinterpret_cast<uint4*>(orow)[0] = make_uint4(out[0], out[1], out[2], out[3]);
                    reinterpret_cast<uint4*>(orow)[1] = make_uint4(out[4], out[5], out[6], out[7]);
                } else {
                    for (int q = 0; q < nvalid; ++q)
                        reinterpret_cast<uint2*>(orow)[q] = make_uint2(out[2 * q], out[2 * q + 1]);
                }
                if (nvalid == 4 && vec_scale_out) {
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
    // Persistent: each workgroup walks tiles, prefetching the next.  About six tiles per
    // workgroup, between 512 workgroups (one per resident slot: two per CU) and 8192; a
    // multiple of 8, so that tiles i and i + 8 stay on one XCD.  One MoE layer (3072 tiles)
    // took 66 us with one tile per workgroup and 61 us with six; launches of many layers
    // are fastest at 8192.
    int64_t g = total / 6 / 8 * 8;
    g = g < 512 ? 512 : (g > 8192 ? 8192 : g);
    g = g < total ? g : total;
    const int vec_in = cols % 32 == 0;
    const int vec_scale_in = cols % 32 == 0 && ((uintptr_t)scales & 1u) == 0;
    const int vec_out = rows % 32 == 0;
    const int vec_scale_out = rows % 64 == 0 && ((uintptr_t)scales_t & 3u) == 0;
    if (total + g < ((int64_t)1 << 32))
        hipLaunchKernelGGL(requant_transpose_sr_kernel<false>, dim3((unsigned)g), dim3(kSThreads), 0, s,
                           codes, scales, tensor_scale, batch, rows, cols, (uint32_t)seed,
                           (uint32_t)(seed >> 32), codes_t, scales_t, tensor_scale_t, tiles_r, tiles_c,
                           vec_in, vec_scale_in, vec_out, vec_scale_out);
    else
        hipLaunchKernelGGL(requant_transpose_sr_kernel<true>, dim3((unsigned)g), dim3(kSThreads), 0, s,
                           codes, scales, tensor_scale, batch, rows, cols, (uint32_t)seed,
                           (uint32_t)(seed >> 32), codes_t, scales_t, tensor_scale_t, tiles_r, tiles_c,
                           vec_in, vec_scale_in, vec_out, vec_scale_out);
}

}  // namespace tq
