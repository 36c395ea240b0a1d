// tq_mxfp8.hip - MXFP8 (E4M3 elements, one E8M0 scale per 32 values) for the
// backward: nearest quantization, and the NVFP4 -> MXFP8 transpose-requantize
// with stochastic rounding (gfx950).
//
// [TML] "싱킹 머신스 랩, 4비트 학습 기법 공개", summary box (MXFP8 backward with
// requantization and stochastic rounding), format-comparison paragraph (8.25
// bits per value: an 8-bit scale per 32 8-bit values) and forward/backward-
// mismatch paragraph.  Formats and readings in include/tq.h: the shared
// exponent of a block with maximum A > 0 is floor(log2 A) - 8, clamped to
// [-127, 127]; elements saturate at 448; zero is +0.
//
// Quantize: one lane per 32-value block (64 bytes of bf16 in, 32 code bytes and
// one scale byte out), E4M3 bytes from the packed hardware conversion.
// Transpose: tiles of 128 input rows x 256 input columns staged through LDS as
// in the NVFP4 transpose (as bf16 pairs here); each thread then owns one output
// row and two new blocks of 32 (its 64 values of the tile), with two
// Philox4x32-10 calls per block for the 32 random bytes, and the codes go back
// through the wave's own LDS rows so that four lanes store one row's 64 bytes.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "tq_device.hpp"
#include "tq_kernels.hpp"

namespace tq {

typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ u16x2 as_u16x2(uint32_t x) { return __builtin_bit_cast(u16x2, x); }
__device__ __forceinline__ uint32_t as_u32(u16x2 x) { return __builtin_bit_cast(uint32_t, x); }

// Shared exponent of a block with maximum magnitude A > 0: floor(log2 A) - 8,
// clamped to [-127, 127] (frexp handles subnormal A).
__device__ __forceinline__ int mx_shared_exp(float A)
{
    const int e = __builtin_amdgcn_frexp_expf(A) - 1 - 8;
    return e < -127 ? -127 : (e > 127 ? 127 : e);
}

// E4M3 bytes of y0..y3 (little-endian in one word): nearest, ties to even, saturating
// at 448, zero as +0, from gfx950's packed f32 -> E4M3 conversion (scale 1).  A device
// check over every finite binary32 input finds the conversion equal to that rule for
// |y| <= 464, except that it writes -0 (0x80) for negative values that round to zero,
// and NaN above 464.  So the values are clamped to +-448 first (the rule's
// saturation), and the sign bit of zero bytes is cleared: bit 7 of a byte is kept iff
// its low seven bits are nonzero (their sum with 0x7F carries into bit 7).
__device__ __forceinline__ uint32_t e4m3x4_nearest(float y0, float y1, float y2, float y3)
{
    typedef short s16x2 __attribute__((ext_vector_type(2)));
    auto clamp = [](float y) { return __builtin_amdgcn_fmed3f(y, -448.0f, 448.0f); };
    s16x2 r = {0, 0};
    r = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(r, clamp(y0), clamp(y1), 1.0f, false);
    r = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(r, clamp(y2), clamp(y3), 1.0f, true);
    const uint32_t w = __builtin_bit_cast(uint32_t, r);
    const uint32_t nz = (w & 0x7F7F7F7Fu) + 0x7F7F7F7Fu;
    return w & (nz | 0x7F7F7F7Fu);
}

// E4M3 stochastic rounding of a >= 0 with random byte k: floor grid point from
// the bits (3 mantissa bits from 2^-6 up, multiples of 2^-9 below), step up iff
// G_lo + k * step / 256 < a (all terms exact); a >= 448 gives 448.
__device__ __forceinline__ uint32_t e4m3_sr_code(float a, float k)
{
    if (a >= 448.0f)
        return 0x7Eu;
    uint32_t lo;
    float glo, q;  // q = spacing / 256
    if (a >= 0x1p-6f) {
        const uint32_t bits = __float_as_uint(a) & 0xFFF00000u;
        glo = __uint_as_float(bits);
        q = __uint_as_float((bits & 0x7F800000u) - ((3u + 8u) << 23));
        lo = ((((bits >> 23) & 0xFFu) - 120u) << 3) | ((bits >> 20) & 7u);
    } else {
        const float f = __builtin_floorf(a * 512.0f);  // exact: a * 2^9 and its floor
        glo = f * 0x1p-9f;
        q = 0x1p-17f;
        lo = (uint32_t)f;
    }
    return lo + ((glo + k * q < a) ? 1u : 0u);
}

template <bool BF16>
__global__ __launch_bounds__(256) void quantize_mxfp8_kernel(const void* __restrict__ x,
                                                             int64_t blocks, uint4* __restrict__ codes,
                                                             uint8_t* __restrict__ scales)
{
    for (int64_t blk = (int64_t)blockIdx.x * 256 + threadIdx.x; blk < blocks;
         blk += (int64_t)gridDim.x * 256) {
        float v[32];
        if (BF16) {
            const uint4* p = static_cast<const uint4*>(x) + 4 * blk;
#pragma unroll
            for (int h = 0; h < 4; ++h) {
                const uint4 q = p[h];
                const uint32_t w[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    v[8 * h + 2 * i] = bf16_lo(w[i]);
                    v[8 * h + 2 * i + 1] = bf16_hi(w[i]);
                }
            }
        } else {
            const float4* p = static_cast<const float4*>(x) + 8 * blk;
#pragma unroll
            for (int h = 0; h < 8; ++h) {
                const float4 q = p[h];
                v[4 * h] = q.x;
                v[4 * h + 1] = q.y;
                v[4 * h + 2] = q.z;
                v[4 * h + 3] = q.w;
            }
        }
        float A = 0.0f;
#pragma unroll
        for (int i = 0; i < 32; ++i)
            A = fmaxf(A, fabsf(v[i]));
        uint32_t w[8] = {0, 0, 0, 0, 0, 0, 0, 0};
        uint32_t sb = 0;
        if (A != 0.0f) {
            const int se = mx_shared_exp(A);
            sb = (uint32_t)(se + 127);
#pragma unroll
            for (int i = 0; i < 8; ++i)
                w[i] = e4m3x4_nearest(__builtin_ldexpf(v[4 * i], -se), __builtin_ldexpf(v[4 * i + 1], -se),
                                      __builtin_ldexpf(v[4 * i + 2], -se), __builtin_ldexpf(v[4 * i + 3], -se));
        }
        codes[2 * blk] = make_uint4(w[0], w[1], w[2], w[3]);
        codes[2 * blk + 1] = make_uint4(w[4], w[5], w[6], w[7]);
        scales[blk] = (uint8_t)sb;
    }
}

constexpr int kMTR = 128, kMTC = 256, kMThreads = 512, kMLdsStride = 68;

// LDS dword of tile column c, input row pair p: the row pair XOR 4 * chunk puts each
// half-wave's 32 stores of the load phase on 32 distinct banks (stores are served 32
// lanes at a time over 32 banks; c * 68 is one bank for all lanes of an instruction).
__device__ __forceinline__ int mlds_slot(int c, int p) { return c * kMLdsStride + (p ^ (4 * (c >> 5))); }

// Persistent: each workgroup walks a strided list of tiles and loads the next
// tile's codes and scales while it requantizes the current one.  WIDE: tile
// indices need 64 bits (otherwise the index arithmetic is done in 32 bits).
template <bool WIDE>
__global__ __launch_bounds__(kMThreads, 2) void requant_transpose_mxfp8_sr_kernel(
    const uint8_t* __restrict__ codes, const uint8_t* __restrict__ scales,
    const float* __restrict__ tensor_scale, int64_t batch, int64_t rows, int64_t cols,
    uint32_t seed_lo, uint32_t seed_hi, uint8_t* __restrict__ codes_t,
    uint8_t* __restrict__ scales_t, float* __restrict__ tensor_scale_t, int64_t tiles_r,
    int64_t tiles_c, int vec_in)
{
    __shared__ __attribute__((aligned(16))) uint32_t u_s[kMTC * kMLdsStride];
    const int64_t tiles_per_tensor = tiles_r * tiles_c;
    const int64_t total_tiles = tiles_per_tensor * batch;
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int64_t sc_pitch = cols / 16, sct_pitch = rows / 32;

    using I = typename std::conditional<WIDE, uint64_t, uint32_t>::type;
    struct Tile { int64_t b, r0, c0; int rows_valid, cols_valid; bool first; };
    auto tile_of = [&](int64_t tile_idx) -> Tile {
        const I tile = (I)tile_idx;
        const I b = tile / (I)tiles_per_tensor;
        const I rem = tile - b * (I)tiles_per_tensor;
        const I tc = rem / (I)tiles_r, tr = rem - tc * (I)tiles_r;
        const int64_t r0 = (int64_t)tr * kMTR, c0 = (int64_t)tc * kMTC;
        return {(int64_t)b, r0, c0, (int)(rows - r0 < kMTR ? rows - r0 : kMTR),  // multiples of 32
                (int)(cols - c0 < kMTC ? cols - c0 : kMTC), tr == 0 && tc == 0};  // multiples of 16
    };
    // load phase operands: input rows (2p, 2p+1), columns [32h, 32h + 32)
    const int lp = 8 * wave + (lane >> 3), lcl = 32 * (lane & 7);
    struct LRegs { uint32_t w[2][4]; uint32_t s[2]; };
    auto load = [&](int64_t tile_idx, LRegs& R) {
#pragma unroll
        for (int rr = 0; rr < 2; ++rr) {
            R.w[rr][0] = R.w[rr][1] = R.w[rr][2] = R.w[rr][3] = 0;
            R.s[rr] = 0;
        }
        if (tile_idx >= total_tiles)
            return;
        const Tile T = tile_of(tile_idx);
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
                R.s[rr] = sp[0];
                if (nb == 2)
                    R.s[rr] |= (uint32_t)sp[1] << 8;
            }
        }
    };
    LRegs R;
    load(blockIdx.x, R);
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): the first tile is needed at once, and no load
                                         // is then pending where the loop begins
    for (int64_t tile = blockIdx.x; tile < total_tiles; tile += gridDim.x) {
        const Tile T = tile_of(tile);
        const int64_t b = T.b, r0 = T.r0, c0 = T.c0;
        const int rows_valid = T.rows_valid, cols_valid = T.cols_valid;
        if (T.first && tid == 0)
            tensor_scale_t[b] = tensor_scale[b];

        // ---- exact dequant of the prefetched codes into LDS ----
        {
            const int p = lp, cl = lcl;
            float d[2][2];
#pragma unroll
            for (int rr = 0; rr < 2; ++rr) {  // both scale bytes by the exact E4M3 decode
                const tq_f32x2 dd = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(R.s[rr], 1.0f, false);
                d[rr][0] = dd[0];
                d[rr][1] = dd[1];
            }
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const float da = d[0][j >> 1], db = d[1][j >> 1];
                const tq_f32x2 a0 = fp4x2_to_f32<0>(R.w[0][j]), a1 = fp4x2_to_f32<1>(R.w[0][j]);
                const tq_f32x2 a2 = fp4x2_to_f32<2>(R.w[0][j]), a3 = fp4x2_to_f32<3>(R.w[0][j]);
                const tq_f32x2 b0 = fp4x2_to_f32<0>(R.w[1][j]), b1 = fp4x2_to_f32<1>(R.w[1][j]);
                const tq_f32x2 b2 = fp4x2_to_f32<2>(R.w[1][j]), b3 = fp4x2_to_f32<3>(R.w[1][j]);
                const float va[8] = {a0[0], a0[1], a1[0], a1[1], a2[0], a2[1], a3[0], a3[1]};
                const float vb[8] = {b0[0], b0[1], b1[0], b1[1], b2[0], b2[1], b3[0], b3[1]};
#pragma unroll
                for (int e = 0; e < 8; ++e)
                    u_s[mlds_slot(cl + 8 * j + e, p)] = pack_hi16(va[e] * da, vb[e] * db);
            }
        }
        // the next tile's codes are in flight during this tile's requantization
        load(tile + gridDim.x, R);
        __syncthreads();

        // ---- requantize: thread -> output row c0 + c, input rows [64 half, 64 half + 64) ----
        {
            const int c = tid & (kMTC - 1), half = tid >> 8, h = c >> 5;
            const int64_t oc = c0 + c;
            // Lanes past the tile's columns compute on the zeros staged there and store
            // nothing: no branch encloses the wait below, which is then on every path.
            const bool active = c < cols_valid;
            // This wave's lanes are 64 consecutive output rows (one half of each); its
            // LDS reads below touch only those rows' dwords [32 half, 32 half + 32), which
            // no other wave reads, so it stages its output codes there: piece p (16
            // bytes, input rows 64 half + 16 p ..) of row c at dword 8 (p ^ x), x = c >> 6
            // being the XOR the block reads use (uniform over the wave).  Block q's
            // pieces go where block q was read from, once it has been read.  Rows of 68
            // dwords put the staging writes (eight rows, one piece) and the read-back
            // (two rows, four pieces) on eight distinct 4-bank groups.
            uint32_t* const stage = u_s + c * kMLdsStride + 32 * half;
            const int xs = c >> 6;
            uint32_t sbq[2] = {0, 0};
            {
#pragma unroll
                for (int q = 0; q < 2; ++q) {
                    const int lr = 64 * half + 32 * q;  // first local input row of the block
                    const bool live = lr < rows_valid;
                    // the block's 32 staged values as bf16 pairs (a zero may carry a
                    // sign: -0 codes and zero scales stage as -0)
                    uint32_t pk[16];
#pragma unroll
                    for (int part = 0; part < 2; ++part) {
                        // row pairs 8X .. 8X+7 sit at 8 (X ^ (h >> 1)) + (t ^ 4 (h & 1))
                        const uint32_t* blk = u_s + c * kMLdsStride + 8 * ((4 * half + 2 * q + part) ^ (h >> 1));
                        const uint4 v0 = *reinterpret_cast<const uint4*>(blk + 4 * (h & 1));
                        const uint4 v1 = *reinterpret_cast<const uint4*>(blk + 4 * ((h & 1) ^ 1));
                        pk[8 * part + 0] = v0.x; pk[8 * part + 1] = v0.y;
                        pk[8 * part + 2] = v0.z; pk[8 * part + 3] = v0.w;
                        pk[8 * part + 4] = v1.x; pk[8 * part + 5] = v1.y;
                        pk[8 * part + 6] = v1.z; pk[8 * part + 7] = v1.w;
                    }
                    auto ubits = [&](int e) -> uint32_t {  // binary32 bits of element e
                        return (e & 1) ? (pk[e >> 1] & 0xFFFF0000u) : (pk[e >> 1] << 16);
                    };
                    // Every u is exact in bf16, so the low 16 bits of its binary32 pattern
                    // are zero and the integer steps below run on the 16-bit magnitude
                    // patterns |u|16, two per packed 16-bit instruction.  Block maximum (the
                    // integer order of |u| bits is the value order) and smallest nonzero
                    // |u|16, less one (a zero wraps to 0xFFFF).
                    u16x2 amax2 = {0, 0}, nzmin2 = {0xFFFF, 0xFFFF};
#pragma unroll
                    for (int j = 0; j < 16; ++j) {
                        const u16x2 a = as_u16x2(pk[j] & 0x7FFF7FFFu);
                        amax2 = __builtin_elementwise_max(amax2, a);
                        nzmin2 = __builtin_elementwise_min(nzmin2, a - (u16x2){1, 1});
                    }
                    const uint32_t Ab = (uint32_t)(amax2[0] > amax2[1] ? amax2[0] : amax2[1]) << 16;
                    const int64_t obase = (b * cols + oc) * rows + r0 + lr;  // output linear index
                    uint32_t wout[8] = {0, 0, 0, 0, 0, 0, 0, 0};
                    uint32_t sb = 0;
                    if (Ab != 0) {
                        const int se = mx_shared_exp(__uint_as_float(Ab));
                        sb = (uint32_t)(se + 127);
                        // Integer path, valid when every nonzero y = u * 2^-se is at
                        // least 2^-6 (E4M3 normal range).  With X = bits(|y|) -
                        // (120 << 23) = bits(|u|) - ((se + 120) << 23), the floor code
                        // is X >> 20 (exponent - 120, three mantissa bits) and the
                        // spacing above it is 2^20 units of X, so the step up
                        // (k < 256 * frac) is "X mod 2^20 > k * 2^12": one carry,
                        // (X + 2^20 - 1 - k * 2^12) >> 20.  Codes past 0x7E clamp
                        // (|y| >= 448 gives 448), and zeros give X = 0 and code 0.
                        // On 16-bit patterns, X = X16 << 16 with X16 = max(|u|16 - K16, 0)
                        // and K16 = (se + 120) << 7; X mod 2^20 is a multiple of 2^16, so
                        // only the high nibble kh of k decides the carry, and the code is
                        // (min(X16, 0x7E0) + 15 - kh) >> 4 (equal to the 32-bit form for
                        // every 16-bit pattern and byte, checked exhaustively).
                        const int kexp = se + 120;
                        const uint32_t nzmin = nzmin2[0] < nzmin2[1] ? nzmin2[0] : nzmin2[1];
                        const bool fast = kexp > 0 && nzmin >= ((uint32_t)(kexp + 1) << 7) - 1u;
                        const uint16_t K16 = (uint16_t)(kexp > 0 ? kexp << 7 : 0);
                        const u16x2 KK = {K16, K16};
#pragma unroll
                        for (int part = 0; part < 2; ++part) {
                            const uint64_t beta = (uint64_t)(obase / 16) + part;
                            const u32x4 rnd = philox4x32_10((uint32_t)beta, (uint32_t)(beta >> 32), 0u,
                                                            0u, seed_lo, seed_hi);
                            const uint32_t rw[4] = {rnd.x, rnd.y, rnd.z, rnd.w};
                            if (fast) {
#pragma unroll
                                for (int d = 0; d < 4; ++d) {  // elements 16 part + 4d .. + 3
                                    const int j0 = 8 * part + 2 * d;
                                    // 15 - kh of the four random bytes, one per byte
                                    const uint32_t T = ~(rw[d] >> 4) & 0x0F0F0F0Fu;
                                    uint32_t m[2];
#pragma unroll
                                    for (int t = 0; t < 2; ++t) {
                                        const u16x2 a = as_u16x2(pk[j0 + t] & 0x7FFF7FFFu);
                                        const u16x2 X = __builtin_elementwise_min(
                                            __builtin_elementwise_sub_sat(a, KK), (u16x2){0x7E0, 0x7E0});
                                        // bytes 2t and 2t + 1 of T into the two 16-bit lanes
                                        const u16x2 kh = as_u16x2(__builtin_amdgcn_perm(
                                            0u, T, t ? 0x0C030C02u : 0x0C010C00u));
                                        m[t] = as_u32((X + kh) >> (u16x2){4, 4});
                                    }
                                    // the four codes (low byte of each lane), and each value's
                                    // sign (bit 7 of bytes 1 and 3 of its pair) as bit 7, kept
                                    // for nonzero codes only (code + 0x7F carries into bit 7
                                    // iff the code is nonzero; codes are at most 0x7E)
                                    const uint32_t codes4 = __builtin_amdgcn_perm(m[1], m[0], 0x06040200u);
                                    const uint32_t sg = __builtin_amdgcn_perm(pk[j0 + 1], pk[j0], 0x07050301u) &
                                                        0x80808080u;
                                    wout[4 * part + d] = codes4 | (sg & (codes4 + 0x7F7F7F7Fu));
                                }
                            } else {
#pragma unroll
                                for (int i = 0; i < 16; ++i) {
                                    const int e = 16 * part + i;
                                    const float y = __builtin_ldexpf(__uint_as_float(ubits(e)), -se);
                                    const float k = (float)((rw[i >> 2] >> (8 * (i & 3))) & 0xFFu);
                                    const uint32_t m = e4m3_sr_code(fabsf(y), k);
                                    const uint32_t code = (y < 0.0f && m != 0u) ? (0x80u | m) : m;
                                    wout[e >> 2] |= code << (8 * (e & 3));
                                }
                            }
                        }
                    }
                    *reinterpret_cast<uint4*>(stage + 8 * ((2 * q) ^ xs)) =
                        make_uint4(wout[0], wout[1], wout[2], wout[3]);
                    *reinterpret_cast<uint4*>(stage + 8 * ((2 * q + 1) ^ xs)) =
                        make_uint4(wout[4], wout[5], wout[6], wout[7]);
                    sbq[q] = live ? sb : 0u;
                }
            }
            // Read the staged codes back so that four lanes write one row's 64 bytes
            // (16 rows per store instruction): lane l takes piece l % 4 of row
            // 16 j + l / 4 of the wave's 64.  LDS operations of one wave complete in
            // order; the fences keep the compiler from moving the reads above the writes.
            __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
            __builtin_amdgcn_wave_barrier();
            __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
            const int pl = lane & 3, cw = c - lane;  // cw: the wave's first row
            const bool live_p = 64 * half + 32 * (pl >> 1) < rows_valid;
            // The next tile's codes were loaded before this phase and have landed by
            // now.  Waiting for them here, before the first store and on every path,
            // keeps the next dequant from waiting on this tile's stores (the vector
            // memory counter covers both).
            __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
#pragma unroll
            for (int j = 0; j < 4; ++j) {  // one piece at a time: no registers held across
                const int cr = cw + 16 * j + (lane >> 2);
                const uint4 v = *reinterpret_cast<const uint4*>(u_s + cr * kMLdsStride + 32 * half + 8 * (pl ^ xs));
                if (cr < cols_valid && live_p)
                    *reinterpret_cast<uint4*>(codes_t + (b * cols + c0 + cr) * rows + r0 + 64 * half + 16 * pl) = v;
            }
            if (active) {
                uint8_t* srow = scales_t + (b * cols + oc) * sct_pitch + (r0 + 64 * half) / 32;
                if (64 * half < rows_valid)
                    srow[0] = (uint8_t)sbq[0];
                if (64 * half + 32 < rows_valid)
                    srow[1] = (uint8_t)sbq[1];
            }
        }
        __syncthreads();
    }
}

__global__ void mx_copy_scalars_kernel(const float* __restrict__ src, float* __restrict__ dst, int64_t n)
{
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n;
         i += (int64_t)gridDim.x * blockDim.x)
        dst[i] = src[i];
}

void launch_quantize_mxfp8(const void* x, bool bf16, int64_t n, uint8_t* codes, uint8_t* scales,
                           hipStream_t s)
{
    const int64_t blocks = n / 32;
    if (blocks == 0)
        return;
    int64_t g = (blocks + 255) / 256;
    g = g < (1 << 30) ? g : (1 << 30);  // one block per lane: see the streaming quantizers
    uint4* c4 = reinterpret_cast<uint4*>(codes);
    if (bf16)
        hipLaunchKernelGGL(quantize_mxfp8_kernel<true>, dim3((unsigned)g), dim3(256), 0, s, x, blocks,
                           c4, scales);
    else
        hipLaunchKernelGGL(quantize_mxfp8_kernel<false>, dim3((unsigned)g), dim3(256), 0, s, x, blocks,
                           c4, scales);
}

void launch_requant_transpose_mxfp8_sr(const uint8_t* codes, const uint8_t* scales,
                                       const float* tensor_scale, int64_t batch, int64_t rows,
                                       int64_t cols, uint64_t seed, uint8_t* codes_t,
                                       uint8_t* scales_t, float* tensor_scale_t, hipStream_t s)
{
    const int64_t tiles_r = (rows + kMTR - 1) / kMTR, tiles_c = (cols + kMTC - 1) / kMTC;
    const int64_t total = tiles_r * tiles_c * batch;
    if (total == 0) {
        if (batch > 0)
            hipLaunchKernelGGL(mx_copy_scalars_kernel, dim3(1), dim3(256), 0, s, tensor_scale,
                               tensor_scale_t, batch);
        return;
    }
    // Persistent: about six tiles per workgroup, between 512 workgroups (two per CU)
    // and 8192, so that each workgroup's loads of its next tile overlap the current one.
    int64_t g = total / 6 / 8 * 8;
    g = g < 512 ? 512 : (g > 8192 ? 8192 : g);
    g = g < total ? g : total;
    if (total + g < ((int64_t)1 << 32))
        hipLaunchKernelGGL(requant_transpose_mxfp8_sr_kernel<false>, dim3((unsigned)g), dim3(kMThreads),
                           0, s, codes, scales, tensor_scale, batch, rows, cols, (uint32_t)seed,
                           (uint32_t)(seed >> 32), codes_t, scales_t, tensor_scale_t, tiles_r, tiles_c,
                           (int)(cols % 32 == 0));
    else
        hipLaunchKernelGGL(requant_transpose_mxfp8_sr_kernel<true>, dim3((unsigned)g), dim3(kMThreads),
                           0, s, codes, scales, tensor_scale, batch, rows, cols, (uint32_t)seed,
                           (uint32_t)(seed >> 32), codes_t, scales_t, tensor_scale_t, tiles_r, tiles_c,
                           (int)(cols % 32 == 0));
}

}  // namespace tq
