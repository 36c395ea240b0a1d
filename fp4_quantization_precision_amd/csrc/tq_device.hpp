// tq_device.hpp - device-side number formats and Philox for libtq (gfx950).
//
// Formats: E2M1 element codes (4 bits, grid {0,0.5,1,1.5,2,3,4,6}, sign in bit 3)
// under an E4M3FN block scale per 16 values and an fp32 tensor scale ([TML]
// "싱킹 머신스 랩, 4비트 학습 기법 공개" summary box: 4.5 bits per value;
// forward/backward-mismatch paragraph: 16 consecutive values share a scale).
//
// All float arithmetic is plain IEEE binary32 (the library is built with
// -ffp-contract=off, denormals preserved and correctly rounded division), so
// every decision below is reproducible bit for bit.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace tq {

// ---------------------------------------------------------------------------
// E4M3FN block scales
// ---------------------------------------------------------------------------

// Value of a non-negative E4M3FN byte (0x00..0x7E).  Subnormals are M * 2^-9;
// normals (8 + M) * 2^(E - 10), built directly as binary32 bits.
__device__ __forceinline__ float e4m3_decode(uint32_t e)
{
    uint32_t E = (e >> 3) & 15u, M = e & 7u;
    float sub = (float)M * 0x1p-9f;  // exact
    float nrm = __uint_as_float(((E + 120u) << 23) | (M << 20));
    return E == 0 ? sub : nrm;
}

// E4M3FN encode of finite d >= 0: round to nearest, ties to even mantissa;
// d >= 448 saturates to 0x7E.  Below 2^-6 the spacing is 2^-9, so the code is
// rint(d * 512) (an exact scaling, then round-half-even); 8 there is 2^-6,
// which is also the code of the smallest normal.  From 2^-6 up the binary32
// mantissa is rounded to 3 bits with round-half-even on the bit pattern.
__device__ __forceinline__ uint32_t e4m3_encode(float d)
{
    if (d >= 448.0f)
        return 0x7Eu;
    if (d < 0x1p-6f)
        return (uint32_t)__builtin_rintf(d * 512.0f);
    uint32_t u = __float_as_uint(d);
    uint32_t r = (u + 0x7FFFFu + ((u >> 20) & 1u)) & 0xFFF00000u;
    uint32_t c = (((r >> 23) - 120u) << 3) | ((r >> 20) & 7u);
    return c > 0x7Eu ? 0x7Eu : c;
}

// ---------------------------------------------------------------------------
// E2M1 element codes
// ---------------------------------------------------------------------------

// Nearest magnitude index for a >= 0 with ties to the even index, saturating at
// 6: count the decision thresholds passed.  Midpoints that tie upward to an even
// index use >=, those that tie downward use >.
__device__ __forceinline__ uint32_t e2m1_nearest(float a)
{
    return (uint32_t)(a > 0.25f) + (uint32_t)(a >= 0.75f) + (uint32_t)(a > 1.25f) +
           (uint32_t)(a >= 1.75f) + (uint32_t)(a > 2.5f) + (uint32_t)(a >= 3.5f) +
           (uint32_t)(a > 5.0f);
}

// Largest index lo with G[lo] <= a (a >= 0).
__device__ __forceinline__ uint32_t e2m1_floor(float a)
{
    return (uint32_t)(a >= 0.5f) + (uint32_t)(a >= 1.0f) + (uint32_t)(a >= 1.5f) +
           (uint32_t)(a >= 2.0f) + (uint32_t)(a >= 3.0f) + (uint32_t)(a >= 4.0f) +
           (uint32_t)(a >= 6.0f);
}

// G[m] as binary32.
__device__ __forceinline__ float e2m1_value(uint32_t m)
{
    // m >= 2: exponent (m >> 1) - 1, mantissa bit m & 1; m = 1 is 0.5; m = 0 is 0.
    float v = __uint_as_float(((126u + (m >> 1)) << 23) | ((m & 1u) << 22));
    return m >= 2 ? v : (m == 1 ? 0.5f : 0.0f);
}

// Smallest index hi with G[hi] >= a, for 0 <= a <= 6.
__device__ __forceinline__ uint32_t e2m1_ceil(float a)
{
    return (uint32_t)(a > 0.0f) + (uint32_t)(a > 0.5f) + (uint32_t)(a > 1.0f) +
           (uint32_t)(a > 1.5f) + (uint32_t)(a > 2.0f) + (uint32_t)(a > 3.0f) +
           (uint32_t)(a > 4.0f);
}

// TRACE guided choice ([TRACE] "TRACE" explainer, paragraph after the rounding
// analogy): of the two grid points around a, take the one whose mantissa bit
// equals the rollout's hint bit h; grid points and a >= 6 are fixed.
__device__ __forceinline__ uint32_t e2m1_guided(float a, uint32_t h)
{
    if (a >= 6.0f)
        return 7u;
    uint32_t lo = e2m1_floor(a);
    uint32_t hi = e2m1_ceil(a);
    if (lo == hi)
        return lo;
    return ((lo & 1u) == h) ? lo : hi;
}

// Stochastic rounding between the two grid points around a with random byte k
// ([TML] forward/backward-mismatch paragraph, the 2.25 example): up iff
// k < 256 * (a - G[lo]) / (G[lo+1] - G[lo]).  The subtraction is exact
// (Sterbenz, or G[lo] = 0) and the division is by a power of two, so the
// threshold is exact and so is the comparison.
__device__ __forceinline__ uint32_t e2m1_sr(float a, uint32_t k)
{
    if (a >= 6.0f)
        return 7u;
    uint32_t lo = e2m1_floor(a);
    float glo = e2m1_value(lo);
    // 256 / (G[lo+1] - G[lo]): 512 below 2, 256 in [2, 4), 128 in [4, 6)
    float inv = lo < 4 ? 512.0f : (lo < 6 ? 256.0f : 128.0f);
    float t = (a - glo) * inv;
    return ((float)k < t) ? lo + 1u : lo;
}

// Sign and magnitude into a 4-bit code; zero is always +0.
__device__ __forceinline__ uint32_t e2m1_code(float y, uint32_t m)
{
    return m | ((y < 0.0f && m != 0u) ? 8u : 0u);
}

// ---------------------------------------------------------------------------
// Fast forms used by the kernels.  Each one is an exact re-expression of the
// rules above (checked bit for bit against the CPU oracle by the GPU tests).
// ---------------------------------------------------------------------------

// Eight nearest codes packed into one dword (element i in nibble i).  gfx950's
// v_cvt_scalef32_pk_fp4_f32 with scale 1 rounds to nearest even and saturates at
// 6 exactly like e2m1_nearest/e2m1_code for every finite binary32 input, except
// that it keeps the sign of a value that rounds to zero; the mask below turns
// every -0 nibble (code 8) into +0.
__device__ __forceinline__ uint32_t clear_negative_zero(uint32_t w)
{
    const uint32_t mag = w & 0x77777777u;
    const uint32_t nonzero = (mag + 0x77777777u) & 0x88888888u;  // bit 3 set iff magnitude != 0
    return mag | (w & nonzero);
}

__device__ __forceinline__ uint32_t pack8_nearest(const float y[8])
{
    uint32_t w = 0;
    w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, y[0], y[1], 1.0f, 0);
    w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, y[2], y[3], 1.0f, 1);
    w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, y[4], y[5], 1.0f, 2);
    w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, y[6], y[7], 1.0f, 3);
    return clear_negative_zero(w);
}

// Mantissa bits (m & 1) of eight packed codes, gathered into bits 0..7.
__device__ __forceinline__ uint32_t parity8(uint32_t w)
{
    uint32_t x = w & 0x11111111u;
    x = (x | (x >> 3)) & 0x03030303u;
    x = (x | (x >> 6)) & 0x000F000Fu;
    x = (x | (x >> 12)) & 0x000000FFu;
    return x;
}

typedef float tq_f32x2 __attribute__((ext_vector_type(2)));

// The two signed E2M1 values of byte `sel` (0..3) of w (low nibble first):
// v_cvt_scalef32_pk_f32_fp4 with scale 1 is exact for all 256 byte values.
template <int SEL>
__device__ __forceinline__ tq_f32x2 fp4x2_to_f32(uint32_t w)
{
    return __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, SEL);
}

// High halves of two binary32 values as one dword (lo from a, hi from b).  Used
// for values whose low 16 bits are zero (exact bf16).
__device__ __forceinline__ uint32_t pack_hi16(float a, float b)
{
    return __builtin_amdgcn_perm(__float_as_uint(b), __float_as_uint(a), 0x07060302u);
}

// Floor grid index of a >= 0 from its bits: above 1 the grid is a binary float
// with one mantissa bit, so lo = (bits >> 22) - 252 (the exponent and the top
// mantissa bit); [0.5, 1) gives 1 and [0, 0.5) gives 0; clamped to 7.
__device__ __forceinline__ uint32_t e2m1_floor_bits(float a)
{
    const int b = (int)(__float_as_uint(a) >> 22) - 252;
    const int lo = b > (int)(a >= 0.5f) ? b : (int)(a >= 0.5f);
    return (uint32_t)(lo < 7 ? lo : 7);
}

// e2m1_guided without compare chains: a is on the grid iff the bits below the
// grid's resolution are zero (22 mantissa bits above 1, 23 in [0.5, 1), all of
// them below 0.5).  Off the grid the bracket is (lo, lo+1) and the hint picks
// the end with its parity: lo + ((lo ^ h) & 1).  a >= 6 gives 7.
__device__ __forceinline__ uint32_t e2m1_guided_bits(float a, uint32_t h)
{
    const uint32_t bits = __float_as_uint(a);
    const uint32_t lo = e2m1_floor_bits(a);
    const uint32_t mask = a >= 1.0f ? 0x3FFFFFu : (a >= 0.5f ? 0x7FFFFFu : 0x7FFFFFFFu);
    const bool on_grid = (bits & mask) == 0u;
    const uint32_t m = on_grid ? lo : lo + ((lo ^ h) & 1u);
    return m < 7u ? m : 7u;
}

// e2m1_sr without compare chains: up iff k < 256 (a - G[lo]) / D with
// D = G[lo+1] - G[lo], i.e. iff G[lo] + k * (D / 256) < a, where G[lo] (at most
// two significant bits) plus k * D / 256 (at most eight) is exact in binary32.
// D / 256 is 2^-9 below 2, 2^-8 in [2, 4) and 2^-7 from 4; a >= 6 gives 7.
__device__ __forceinline__ uint32_t e2m1_sr_bits(float a, float k)
{
    const uint32_t lo = e2m1_floor_bits(a);
    const float glo = lo >= 2u ? __uint_as_float((lo + 252u) << 22) : (lo == 1u ? 0.5f : 0.0f);
    const float q = lo < 4u ? 0x1p-9f : (lo < 6u ? 0x1p-8f : 0x1p-7f);
    const uint32_t m = lo + ((glo + k * q < a) ? 1u : 0u);
    return m < 7u ? m : 7u;
}

// ---------------------------------------------------------------------------
// bf16 helpers
// ---------------------------------------------------------------------------

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// ---------------------------------------------------------------------------
// Philox4x32-10 (Salmon, Moraes, Dror, Shaw, SC'11)
// ---------------------------------------------------------------------------

struct u32x4 {
    uint32_t x, y, z, w;
};

__device__ __forceinline__ u32x4 philox4x32_10(uint32_t c0, uint32_t c1, uint32_t c2,
                                               uint32_t c3, uint32_t k0, uint32_t k1)
{
#pragma unroll
    for (int r = 0; r < 10; ++r) {
        if (r > 0) {
            k0 += 0x9E3779B9u;
            k1 += 0xBB67AE85u;
        }
        uint64_t p0 = (uint64_t)0xD2511F53u * c0;
        uint64_t p1 = (uint64_t)0xCD9E8D57u * c2;
        // three-way XORs as single v_bitop3_b32 (truth table 0x96)
        uint32_t n0 = __builtin_amdgcn_bitop3_b32((uint32_t)(p1 >> 32), c1, k0, 0x96);
        uint32_t n2 = __builtin_amdgcn_bitop3_b32((uint32_t)(p0 >> 32), c3, k1, 0x96);
        c1 = (uint32_t)p1;
        c3 = (uint32_t)p0;
        c0 = n0;
        c2 = n2;
    }
    return {c0, c1, c2, c3};
}

}  // namespace tq
