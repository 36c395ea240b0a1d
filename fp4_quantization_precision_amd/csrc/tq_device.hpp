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

// G[m] as binary32.
__device__ __forceinline__ float e2m1_value(uint32_t m)
{
    // m >= 2: exponent (m >> 1) - 1, mantissa bit m & 1; m = 1 is 0.5; m = 0 is 0.
    float v = __uint_as_float(((126u + (m >> 1)) << 23) | ((m & 1u) << 22));
    return m >= 2 ? v : (m == 1 ? 0.5f : 0.0f);
}

// The rounding rules the kernels implement, for a = |y| on the grid G above:
//  nearest: the grid point nearest to a, ties to the even index, a > 5 -> 6;
//  guided ([TRACE] "TRACE" explainer, paragraph after the rounding analogy):
//    a >= 6 -> 6; a on the grid keeps its index lo; otherwise the one of lo and
//    lo + 1 whose mantissa bit (index & 1) equals the hint bit;
//  stochastic ([TML] forward/backward-mismatch paragraph, the 2.25 example):
//    a >= 6 -> 6; otherwise lo + 1 iff k < 256 (a - G[lo]) / (G[lo+1] - G[lo])
//    for the element's random byte k (exact: the subtraction is exact and the
//    divisor a power of two).
// A code is the magnitude index plus 8 for y < 0; zero is always +0.

// ---------------------------------------------------------------------------
// Packed forms used by the kernels.  Each one is an exact re-expression of the
// rules above (checked bit for bit against the CPU oracle by the GPU tests).
// ---------------------------------------------------------------------------

// Eight nearest codes packed into one dword (element i in nibble i).  gfx950's
// v_cvt_scalef32_pk_fp4_f32 with scale 1 rounds to nearest even and saturates at
// 6 exactly like the nearest rule for every finite binary32 input, except
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

// Byte SEL of `w` <- the two floor codes of (a, b): v_cvt_scalef32_sr_pk_fp4_f32
// with a zero seed and unit scale truncates each value to the grid toward zero
// (sign kept) and leaves the other three bytes of the destination unchanged.
// Written in asm because the compiler does not treat this destination as tied
// to its previous value; a byte-selected write needs one wait state before the
// register is read again (the s_nop the compiler puts after such writes).
template <int SEL>
__device__ __forceinline__ uint32_t floor_pk_fp4(uint32_t w, float a, float b)
{
    typedef float f2 __attribute__((ext_vector_type(2)));
    const f2 v = {a, b};
    if (SEL == 0)
        asm("v_cvt_scalef32_sr_pk_fp4_f32 %0, %1, 0, 1.0" : "+v"(w) : "v"(v));
    else if (SEL == 1)
        asm("v_cvt_scalef32_sr_pk_fp4_f32 %0, %1, 0, 1.0 op_sel:[0,0,1,0]\n\ts_nop 0" : "+v"(w) : "v"(v));
    else if (SEL == 2)
        asm("v_cvt_scalef32_sr_pk_fp4_f32 %0, %1, 0, 1.0 op_sel:[0,0,0,1]\n\ts_nop 0" : "+v"(w) : "v"(v));
    else
        asm("v_cvt_scalef32_sr_pk_fp4_f32 %0, %1, 0, 1.0 op_sel:[0,0,1,1]\n\ts_nop 0" : "+v"(w) : "v"(v));
    return w;
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

// Bits 0..7 of h spread to bit 0 of nibbles 0..7 (the inverse of parity8).
__device__ __forceinline__ uint32_t spread8(uint32_t h)
{
    uint32_t x = h & 0xFFu;
    x = (x | (x << 12)) & 0x000F000Fu;
    x = (x | (x << 6)) & 0x03030303u;
    x = (x | (x << 3)) & 0x11111111u;
    return x;
}

// Eight guided codes packed into one dword (element i in nibble i), hint bit i
// in bit i of h: the guided rule on values clamped to [-6, 6] (which
// leaves every decision unchanged and makes a >= 6 an on-grid 6).  Floor codes
// come from the hardware truncation; off the grid the code steps up by one
// exactly when the floor's mantissa bit differs from the hint.
__device__ __forceinline__ uint32_t pack8_guided(const float y[8], uint32_t h)
{
    float yc[8];
#pragma unroll
    for (int i = 0; i < 8; ++i)
        yc[i] = __builtin_amdgcn_fmed3f(y[i], -6.0f, 6.0f);
    uint32_t P = 0;
    P = floor_pk_fp4<0>(P, yc[0], yc[1]);
    P = floor_pk_fp4<1>(P, yc[2], yc[3]);
    P = floor_pk_fp4<2>(P, yc[4], yc[5]);
    P = floor_pk_fp4<3>(P, yc[6], yc[7]);
    const tq_f32x2 g0 = fp4x2_to_f32<0>(P), g1 = fp4x2_to_f32<1>(P);
    const tq_f32x2 g2 = fp4x2_to_f32<2>(P), g3 = fp4x2_to_f32<3>(P);
    const float g[8] = {g0[0], g0[1], g1[0], g1[1], g2[0], g2[1], g3[0], g3[1]};
    uint32_t off = 0;
#pragma unroll
    for (int i = 0; i < 8; ++i)
        off |= (fabsf(g[i]) != fabsf(yc[i])) ? (1u << (4 * i)) : 0u;
    const uint32_t up = (P ^ spread8(h)) & off;  // bit 0 of each nibble
    return clear_negative_zero(P + up);
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
