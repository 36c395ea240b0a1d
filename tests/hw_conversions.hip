// hw_conversions.hip - device checks of the gfx950 conversions and arithmetic shortcuts
// that the libtq kernels rely on, each over its whole input domain.
//
// TEST INFRASTRUCTURE.  Built by __graft_entry__.build() into tests/libtq_hwcheck.so and
// run by tests/test_hw_conversions.py.  The reference side of every check is written
// here from the definition of the rule (grids, midpoints, ties to the even code), in
// fp64 where a difference has to be exact; nothing is shared with the library or the
// oracle.
//
// Each check counts mismatches into counts[0] (and, where a second class is reported,
// counts[1]) and records the first mismatching input in first[1..3] (first[0] is a
// claim flag).
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

namespace {

typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef short s16x2 __attribute__((ext_vector_type(2)));

// E2M1 magnitudes (index 0..7) and the midpoints between neighbours
__device__ const float kG[8] = {0.0f, 0.5f, 1.0f, 1.5f, 2.0f, 3.0f, 4.0f, 6.0f};
__device__ const float kMid[7] = {0.25f, 0.75f, 1.25f, 1.75f, 2.5f, 3.5f, 5.0f};

// nearest index of a >= 0: above every midpoint below it; a tie takes the even index
__device__ int e2m1_nearest_index(float a)
{
    int idx = 0;
    for (int i = 0; i < 7; ++i) {
        if (a > kMid[i]) {
            idx = i + 1;
        } else {
            if (a == kMid[i])
                idx = (i % 2 == 0) ? i : i + 1;
            break;
        }
    }
    return idx;
}

// largest index whose grid value is <= a (a >= 0)
__device__ int e2m1_floor_index(float a)
{
    int idx = 0;
    for (int i = 1; i < 8; ++i)
        if (kG[i] <= a)
            idx = i;
    return idx;
}

// value of an E4M3FN byte as double (NaN for the two NaN codes)
__device__ double e4m3_value(uint32_t b)
{
    const uint32_t E = (b >> 3) & 15u, M = b & 7u;
    if (E == 15u && M == 7u)
        return __longlong_as_double(0x7FF8000000000000ll);
    const double v = E == 0u ? ldexp((double)M, -9) : ldexp(1.0 + M / 8.0, (int)E - 7);
    return (b & 0x80u) ? -v : v;
}

// nearest E4M3 magnitude code of 0 <= a <= 464 (448 from 448 up): binary search for the largest code whose
// value is <= a, then the nearer of it and the next code, a tie taking the even code
__device__ uint32_t e4m3_nearest_code(float a)
{
    uint32_t lo = 0, hi = 0x7E;
    while (lo < hi) {
        const uint32_t mid = (lo + hi + 1) / 2;
        if (e4m3_value(mid) <= (double)a)
            lo = mid;
        else
            hi = mid - 1;
    }
    if (lo == 0x7E)
        return lo;
    const double dl = (double)a - e4m3_value(lo), du = e4m3_value(lo + 1) - (double)a;
    if (dl < du)
        return lo;
    if (du < dl)
        return lo + 1;
    return (lo & 1u) ? lo + 1 : lo;
}

__device__ void record(uint32_t* first, uint32_t a, uint32_t b, uint32_t c)
{
    if (atomicCAS(first, 0u, 1u) == 0u) {
        first[1] = a;
        first[2] = b;
        first[3] = c;
    }
}

__device__ bool finite_bits(uint32_t u) { return ((u >> 23) & 0xFFu) != 0xFFu; }

// v_cvt_scalef32_pk_fp4_f32, scale 1: the E2M1 nearest code with the sign of x
__global__ void k_fp4_nearest(unsigned long long* counts, uint32_t* first)
{
    unsigned long long bad = 0;
    for (uint64_t i = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x; i < (1ull << 31);
         i += (uint64_t)gridDim.x * blockDim.x) {
        const uint32_t u0 = (uint32_t)(2 * i), u1 = u0 + 1;
        const float x0 = __uint_as_float(u0), x1 = __uint_as_float(u1);
        const uint32_t hw = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(0u, x0, x1, 1.0f, 0) & 0xFFu;
        const uint32_t u[2] = {u0, u1};
        for (int j = 0; j < 2; ++j) {
            if (!finite_bits(u[j]))
                continue;
            const float x = __uint_as_float(u[j]);
            const uint32_t ref = ((u[j] >> 31) << 3) | (uint32_t)e2m1_nearest_index(fabsf(x));
            const uint32_t got = (hw >> (4 * j)) & 0xFu;
            if (got != ref) {
                ++bad;
                record(first, u[j], got, ref);
            }
        }
    }
    atomicAdd(counts, bad);
}

// v_cvt_scalef32_sr_pk_fp4_f32 with a zero seed, scale 1: the floor index of |x| (6 and
// above give 6) with the sign of x
__global__ void k_fp4_floor(unsigned long long* counts, uint32_t* first)
{
    unsigned long long bad = 0;
    for (uint64_t i = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x; i < (1ull << 31);
         i += (uint64_t)gridDim.x * blockDim.x) {
        const uint32_t u0 = (uint32_t)(2 * i), u1 = u0 + 1;
        const f32x2 v = {__uint_as_float(u0), __uint_as_float(u1)};
        const uint32_t hw = __builtin_amdgcn_cvt_scalef32_sr_pk_fp4_f32(0u, v, 0u, 1.0f, 0) & 0xFFu;
        const uint32_t u[2] = {u0, u1};
        for (int j = 0; j < 2; ++j) {
            if (!finite_bits(u[j]))
                continue;
            const uint32_t ref = ((u[j] >> 31) << 3) | (uint32_t)e2m1_floor_index(fabsf(__uint_as_float(u[j])));
            const uint32_t got = (hw >> (4 * j)) & 0xFu;
            if (got != ref) {
                ++bad;
                record(first, u[j], got, ref);
            }
        }
    }
    atomicAdd(counts, bad);
}

// v_cvt_scalef32_pk_f32_fp4 on all 256 bytes, at scale 1 and at scale 2^-9: +-G[m] * scale
__global__ void k_fp4_decode(unsigned long long* counts, uint32_t* first)
{
    const uint32_t b = threadIdx.x;  // 0..255
    const float scales[2] = {1.0f, 0x1p-9f};
    for (int s = 0; s < 2; ++s) {
        const f32x2 hw = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(b, scales[s], 0);
        for (int j = 0; j < 2; ++j) {
            const uint32_t c = (b >> (4 * j)) & 0xFu;
            const float ref = ((c & 8u) ? -kG[c & 7u] : kG[c & 7u]) * scales[s];
            if (!(hw[j] == ref) || (ref != 0.0f && __float_as_uint(hw[j]) != __float_as_uint(ref))) {
                atomicAdd(counts, 1ull);
                record(first, b | (uint32_t)(s << 8), __float_as_uint(hw[j]), __float_as_uint(ref));
            }
        }
    }
}

// v_cvt_scalef32_pk_f32_fp8 on all 65536 byte pairs: the E4M3 values (NaN codes give NaN)
__global__ void k_fp8_decode(unsigned long long* counts, uint32_t* first)
{
    const uint32_t w = blockIdx.x * blockDim.x + threadIdx.x;  // 0..65535
    const f32x2 hw = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(w, 1.0f, false);
    for (int j = 0; j < 2; ++j) {
        const uint32_t b = (w >> (8 * j)) & 0xFFu;
        const double ref = e4m3_value(b);
        const bool ok = isnan(ref) ? isnan(hw[j]) : ((double)hw[j] == ref && signbit(hw[j]) == signbit(ref));
        if (!ok) {
            atomicAdd(counts, 1ull);
            record(first, w, __float_as_uint(hw[j]), b);
        }
    }
}

// v_cvt_scalef32_pk_fp8_f32, scale 1: for |y| <= 464 the nearest E4M3 code (ties to the
// even code; 448 < |y| <= 464 rounds to 448) with the sign of y; counts[1] counts
// |y| > 464 (where the rule saturates at 448) that do not give NaN
__global__ void k_fp8_nearest(unsigned long long* counts, uint32_t* first)
{
    unsigned long long bad = 0, big_not_nan = 0;
    for (uint64_t i = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x; i < (1ull << 31);
         i += (uint64_t)gridDim.x * blockDim.x) {
        const uint32_t u0 = (uint32_t)(2 * i), u1 = u0 + 1;
        const s16x2 r = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(s16x2{0, 0}, __uint_as_float(u0),
                                                                 __uint_as_float(u1), 1.0f, false);
        const uint32_t hw = (uint32_t)(uint16_t)r.x;
        const uint32_t u[2] = {u0, u1};
        for (int j = 0; j < 2; ++j) {
            if (!finite_bits(u[j]))
                continue;
            const float a = fabsf(__uint_as_float(u[j]));
            const uint32_t got = (hw >> (8 * j)) & 0xFFu;
            if (a > 464.0f) {
                if ((got & 0x7Fu) != 0x7Fu)
                    ++big_not_nan;
                continue;
            }
            const uint32_t ref = ((u[j] >> 31) << 7) | e4m3_nearest_code(a);
            if (got != ref) {
                ++bad;
                record(first, u[j], got, ref);
            }
        }
    }
    atomicAdd(counts, bad);
    atomicAdd(counts + 1, big_not_nan);
}

// A / 6 as A * RN(1/6) with one FMA correction, against the correctly rounded quotient
// (fp64 quotient rounded once to binary32: A / 6 never lies exactly on a binary32
// midpoint, so the double rounding is exact), for A = 0 and every finite A >= 2^-125
__global__ void k_div6(unsigned long long* counts, uint32_t* first)
{
    unsigned long long bad = 0;
    const float c = 1.0f / 6.0f;
    for (uint64_t i = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x; i < 0x7F800000ull;
         i += (uint64_t)gridDim.x * blockDim.x) {
        const uint32_t u = (uint32_t)i;
        if (u != 0u && u < 0x01000000u)
            continue;
        const float A = __uint_as_float(u);
        const float q0 = A * c;
        const float q = __builtin_fmaf(__builtin_fmaf(-q0, 6.0f, A), c, q0);
        const float ref = (float)((double)A / 6.0);
        if (__float_as_uint(q) != __float_as_uint(ref)) {
            ++bad;
            record(first, u, __float_as_uint(q), __float_as_uint(ref));
        }
    }
    atomicAdd(counts, bad);
}

// 1 / d as v_rcp_f32 plus one Newton step, against the correctly rounded reciprocal, for
// the 126 nonzero finite E4M3 values d; counts[1] counts those where v_rcp_f32 alone differs
__global__ void k_rcp_e4m3(unsigned long long* counts, uint32_t* first)
{
    const uint32_t b = threadIdx.x + 1;  // 1..126
    if (b > 0x7Eu)
        return;
    const float d = (float)e4m3_value(b);
    const float r0 = __builtin_amdgcn_rcpf(d);
    const float r = __builtin_fmaf(__builtin_fmaf(-d, r0, 1.0f), r0, r0);
    const float ref = (float)(1.0 / (double)d);
    if (__float_as_uint(r) != __float_as_uint(ref)) {
        atomicAdd(counts, 1ull);
        record(first, b, __float_as_uint(r), __float_as_uint(ref));
    }
    if (__float_as_uint(r0) != __float_as_uint(ref))
        atomicAdd(counts + 1, 1ull);
}

typedef _Float16 h16x2 __attribute__((ext_vector_type(2)));

// v_cvt_scalef32_pk_f16_fp4 (scale 1) on all 256 bytes, in each of the four byte
// positions of the source word: +-G[m] as binary16, -0 for the code of -0
template <int S>
__device__ void fp4_f16_one(uint32_t b, unsigned long long* counts, uint32_t* first)
{
    const h16x2 hw = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(b << (8 * S), 1.0f, S);
    for (int j = 0; j < 2; ++j) {
        const uint32_t c = (b >> (4 * j)) & 0xFu;
        const float ref = (c & 8u) ? -kG[c & 7u] : kG[c & 7u];
        const float got = (float)hw[j];
        if (!(got == ref) || signbit(got) != signbit(ref)) {
            atomicAdd(counts, 1ull);
            record(first, b | (uint32_t)(S << 8), __float_as_uint(got), __float_as_uint(ref));
        }
    }
}
__global__ void k_fp4_decode_f16(unsigned long long* counts, uint32_t* first)
{
    const uint32_t b = threadIdx.x;  // 0..255
    fp4_f16_one<0>(b, counts, first);
    fp4_f16_one<1>(b, counts, first);
    fp4_f16_one<2>(b, counts, first);
    fp4_f16_one<3>(b, counts, first);
}

// v_cvt_scalef32_pk_f16_fp8 (scale 1) on all 65536 byte pairs: the E4M3 values as
// binary16 (every finite E4M3 value is one), NaN codes give NaN
__global__ void k_fp8_decode_f16(unsigned long long* counts, uint32_t* first)
{
    const uint32_t w = blockIdx.x * blockDim.x + threadIdx.x;  // 0..65535
    const h16x2 hw = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w, 1.0f, false);
    for (int j = 0; j < 2; ++j) {
        const uint32_t b = (w >> (8 * j)) & 0xFFu;
        const double ref = e4m3_value(b);
        const float got = (float)hw[j];
        const bool ok = isnan(ref) ? isnan(got) : ((double)got == ref && signbit(got) == signbit(ref));
        if (!ok) {
            atomicAdd(counts, 1ull);
            record(first, w, __float_as_uint(got), b);
        }
    }
}

// For every signed E2M1 code m (16) and E4M3 scale byte e (0..0x7E): the binary16
// product G[m] * dec(e) from v_pk_mul_f16 is exact (checked in fp64), and for each
// reciprocal r = 1/dec(e') that the SR kernel uses (the correctly rounded one, and 0
// for e' = 0) the mixed-precision FMA of that f16 value, r and -0 equals the binary32
// product RN(u * r) with its sign of zero (the fp64 product is exact, so rounding it
// once to binary32 is the correctly rounded product).  counts[1] counts f16 products
// that are not exact.
__global__ void k_f16_scale_products(unsigned long long* counts, uint32_t* first)
{
    const uint32_t m = threadIdx.x & 15u, e = blockIdx.x;  // e: 0..126
    const float G = (m & 8u) ? -kG[m & 7u] : kG[m & 7u];
    const double dec = e4m3_value(e);
    const h16x2 g2 = {(_Float16)G, (_Float16)-G};
    const h16x2 d2 = {(_Float16)dec, (_Float16)dec};
    const uint32_t uw = __builtin_bit_cast(uint32_t, g2 * d2);  // both halves: +-G * dec
    for (int j = 0; j < 2; ++j) {
        const double exact = (j ? -(double)G : (double)G) * dec;
        const float got = (float)__builtin_bit_cast(h16x2, uw)[j];
        if ((double)got != exact || signbit(got) != signbit(exact)) {
            atomicAdd(counts + 1, 1ull);
            record(first, (m << 8) | e, __float_as_uint(got), 0xFFFFFFFFu);
        }
    }
    float neg_zero = -0.0f;
    asm("" : "+v"(neg_zero));
    for (uint32_t e2 = threadIdx.x >> 4; e2 <= 0x7Eu; e2 += blockDim.x >> 4) {
        const double d = e4m3_value(e2);
        const float r = e2 == 0u ? 0.0f : (float)(1.0 / d);
        uint32_t uwl = uw;
        asm("" : "+v"(uwl));  // keeps the f16 -> f32 step inside the FMA, as in the kernel
        const h16x2 hv = __builtin_bit_cast(h16x2, uwl);
        const float y[2] = {__builtin_fmaf((float)hv[0], r, neg_zero), __builtin_fmaf((float)hv[1], r, neg_zero)};
        for (int j = 0; j < 2; ++j) {
            const double exact = (j ? -(double)G : (double)G) * dec;
            const float ref = (float)(exact * (double)r);
            if (__float_as_uint(y[j]) != __float_as_uint(ref)) {
                atomicAdd(counts, 1ull);
                record(first, (j << 24) | (m << 16) | (e << 8) | e2, __float_as_uint(y[j]), __float_as_uint(ref));
            }
        }
    }
}

}  // namespace

#define HWC_ENTRY(name, kernel, grid, block)                                                      \
    extern "C" __attribute__((visibility("default"))) int name(unsigned long long* counts,          \
                                                               uint32_t* first)                  \
    {                                                                                              \
        hipLaunchKernelGGL(kernel, dim3(grid), dim3(block), 0, 0, counts, first);                  \
        return (int)hipDeviceSynchronize();                                                        \
    }

HWC_ENTRY(hwc_fp4_nearest, k_fp4_nearest, 65536, 256)
HWC_ENTRY(hwc_fp4_floor, k_fp4_floor, 65536, 256)
HWC_ENTRY(hwc_fp4_decode, k_fp4_decode, 1, 256)
HWC_ENTRY(hwc_fp8_decode, k_fp8_decode, 256, 256)
HWC_ENTRY(hwc_fp8_nearest, k_fp8_nearest, 65536, 256)
HWC_ENTRY(hwc_div6, k_div6, 65536, 256)
HWC_ENTRY(hwc_rcp_e4m3, k_rcp_e4m3, 1, 128)
HWC_ENTRY(hwc_fp4_decode_f16, k_fp4_decode_f16, 1, 256)
HWC_ENTRY(hwc_fp8_decode_f16, k_fp8_decode_f16, 256, 256)
HWC_ENTRY(hwc_f16_scale_products, k_f16_scale_products, 127, 256)
