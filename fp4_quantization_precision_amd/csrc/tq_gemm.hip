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
// Work decomposition.  One workgroup (4 waves) computes a kBM x kBN = 128 x 256
// output tile of one group (expert); each wave owns a 64 x 128 sub-tile of 2 x 4
// MFMA 32x32x16 tiles, which reads 0.75 KiB of LDS fragments per MFMA (1 KiB at
// 64 x 64); LDS fragment bandwidth, not the MFMA rate, is what bounds this loop.
// The tile list is derived on the device from the group offsets (a wave-wide
// prefix sum of per-group tile counts), so no host synchronisation is needed.
// Consecutive workgroup ids are dealt round-robin to the 8 XCDs; the id -> tile
// map undoes that, so each XCD walks a contiguous run of tiles in (M-tile,
// N-tile) order and the N-tiles of one M-tile share their activation rows
// through that XCD's L2.
//
// Pipeline.  The K loop is software-pipelined through registers: the global
// loads of K-slice s+1 (activations, weight codes, block scales) are issued
// before the MFMAs of slice s and only written to LDS (activations as is,
// weights dequantized with gfx950's packed FP4 -> f32 conversion) after them.
// All operand loads are buffer loads against per-workgroup resources: the
// per-thread byte offsets are fixed for the whole K loop and the slice position
// is a scalar offset, so the loop spends no vector instructions on addresses,
// and rows past the end of A or W read as zeros in hardware (such rows only
// feed output rows or columns that are never stored).  Only a partial last
// K-slice (K not a multiple of 64) masks its loads in registers.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "tq_device.hpp"
#include "tq_kernels.hpp"

namespace tq {

#ifndef TQ_GEMM_BN
#define TQ_GEMM_BN 256
#endif
constexpr int kBM = 128, kBN = TQ_GEMM_BN, kBK = 64, kGThreads = 256;
#ifndef TQ_GEMM_SWZ
#define TQ_GEMM_SWZ 1
#endif
constexpr int kRowPitch = TQ_GEMM_SWZ == 2 ? 144 : 128;  // bytes per LDS row of an operand tile
constexpr int kATile = kBM * kRowPitch;                  // bf16 activation tile in LDS
constexpr int kWTile = kBN * kRowPitch;                  // dequantized weight tile in LDS
constexpr int kSmem = kATile + 2 * kWTile;
constexpr int kCLd = kBN + 8;                            // bf16 per LDS row of the staged output
constexpr int kWPieces = kBN / 128;                      // 32-k weight pieces per thread per slice
constexpr int kNJ = kBN / 64;                            // MFMA tiles per wave along N
constexpr int kOcc = kBN == 128 ? 3 : 2;                 // workgroups per CU
static_assert(kBM * kCLd * 2 <= kSmem, "output tile must fit in the operand tiles' LDS");

// Byte offset of 16-byte chunk j (0..7) of LDS row r.  Rows are 128 bytes; the
// chunk index is XORed with (r / 2) % 8, so any 16 consecutive rows read at one
// chunk, and any 2 rows written in full, cover all 16 four-bank groups.
__device__ __forceinline__ int swz(int r, int j)
{
#if TQ_GEMM_SWZ == 2
    return r * 144 + 16 * j;
#elif TQ_GEMM_SWZ == 0
    return r * 128 + 16 * (j ^ (r & 7));
#else
    return r * 128 + 16 * (j ^ ((r >> 1) & 7));
#endif
}

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));


// Eight codes (one dword, element 2j in the low nibble of byte j) times the
// block scale d as four dwords of bf16 pairs.  Exact.
__device__ __forceinline__ uint4 dequant8_bf16(uint32_t w, float d)
{
    const tq_f32x2 p0 = fp4x2_to_f32<0>(w), p1 = fp4x2_to_f32<1>(w);
    const tq_f32x2 p2 = fp4x2_to_f32<2>(w), p3 = fp4x2_to_f32<3>(w);
    return make_uint4(pack_hi16(p0[0] * d, p0[1] * d), pack_hi16(p1[0] * d, p1[1] * d),
                      pack_hi16(p2[0] * d, p2[1] * d), pack_hi16(p3[0] * d, p3[1] * d));
}

// Activation registers of one slice: bf16 pieces, or (NVFP4 activations) one
// 32-k piece of one row: codes and two block scales, as for the weights.
template <bool A_FP4>
struct ARegs {
    uint4 a[4];   // 4 x 8 bf16 of the A tile
};
template <>
struct ARegs<true> {
    uint4 w;      // 32 activation codes (one row, 32 consecutive k)
    uint32_t s;   // their two E4M3 block scales (low 16 bits)
};
struct WRegs {
    uint4 w[kWPieces];     // per piece: 32 weight codes (one row, 32 consecutive k)
    uint32_t s[kWPieces];  // per piece: its two E4M3 block scales (low 16 bits)
};

typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));

__device__ __forceinline__ uint4 to_uint4(u32x4_t v) { return make_uint4(v[0], v[1], v[2], v[3]); }

// A_FP4 = false: `a` is bf16 [m_total][k].  A_FP4 = true: `a` holds NVFP4 codes
// [m_total][k/2] with block scales `a_scales` [m_total][k/16] and the single
// tensor scale a_tensor_scale[0]; the activation tile is dequantized exactly into
// LDS like the weights.
template <bool A_FP4>
__global__ __launch_bounds__(kGThreads, kOcc) void grouped_gemm_nvfp4_kernel(
    const void* __restrict__ a, const uint8_t* __restrict__ a_scales,
    const float* __restrict__ a_tensor_scale, const int32_t* __restrict__ group_offsets,
    int num_groups, int64_t m_total, int64_t n, int64_t k, const uint8_t* __restrict__ w_codes,
    const uint8_t* __restrict__ w_scales, const float* __restrict__ w_tensor_scale,
    uint16_t* __restrict__ out, int n_tiles)
{
    // A tile, then two dequantized W tiles (the one being read, the one being filled).
    // The tile id is passed through the start of the second W tile, which is first
    // written after the prologue's barrier.
    __shared__ __attribute__((aligned(16))) uint8_t smem[kSmem];
    int64_t* s_tile = reinterpret_cast<int64_t*>(smem + kATile + kWTile);
    uint8_t* As = smem;

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

    // per-workgroup buffer resources over the tile's rows of A and W (and W's
    // scales); loads past num_records return zeros
    const int64_t a_rows = m_total - row0 < kBM ? m_total - row0 : kBM;
    const int64_t w_rows = n - col0 < kBN ? n - col0 : kBN;
    const __amdgpu_buffer_rsrc_t rs_a = A_FP4
        ? __builtin_amdgcn_make_buffer_rsrc((void*)((const uint8_t*)a + row0 * (k / 2)), 0,
                                            (int)(a_rows * (k / 2)), 0x00020000)
        : __builtin_amdgcn_make_buffer_rsrc((void*)((const uint16_t*)a + row0 * k), 0,
                                            (int)(a_rows * k * 2), 0x00020000);
    const __amdgpu_buffer_rsrc_t rs_as = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(A_FP4 ? a_scales + row0 * kb : w_scales), 0, A_FP4 ? (int)(a_rows * kb) : 0,
        0x00020000);
    const __amdgpu_buffer_rsrc_t rs_w = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(w_codes + (e * n + col0) * (k / 2)), 0, (int)(w_rows * (k / 2)), 0x00020000);
    const __amdgpu_buffer_rsrc_t rs_s = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(w_scales + (e * n + col0) * kb), 0, (int)(w_rows * kb), 0x00020000);
    // per-thread byte offsets: A pieces (row r, 8 k at c8), one weight row half
    int voff_a[4];
#pragma unroll
    for (int it = 0; it < 4; ++it) {
        const int idx = tid + it * kGThreads;
        voff_a[it] = ((idx >> 3) * (int)k + 8 * (idx & 7)) * 2;
    }
    // NVFP4 activations: one 32-k piece per thread, row tid / 2, k half tid % 2
    const int an_row = tid >> 1;
    const int voff_ac = an_row * (int)(k / 2) + 16 * (tid & 1);
    const int voff_as = an_row * (int)kb + 2 * (tid & 1);
    // weight pieces: piece q = tid + 256 p covers row q / 2, k half q % 2 of the slice
    int wn_row[kWPieces], voff_w[kWPieces], voff_s[kWPieces];
    const int wk_half = tid & 1;
#pragma unroll
    for (int p = 0; p < kWPieces; ++p) {
        wn_row[p] = (tid + kGThreads * p) >> 1;
        voff_w[p] = wn_row[p] * (int)(k / 2) + 16 * wk_half;
        voff_s[p] = wn_row[p] * (int)kb + 2 * wk_half;
    }

    // K-slices: when K is not a multiple of 64 the partial slice [0, K % 64) comes
    // first and is loaded (masked) before the loop; every slice the loop loads is
    // full, so the loop issues the same loads every time, and a slice past the
    // end is loaded with an out-of-range scalar offset, which reads zeros.
    const int64_t r_tail = k % kBK;
    const int64_t steps = k / kBK + (r_tail ? 1 : 0);
    auto kofs = [&](int64_t t) -> int64_t {
        return r_tail ? (t == 0 ? 0 : r_tail + kBK * (t - 1)) : kBK * t;
    };
    constexpr int kOutOfRange = 0x7FFFFF00;  // + any per-thread offset: beyond num_records
    auto load_a = [&](int64_t t, ARegs<A_FP4>& R) {
        if constexpr (A_FP4) {
            const bool ok = t < steps;
            const int so_c = ok ? (int)(kofs(t) / 2) : kOutOfRange;
            const int so_s = ok ? (int)(kofs(t) / 16) : kOutOfRange;
            R.w = to_uint4(__builtin_amdgcn_raw_buffer_load_b128(rs_a, voff_ac, so_c, 0));
            R.s = (uint32_t)__builtin_amdgcn_raw_buffer_load_b8(rs_as, voff_as, so_s, 0) |
                  ((uint32_t)__builtin_amdgcn_raw_buffer_load_b8(rs_as, voff_as + 1, so_s, 0) << 8);
        } else {
            const int so = t < steps ? (int)(kofs(t) * 2) : kOutOfRange;
#pragma unroll
            for (int it = 0; it < 4; ++it)
                R.a[it] = to_uint4(__builtin_amdgcn_raw_buffer_load_b128(rs_a, voff_a[it], so, 0));
        }
    };
    auto load_w = [&](int64_t t, WRegs& R) {
        const bool ok = t < steps;
        const int so_w = ok ? (int)(kofs(t) / 2) : kOutOfRange;
        const int so_s = ok ? (int)(kofs(t) / 16) : kOutOfRange;
#pragma unroll
        for (int p = 0; p < kWPieces; ++p) {
            R.w[p] = to_uint4(__builtin_amdgcn_raw_buffer_load_b128(rs_w, voff_w[p], so_w, 0));
            R.s[p] = (uint32_t)__builtin_amdgcn_raw_buffer_load_b8(rs_s, voff_s[p], so_s, 0) |
                     ((uint32_t)__builtin_amdgcn_raw_buffer_load_b8(rs_s, voff_s[p] + 1, so_s, 0) << 8);
        }
    };
    // the partial first slice: activations at or beyond K % 64 are zeroed, weights
    // are loaded block by block (a 16-byte load could run past the row)
    auto load_partial = [&](ARegs<A_FP4>& RA_, WRegs& RW_) {
        if constexpr (A_FP4) {
            RA_.w = make_uint4(0, 0, 0, 0);
            RA_.s = 0;
            if (32 * (tid & 1) < r_tail) {
                const u32x2_t lo = __builtin_amdgcn_raw_buffer_load_b64(rs_a, voff_ac, 0, 0);
                RA_.w.x = lo[0];
                RA_.w.y = lo[1];
                RA_.s = __builtin_amdgcn_raw_buffer_load_b8(rs_as, voff_as, 0, 0);
            }
            if (32 * (tid & 1) + 16 < r_tail) {
                const u32x2_t hi = __builtin_amdgcn_raw_buffer_load_b64(rs_a, voff_ac + 8, 0, 0);
                RA_.w.z = hi[0];
                RA_.w.w = hi[1];
                RA_.s |= (uint32_t)__builtin_amdgcn_raw_buffer_load_b8(rs_as, voff_as + 1, 0, 0) << 8;
            }
        } else {
#pragma unroll
            for (int it = 0; it < 4; ++it) {
                RA_.a[it] = make_uint4(0, 0, 0, 0);
                if (8 * ((tid + it * kGThreads) & 7) < r_tail)
                    RA_.a[it] = to_uint4(__builtin_amdgcn_raw_buffer_load_b128(rs_a, voff_a[it], 0, 0));
            }
        }
#pragma unroll
        for (int p = 0; p < kWPieces; ++p) {
            RW_.w[p] = make_uint4(0, 0, 0, 0);
            RW_.s[p] = 0;
            if (32 * wk_half < r_tail) {
                const u32x2_t lo = __builtin_amdgcn_raw_buffer_load_b64(rs_w, voff_w[p], 0, 0);
                RW_.w[p].x = lo[0];
                RW_.w[p].y = lo[1];
                RW_.s[p] = __builtin_amdgcn_raw_buffer_load_b8(rs_s, voff_s[p], 0, 0);
            }
            if (32 * wk_half + 16 < r_tail) {
                const u32x2_t hi = __builtin_amdgcn_raw_buffer_load_b64(rs_w, voff_w[p] + 8, 0, 0);
                RW_.w[p].z = hi[0];
                RW_.w[p].w = hi[1];
                RW_.s[p] |= (uint32_t)__builtin_amdgcn_raw_buffer_load_b8(rs_s, voff_s[p] + 1, 0, 0) << 8;
            }
        }
    };
    auto store_a = [&](const ARegs<A_FP4>& R) {
        if constexpr (A_FP4) {
            const f32x2_t d = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(R.s, 1.0f, false);
            const int j0 = 4 * (tid & 1);
            *reinterpret_cast<uint4*>(As + swz(an_row, j0 + 0)) = dequant8_bf16(R.w.x, d[0]);
            *reinterpret_cast<uint4*>(As + swz(an_row, j0 + 1)) = dequant8_bf16(R.w.y, d[0]);
            *reinterpret_cast<uint4*>(As + swz(an_row, j0 + 2)) = dequant8_bf16(R.w.z, d[1]);
            *reinterpret_cast<uint4*>(As + swz(an_row, j0 + 3)) = dequant8_bf16(R.w.w, d[1]);
        } else {
#pragma unroll
            for (int it = 0; it < 4; ++it) {
                const int idx = tid + it * kGThreads;
                *reinterpret_cast<uint4*>(As + swz(idx >> 3, idx & 7)) = R.a[it];
            }
        }
    };
    // one quarter (8 codes) of weight piece p, dequantized into buffer Wd
    auto dequant_quarter = [&](const WRegs& R, int p, int q, uint8_t* Wd) {
        const f32x2_t d = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(R.s[p], 1.0f, false);
        const uint32_t w = q == 0 ? R.w[p].x : (q == 1 ? R.w[p].y : (q == 2 ? R.w[p].z : R.w[p].w));
        *reinterpret_cast<uint4*>(Wd + swz(wn_row[p], 4 * wk_half + q)) =
            dequant8_bf16(w, q < 2 ? d[0] : d[1]);
    };

    const int wm = wave >> 1, wn = wave & 1;
    const bool live[2] = {row0 + 64 * wm < row_end, row0 + 64 * wm + 32 < row_end};
    f32x16_t acc[2][kNJ];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < kNJ; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r)
                acc[i][j][r] = 0.0f;

    // Slice t reads A from As and W from buffer t % 2.  During slice t the
    // activations of t + 1 and the weight codes of t + 2 are in flight, and the
    // codes of t + 1 (loaded one slice earlier) are dequantized into the other W
    // buffer between the MFMAs.
    ARegs<A_FP4> RA;
    WRegs RW, RW2 = {};
    if (steps > 0) {
        if (r_tail) {
            load_partial(RA, RW);
        } else {
            load_a(0, RA);
            load_w(0, RW);
        }
        store_a(RA);
#pragma unroll
        for (int p = 0; p < kWPieces; ++p)
#pragma unroll
            for (int q = 0; q < 4; ++q)
                dequant_quarter(RW, p, q, smem + kATile);
        load_w(1, RW);
    }
    __syncthreads();
    // one K-slice; `cur` holds the codes of slice t + 1, `nxt` receives those of t + 2
    auto step = [&](int64_t t, const WRegs& cur, WRegs& nxt) {
        const bool more = t + 1 < steps;
        load_a(t + 1, RA);
        load_w(t + 2, nxt);
        const uint8_t* Wc = smem + kATile + kWTile * (int)(t & 1);
        uint8_t* Wn = smem + kATile + kWTile * (1 - (int)(t & 1));
#pragma unroll
        for (int kk = 0; kk < kBK / 16; ++kk) {
            const int ch = 2 * kk + (lane >> 5);
            bf16x8_t af[2], bfr[kNJ];
#pragma unroll
            for (int i = 0; i < 2; ++i)
                af[i] = __builtin_bit_cast(bf16x8_t, *reinterpret_cast<const uint4*>(
                    As + swz(64 * wm + 32 * i + (lane & 31), ch)));
#pragma unroll
            for (int j = 0; j < kNJ; ++j)
                bfr[j] = __builtin_bit_cast(bf16x8_t, *reinterpret_cast<const uint4*>(
                    Wc + swz((kBN / 2) * wn + 32 * j + (lane & 31), ch)));
            if (more) {
#pragma unroll
                for (int p = 0; p < kWPieces; ++p)
                    dequant_quarter(cur, p, kk, Wn);
            }
#pragma unroll
            for (int i = 0; i < 2; ++i)
                if (live[i])  // 32-row blocks past the group's end only feed unstored rows
#pragma unroll
                    for (int j = 0; j < kNJ; ++j)
                        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[i], bfr[j], acc[i][j], 0, 0, 0);
        }
        __syncthreads();
        if (more) {
            store_a(RA);
            __syncthreads();
        }
    };
    // two slices per trip so that the two code registers swap roles without copies
    for (int64_t t = 0; t < steps; t += 2) {
        step(t, RW, RW2);
        if (t + 1 < steps)
            step(t + 1, RW2, RW);
    }

    // ---- epilogue: scale, RNE to bf16, stage the tile in LDS, coalesced stores ----
    const float s_e = A_FP4 ? w_tensor_scale[e] * a_tensor_scale[0] : w_tensor_scale[e];
    // Lane l holds column l % 32 of rows R (register r, even) and R + 1 (r + 1).
    // Neighbouring lanes swap one value (DPP quad_perm [1,0,3,2]) so that each
    // writes one dword of two adjacent columns: the even lane row R at columns
    // (c, c+1), the odd lane row R + 1 at columns (c-1, c).  The pair is rounded
    // to bf16 (nearest even) by one packed conversion.
    uint32_t* Cw = reinterpret_cast<uint32_t*>(smem);
    const bool odd = lane & 1;
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < kNJ; ++j)
#pragma unroll
            for (int r = 0; r < 16; r += 2) {
                const float v0 = acc[i][j][r] * s_e, v1 = acc[i][j][r + 1] * s_e;
                const float send = odd ? v0 : v1;
                const float recv = __int_as_float(
                    __builtin_amdgcn_mov_dpp(__float_as_int(send), 0xB1, 0xF, 0xF, false));
                const f32x2_t pair = {odd ? recv : v0, odd ? v1 : recv};
                const uint32_t w = __builtin_bit_cast(uint32_t, __builtin_convertvector(pair, bf16x2_t));
                const int row = 64 * wm + 32 * i + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3) + (odd ? 1 : 0);
                const int col = (kBN / 2) * wn + 32 * j + (lane & 31) - (odd ? 1 : 0);
                Cw[(row * kCLd + col) >> 1] = w;
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
        const uint4 v = *reinterpret_cast<const uint4*>(Cw + ((r * kCLd + 8 * c8) >> 1));
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

template <bool A_FP4>
static void launch_gemm(const void* a, const uint8_t* a_scales, const float* a_tensor_scale,
                        const int32_t* group_offsets, int num_groups, int64_t m_total, int64_t n,
                        int64_t k, const uint8_t* w_codes, const uint8_t* w_scales,
                        const float* w_tensor_scale, uint16_t* out, hipStream_t s)
{
    const int n_tiles = (int)((n + kBN - 1) / kBN);
    const int64_t m_tiles_max = (m_total + kBM - 1) / kBM + num_groups;
    int64_t grid = m_tiles_max * n_tiles;
    if (grid == 0)
        return;
    // a multiple of 8 with at least ceil(total/8) groups per XCD slot
    grid = ((grid + 7) / 8) * 8;
    hipLaunchKernelGGL(grouped_gemm_nvfp4_kernel<A_FP4>, dim3((unsigned)grid), dim3(kGThreads), 0,
                       s, a, a_scales, a_tensor_scale, group_offsets, num_groups, m_total, n, k,
                       w_codes, w_scales, w_tensor_scale, out, n_tiles);
}

void launch_grouped_gemm_nvfp4(const uint16_t* a, const int32_t* group_offsets, int num_groups,
                               int64_t m_total, int64_t n, int64_t k, const uint8_t* w_codes,
                               const uint8_t* w_scales, const float* w_tensor_scale, uint16_t* out,
                               hipStream_t s)
{
    launch_gemm<false>(a, nullptr, nullptr, group_offsets, num_groups, m_total, n, k, w_codes,
                       w_scales, w_tensor_scale, out, s);
}

void launch_grouped_gemm_w4a4(const uint8_t* a_codes, const uint8_t* a_scales,
                              const float* a_tensor_scale, const int32_t* group_offsets,
                              int num_groups, int64_t m_total, int64_t n, int64_t k,
                              const uint8_t* w_codes, const uint8_t* w_scales,
                              const float* w_tensor_scale, uint16_t* out, hipStream_t s)
{
    launch_gemm<true>(a_codes, a_scales, a_tensor_scale, group_offsets, num_groups, m_total, n, k,
                      w_codes, w_scales, w_tensor_scale, out, s);
}

}  // namespace tq
