// tq_gemm.hip - grouped GEMM with NVFP4 expert weights and bf16 activations (gfx950).
//
// [TML] "싱킹 머신스 랩, 4비트 학습 기법 공개", summary box and the paragraph on
// where 4-bit compute is used: the MoE layers' forward runs with NVFP4 operands.
// Here the weights are NVFP4 and the activations bf16: each weight fragment is
// dequantized exactly in registers (G[m] * dec(e) has at most 6 significant
// bits, so bf16 holds it), the products go through bf16 MFMA with fp32
// accumulation, and the per-expert fp32 tensor scale is applied once in the
// epilogue before the round-to-nearest-even conversion to bf16.
//
// Work decomposition.  One workgroup (4 waves) computes a kBM x kBN = 128 x 256
// output tile of one group (expert); wave w owns all 128 rows and columns
// 64 w .. 64 w + 63 as 4 x 2 MFMA 32x32x16 tiles, with the weights as the
// MFMA's row operand and the activations as its column operand (so a lane's
// accumulators hold one output row and runs of four consecutive columns, which
// the epilogue stages with 8-byte LDS writes).  Only the activations go
// through LDS (each wave reads all of them: 0.5 KiB of LDS per MFMA); the
// weight codes go straight from memory to the registers of the lanes that feed
// them to the MFMA and are dequantized there, so no weight value is written to
// or read from LDS.  Within a K-slice the MFMA's k order is free as long as both
// operands agree: lane half h = lane / 32 supplies k = 32 h + 8 kk .. + 7 in the
// kk-th MFMA, which makes a lane's weights for one column 32 consecutive codes
// (one 16-byte load) and its activations chunk 4 h + kk of the LDS row.
// The tile list is derived on the device from the group offsets (a wave-wide
// prefix scan of per-group tile counts, then a ballot for the tile's group), so
// no host synchronisation is needed.
// Consecutive workgroup ids are dealt round-robin to the 8 XCDs; the id -> tile
// map undoes that, so each XCD walks a contiguous run of tiles in (M-tile,
// N-tile) order and the N-tiles of one M-tile share their activation rows
// through that XCD's L2.
//
// Block scales.  Per-lane byte loads of scales touch one cache line per lane
// and cost far more than their size, so when a tile's block scales fit in LDS
// (K <= 2048, 16-byte aligned rows) they are copied there once per tile with
// 16-byte loads and read from LDS in the loop; otherwise they are loaded two
// bytes per lane and slice.
//
// Pipeline.  The weight codes of slice t + 2 are in flight during K-slice t
// (three code register sets rotate).  With bf16 activations and staged scales
// the activation tiles form a ring of three in LDS: the activations of slice
// t + 2 are loaded during slice t and written at its end into the tile slice
// t - 1 read, so slice t + 1's tile is complete before slice t ends and the
// first fragments of slice t + 1 are produced before the barrier.  Otherwise
// two tiles alternate and slice t + 1's activations are loaded during slice t.
// Either way one barrier per slice suffices.  The fragments of MFMA step kk + 1
// (weights dequantized, activations read) are produced while the MFMAs of step
// kk run, in a fixed issue order: the fragment reads first, then one MFMA per
// four dequantization VALU instructions.  All operand loads are buffer loads against per-workgroup resources:
// the per-thread byte offsets are fixed for the whole K loop and the slice
// position is a scalar offset, and rows past the end of A or W read as zeros in
// hardware (such rows only feed output rows or columns that are never stored).
// Only a partial first K-slice (K not a multiple of 64) masks its loads.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "tq_device.hpp"
#include "tq_kernels.hpp"

namespace tq {

constexpr int kBM = 128, kBN = 256, kBK = 64, kGThreads = 256;
constexpr int kATile = kBM * 128;                 // bf16 activation tile in LDS (128 B rows)
constexpr int kWSTile = 32768;                    // a tile's weight block scales (kBN rows, K <= 2048)
constexpr int kASTile = 16384;                    // a tile's activation block scales (kBM rows)
constexpr int kNI = kBM / 32;                     // MFMA tiles per wave along M
constexpr int kNJ = 2;                            // MFMA tiles per wave along N (64 columns)

constexpr int kCP = 64 + 4;                       // bf16 per staged output row of one wave

// Activation tiles in LDS: a ring of three with bf16 activations (slice t + 1
// is complete before slice t ends, so its first fragments are read before the
// barrier); two with NVFP4 activations, whose staged activation scales leave no
// room for a third tile at two workgroups per CU, and two without staged scales
// (the per-slice scale registers leave none for the early fragments).
template <bool A_FP4, bool SLDS>
constexpr int ring() { return A_FP4 || !SLDS ? 2 : 3; }

template <bool A_FP4, bool SLDS>
constexpr int smem_bytes()
{
    const int ops = ring<A_FP4, SLDS>() * kATile + (SLDS ? kWSTile + (A_FP4 ? kASTile : 0) : 0);
    const int out = 4 * kBM * kCP * 2;  // each wave's staged 128 x 64 output block
    return ops > out ? ops : out;
}

// Byte offset of 16-byte chunk j (0..7) of LDS row r.  Rows are 128 bytes; the
// chunk index is XORed with (r / 2) % 8, so any 16 consecutive rows read at one
// chunk, and any 2 rows written in full, cover all 16 four-bank groups.
__device__ __forceinline__ int swz(int r, int j) { return r * 128 + 16 * (j ^ ((r >> 1) & 7)); }

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));

__device__ __forceinline__ uint4 to_uint4(u32x4_t v) { return make_uint4(v[0], v[1], v[2], v[3]); }

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
// 32-k piece of one row: codes and, without LDS scales, its two block scales.
template <bool A_FP4>
struct ARegs {
    uint4 a[4];   // 4 x 8 bf16 of the A tile
};
template <>
struct ARegs<true> {
    uint4 w;      // 32 activation codes (one row, 32 consecutive k)
    uint32_t s;   // their two E4M3 block scales (low 16 bits)
};
// The weight codes one lane feeds to the MFMAs of one slice: for each of its
// kNJ columns, 32 consecutive k (its half of the slice), and, without LDS
// scales, their two block scales.
struct WRegs {
    uint4 w[kNJ];
    uint32_t s[kNJ];
};

// A_FP4 = false: `a` is bf16 [m_total][k].  A_FP4 = true: `a` holds NVFP4 codes
// [m_total][k/2] with block scales `a_scales` [m_total][k/16] and the single
// tensor scale a_tensor_scale[0]; the activation tile is dequantized exactly into
// LDS.  SLDS: block scales are staged in LDS per tile (see the launcher for the
// conditions).
template <bool A_FP4, bool SLDS>
__global__ __launch_bounds__(kGThreads, 2) void grouped_gemm_nvfp4_kernel(
    const void* __restrict__ a, const uint8_t* __restrict__ a_scales,
    const float* __restrict__ a_tensor_scale, const int32_t* __restrict__ group_offsets,
    int num_groups, int64_t m_total, int64_t n, int64_t k, const uint8_t* __restrict__ w_codes,
    const uint8_t* __restrict__ w_scales, const float* __restrict__ w_tensor_scale,
    uint16_t* __restrict__ out, int n_tiles, int sw_l2d)
{
    // The ring of activation tiles, then the staged scales; the output tile is
    // staged over the same bytes.
    __shared__ __attribute__((aligned(16))) uint8_t smem[smem_bytes<A_FP4, SLDS>()];
    constexpr int kRing = ring<A_FP4, SLDS>();
    uint8_t* const Ws = smem + kRing * kATile;              // weight scales [kBN][K/16]
    uint8_t* const As_s = smem + kRing * kATile + kWSTile;  // activation scales [kBM][K/16]

    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;

    // ---- tile id, XCD-aware order ----
    // Every wave computes it (no LDS handoff or barrier).  Lane l holds group
    // g0 + l: its row offsets and M-tile count; an inclusive wave scan of the
    // counts gives each group's first tile.  The tile's group is the first lane
    // whose running count passes the tile index (a ballot), and its values are
    // read from that lane.  With at most 64 groups this is one memory round trip
    // and one scan.  Tile counts fit 32 bits (the launcher checks).
    auto mtiles = [](int32_t rows) -> uint32_t { return rows > 0 ? ((uint32_t)rows + kBM - 1) / kBM : 0u; };
    auto scan = [&](uint32_t v) -> uint32_t {
        // rows of 16 lanes by row shifts (a lane whose source lies outside its
        // row adds 0), then the totals of rows 0 and 2 into rows 1 and 3
        // (broadcast of lane 15 of each row), then that of rows 0-1 into rows
        // 2-3 (broadcast of lane 31)
        v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x111, 0xF, 0xF, false);  // row_shr:1
        v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x112, 0xF, 0xF, false);  // row_shr:2
        v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x114, 0xF, 0xF, false);  // row_shr:4
        v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x118, 0xF, 0xF, false);  // row_shr:8
        v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x142, 0xA, 0xF, false);  // row_bcast:15
        v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x143, 0xC, 0xF, false);  // row_bcast:31
        return v;
    };
    int32_t o0 = 0, o1 = 0;  // offsets of group `lane` (first chunk)
    if (lane < num_groups) {
        o0 = group_offsets[lane];
        o1 = group_offsets[lane + 1];
    }
    uint32_t cnt = mtiles(o1 - o0);
    uint32_t incl = scan(cnt);
    uint32_t total_m = __builtin_amdgcn_readlane(incl, 63);
    for (int g0 = 64; g0 < num_groups; g0 += 64) {  // more than 64 groups
        const int g = g0 + lane;
        uint32_t c = g < num_groups ? mtiles(group_offsets[g + 1] - group_offsets[g]) : 0u;
#pragma unroll
        for (int off = 32; off >= 1; off >>= 1)
            c += __shfl_xor(c, off, 64);
        total_m += __builtin_amdgcn_readfirstlane(c);
    }
    const uint32_t total = total_m * (uint32_t)n_tiles;
    const uint32_t per_xcd = (total + 7) / 8;
    const uint32_t bx = blockIdx.x;
    const uint32_t L = (bx & 7) * per_xcd + (bx >> 3);
    if ((bx >> 3) >= per_xcd || L >= total)
        return;
    const uint32_t t_m = L / (uint32_t)n_tiles;
    const int64_t col0 = (int64_t)(L - t_m * (uint32_t)n_tiles) * kBN;
    int64_t e = -1, row0 = 0, row_end = 0;
    for (uint32_t carry = 0, g0 = 0; g0 < (uint32_t)num_groups; g0 += 64) {
        if (g0 > 0) {  // next chunk of groups (more than 64 groups)
            carry += __builtin_amdgcn_readlane(incl, 63);
            const int g = g0 + lane;
            o0 = g < num_groups ? group_offsets[g] : 0;
            o1 = g < num_groups ? group_offsets[g + 1] : 0;
            cnt = mtiles(o1 - o0);
            incl = scan(cnt);
        }
        const uint64_t hit = __ballot(t_m < carry + incl);
        if (hit) {
            const int l = __builtin_ctzll(hit);
            const uint32_t first = carry + __builtin_amdgcn_readlane(incl - cnt, l);
            e = g0 + l;
            row0 = (int64_t)__builtin_amdgcn_readlane(o0, l) + (int64_t)(t_m - first) * kBM;
            row_end = __builtin_amdgcn_readlane(o1, l);
            break;
        }
    }
    if (e < 0)  // only with offsets that break the preconditions
        return;
    const int kb = (int)(k / 16);  // scale blocks per row
    const int kh = (int)(k / 2);   // code bytes per NVFP4 row

    // per-workgroup buffer resources over the tile's rows of A and W (and their
    // scales); loads past num_records return zeros
    const int a_rows = (int)(m_total - row0 < kBM ? m_total - row0 : kBM);
    const int w_rows = (int)(n - col0 < kBN ? n - col0 : kBN);
    const __amdgpu_buffer_rsrc_t rs_a = A_FP4
        ? __builtin_amdgcn_make_buffer_rsrc((void*)((const uint8_t*)a + row0 * kh), 0,
                                            a_rows * kh, 0x00020000)
        : __builtin_amdgcn_make_buffer_rsrc((void*)((const uint16_t*)a + row0 * k), 0,
                                            a_rows * (int)k * 2, 0x00020000);
    const __amdgpu_buffer_rsrc_t rs_as = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(A_FP4 ? a_scales + row0 * kb : w_scales), 0, A_FP4 ? a_rows * kb : 0, 0x00020000);
    const __amdgpu_buffer_rsrc_t rs_w = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(w_codes + (e * n + col0) * kh), 0, w_rows * kh, 0x00020000);
    const __amdgpu_buffer_rsrc_t rs_s = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(w_scales + (e * n + col0) * kb), 0, w_rows * kb, 0x00020000);
    // per-thread byte offsets: bf16 activation pieces (row r, 8 k at c8)
    int voff_a[4];
#pragma unroll
    for (int it = 0; it < 4; ++it) {
        const int idx = tid + it * kGThreads;
        voff_a[it] = ((idx >> 3) * (int)k + 8 * (idx & 7)) * 2;
    }
    // NVFP4 activations: one 32-k piece per thread, row tid / 2, k half tid % 2
    const int an_row = tid >> 1;
    const int voff_ac = an_row * kh + 16 * (tid & 1);
    const int voff_as = an_row * kb + 2 * (tid & 1);
    // weights: this lane's column of each of its two 32-column MFMA tiles, k half h
    const int h = lane >> 5;
    int wcol[kNJ], voff_w[kNJ], voff_s[kNJ];
#pragma unroll
    for (int j = 0; j < kNJ; ++j) {
        wcol[j] = 64 * wave + 32 * j + (lane & 31);
        voff_w[j] = wcol[j] * kh + 16 * h;
        voff_s[j] = wcol[j] * kb + 2 * h;
    }

    // K-slices: when K is not a multiple of 64 the partial slice [0, K % 64) comes
    // first and is loaded (masked) before the loop; every slice the loop loads is
    // full, so the loop issues the same loads every time, and a slice past the
    // end is loaded with an out-of-range scalar offset, which reads zeros.
    const int r_tail = (int)(k % kBK);
    const int steps = (int)(k / kBK) + (r_tail ? 1 : 0);
    const int k_shift = r_tail ? kBK - r_tail : 0;  // slice t >= 1 starts at 64 t - k_shift
    auto kofs = [&](int t) -> int { return t == 0 ? 0 : kBK * t - k_shift; };
    constexpr int kOutOfRange = 0x7FFFFF00;  // + any per-thread offset: beyond num_records
    auto load_a = [&](int t, ARegs<A_FP4>& R) {
        if constexpr (A_FP4) {
            const bool ok = t < steps;
            R.w = to_uint4(__builtin_amdgcn_raw_buffer_load_b128(rs_a, voff_ac, ok ? kofs(t) / 2 : kOutOfRange, 0));
            if constexpr (!SLDS) {
                const int so_s = ok ? kofs(t) / 16 : kOutOfRange;
                R.s = (uint32_t)__builtin_amdgcn_raw_buffer_load_b8(rs_as, voff_as, so_s, 0) |
                      ((uint32_t)__builtin_amdgcn_raw_buffer_load_b8(rs_as, voff_as + 1, so_s, 0) << 8);
            }
        } else {
            const int so = t < steps ? kofs(t) * 2 : kOutOfRange;
#pragma unroll
            for (int it = 0; it < 4; ++it)
                R.a[it] = to_uint4(__builtin_amdgcn_raw_buffer_load_b128(rs_a, voff_a[it], so, 0));
        }
    };
    auto load_w = [&](int t, WRegs& R) {
        const bool ok = t < steps;
        const int so_w = ok ? kofs(t) / 2 : kOutOfRange;
        const int so_s = ok ? kofs(t) / 16 : kOutOfRange;
#pragma unroll
        for (int j = 0; j < kNJ; ++j) {
            R.w[j] = to_uint4(__builtin_amdgcn_raw_buffer_load_b128(rs_w, voff_w[j], so_w, 0));
            if constexpr (!SLDS)
                R.s[j] = (uint32_t)__builtin_amdgcn_raw_buffer_load_b8(rs_s, voff_s[j], so_s, 0) |
                         ((uint32_t)__builtin_amdgcn_raw_buffer_load_b8(rs_s, voff_s[j] + 1, so_s, 0) << 8);
        }
    };
    // The partial first slice: codes at or beyond K % 64 are zeroed and loaded
    // block by block (a 16-byte load could run past the row); so are bf16
    // activations.  Scales of blocks past K % 64 are zeroed where they are used.
    auto load_partial = [&](ARegs<A_FP4>& RA_, WRegs& RW_) {
        if constexpr (A_FP4) {
            RA_.w = make_uint4(0, 0, 0, 0);
            RA_.s = 0;
            if (32 * (tid & 1) < r_tail) {
                const u32x2_t lo = __builtin_amdgcn_raw_buffer_load_b64(rs_a, voff_ac, 0, 0);
                RA_.w.x = lo[0];
                RA_.w.y = lo[1];
                if constexpr (!SLDS)
                    RA_.s = __builtin_amdgcn_raw_buffer_load_b8(rs_as, voff_as, 0, 0);
            }
            if (32 * (tid & 1) + 16 < r_tail) {
                const u32x2_t hi = __builtin_amdgcn_raw_buffer_load_b64(rs_a, voff_ac + 8, 0, 0);
                RA_.w.z = hi[0];
                RA_.w.w = hi[1];
                if constexpr (!SLDS)
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
        for (int j = 0; j < kNJ; ++j) {
            RW_.w[j] = make_uint4(0, 0, 0, 0);
            RW_.s[j] = 0;
            if (32 * h < r_tail) {
                const u32x2_t lo = __builtin_amdgcn_raw_buffer_load_b64(rs_w, voff_w[j], 0, 0);
                RW_.w[j].x = lo[0];
                RW_.w[j].y = lo[1];
                if constexpr (!SLDS)
                    RW_.s[j] = __builtin_amdgcn_raw_buffer_load_b8(rs_s, voff_s[j], 0, 0);
            }
            if (32 * h + 16 < r_tail) {
                const u32x2_t hi = __builtin_amdgcn_raw_buffer_load_b64(rs_w, voff_w[j] + 8, 0, 0);
                RW_.w[j].z = hi[0];
                RW_.w[j].w = hi[1];
                if constexpr (!SLDS)
                    RW_.s[j] |= (uint32_t)__builtin_amdgcn_raw_buffer_load_b8(rs_s, voff_s[j] + 1, 0, 0) << 8;
            }
        }
    };
    // SLDS: copy the tile's block scales (rows x K/16 bytes, contiguous and
    // 16-byte aligned) into LDS with 16-byte loads; loads past the tile's rows
    // read zeros.
    // l2d >= 0: rows of D = 2^l2d dwords, dword w of row r stored at w ^ rot(r) (see wrot)
    auto copy_scales = [&](__amdgpu_buffer_rsrc_t rs, int bytes, uint8_t* dst, auto cap, int l2d) __attribute__((always_inline)) {
        constexpr int kRounds = decltype(cap)::value / (16 * kGThreads);
        uint4 v[kRounds];
#pragma unroll
        for (int u = 0; u < kRounds; ++u)
            if (u * 16 * kGThreads < bytes)
                v[u] = to_uint4(__builtin_amdgcn_raw_buffer_load_b128(rs, 16 * (tid + kGThreads * u), 0, 0));
#pragma unroll
        for (int u = 0; u < kRounds; ++u)
            if (u * 16 * kGThreads < bytes) {
                if (l2d < 0) {
                    *reinterpret_cast<uint4*>(dst + 16 * (tid + kGThreads * u)) = v[u];
                } else {
                    const uint32_t e[4] = {v[u].x, v[u].y, v[u].z, v[u].w};
                    const uint32_t dm = (1u << l2d) - 1u;
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const uint32_t q = 4u * (uint32_t)(tid + kGThreads * u) + (uint32_t)i;
                        const uint32_t r = q >> l2d, rot = (r >> (5 - l2d)) & dm;
                        reinterpret_cast<uint32_t*>(dst)[(r << l2d) + ((q & dm) ^ rot)] = e[i];
                    }
                }
            }
    };
    // two scale bytes (blocks 2 q, 2 q + 1 of a 32-k piece) of slice t from a staged row
    auto lds_scales = [&](const uint8_t* rowp, int t, int q) -> uint32_t {
        const uint8_t* p = rowp + kofs(t) / 16 + 2 * q;
        return (uint32_t)p[0] | ((uint32_t)p[1] << 8);
    };
    // Weight scales of slice t for column wcol[j].  With sw_l2d >= 0 (K % 64 == 0 and
    // K / 64 = D a power of two) the staged rows are rotated: dword w of row r sits at
    // w ^ ((r >> (5 - l2d)) & (D - 1)), which puts the 32 rows that a half-wave reads
    // at one slice on 32 distinct banks.  Unrotated, rows D dwords apart fall on only
    // 32 / D distinct banks (one bank for all 32 lanes at K = 2048).
    auto lds_wscales = [&](int j, int t) -> uint32_t {
        const int rot = sw_l2d >= 0 ? (wcol[j] >> (5 - sw_l2d)) & ((1 << sw_l2d) - 1) : 0;
        const uint8_t* p = Ws + wcol[j] * kb + kofs(t) / 16 + 4 * ((t ^ rot) - t) + 2 * h;
        return (uint32_t)p[0] | ((uint32_t)p[1] << 8);
    };
    // blocks of a partial first slice past K % 64 get zero scales
    auto mask_partial = [&](uint32_t s, int q) -> uint32_t {
        if (32 * q >= r_tail)
            s &= 0xFF00u;
        if (32 * q + 16 >= r_tail)
            s &= 0x00FFu;
        return s;
    };
    // activations of slice t into LDS tile As (NVFP4 ones dequantized exactly)
    auto store_a = [&](const ARegs<A_FP4>& R, int t, uint8_t* As) {
        if constexpr (A_FP4) {
            uint32_t s = R.s;
            if constexpr (SLDS) {
                s = lds_scales(As_s + an_row * kb, t < steps ? t : steps - 1, tid & 1);
                if (t == 0 && r_tail)
                    s = mask_partial(s, tid & 1);
            }
            const f32x2_t d = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(s, 1.0f, false);
            const int j0 = 4 * (tid & 1);
            *reinterpret_cast<uint4*>(As + swz(an_row, j0 + 0)) = dequant8_bf16(R.w.x, d[0]);
            *reinterpret_cast<uint4*>(As + swz(an_row, j0 + 1)) = dequant8_bf16(R.w.y, d[0]);
            *reinterpret_cast<uint4*>(As + swz(an_row, j0 + 2)) = dequant8_bf16(R.w.z, d[1]);
            *reinterpret_cast<uint4*>(As + swz(an_row, j0 + 3)) = dequant8_bf16(R.w.w, d[1]);
        } else {
            (void)t;
#pragma unroll
            for (int it = 0; it < 4; ++it) {
                const int idx = tid + it * kGThreads;
                *reinterpret_cast<uint4*>(As + swz(idx >> 3, idx & 7)) = R.a[it];
            }
        }
    };

    f32x16_t acc[kNI][kNJ];
#pragma unroll
    for (int i = 0; i < kNI; ++i)
#pragma unroll
        for (int j = 0; j < kNJ; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r)
                acc[i][j][r] = 0.0f;

    ARegs<A_FP4> RA;
    WRegs S0, S1, S2 = {};
    // Decoded weight scales of the slice whose fragments are being produced.
    // The first fragments of slice t + 1 are produced at the end of slice t
    // (before its barrier), so that slice t + 1 opens with its MFMAs.
    f32x2_t dcur[kNJ];
    bf16x8_t bf_ring[2][kNJ], af_ring[2][kNI];
    auto afrag = [&](const uint8_t* Ab, int i, int kk) -> bf16x8_t {
        return __builtin_bit_cast(bf16x8_t, *reinterpret_cast<const uint4*>(
            Ab + swz(32 * i + (lane & 31), 4 * h + kk)));
    };
    auto word = [&](const WRegs& R, int j, int kk) -> uint32_t {
        return kk == 0 ? R.w[j].x : (kk == 1 ? R.w[j].y : (kk == 2 ? R.w[j].z : R.w[j].w));
    };
    // weight scale bytes of slice t for column j (staged or in the slice's registers)
    auto wsc = [&](const WRegs& R, int j, int t) -> uint32_t {
        if constexpr (SLDS)
            return lds_wscales(j, t < steps ? t : steps - 1);
        else
            return R.s[j];
    };
    if (steps > 0) {
        // slice 0 (and with a ring of three, slice 1) into the first LDS tiles
        ARegs<A_FP4> RA1;
        if (r_tail) {
            load_partial(RA, S0);
        } else {
            load_a(0, RA);
            load_w(0, S0);
        }
        if constexpr (kRing == 3)
            load_a(1, RA1);
        load_w(1, S1);
        if constexpr (SLDS) {
            copy_scales(rs_s, w_rows * kb, Ws, std::integral_constant<int, kWSTile>{}, sw_l2d);
            if constexpr (A_FP4) {
                copy_scales(rs_as, a_rows * kb, As_s, std::integral_constant<int, kASTile>{}, -1);
                __syncthreads();  // store_a reads activation scales other threads copied
            }
        }
        store_a(RA, 0, smem);
        if constexpr (kRing == 3)
            store_a(RA1, 1, smem + kATile);
    }
    __syncthreads();
    const int nl_all = (int)((row_end - row0 + 31) / 32);  // live 32-row blocks (the tile's rows)
    if (kRing == 3 && steps > 0) {
#pragma unroll
        for (int j = 0; j < kNJ; ++j) {
            uint32_t s0 = wsc(S0, j, 0);
            if (r_tail)
                s0 = mask_partial(s0, h);
            dcur[j] = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(s0, 1.0f, false);
            bf_ring[0][j] = __builtin_bit_cast(bf16x8_t, dequant8_bf16(word(S0, j, 0), dcur[j][0]));
        }
#pragma unroll
        for (int i = 0; i < kNI; ++i)
            if (i < nl_all)
                af_ring[0][i] = afrag(smem, i, 0);
    }
    // One slice with NL live 32-row blocks (blocks past the group's end only feed
    // rows that are never stored, so their MFMAs are skipped).  With three tiles
    // the fragments of its first MFMA step are in bf[0] / af[0] on entry; with two
    // they are produced at the top of the slice.  `cur` holds its codes, `nx1`
    // those of t + 1, and `nxt` receives those of t + 2.  Slice t
    // reads LDS tile t % kRing.  With three tiles the activations of t + 2 go into
    // tile (t + 2) % 3, which slice t - 1 read before the previous barrier, and
    // tile (t + 1) % 3 is read for slice t + 1's first step before this slice's
    // barrier.  With two, the activations of t + 1 go into tile (t + 1) % 2 and
    // are read after the barrier.
    auto step = [&](auto nl, int t, const WRegs& cur, const WRegs& nx1, WRegs& nxt) __attribute__((always_inline)) {
        constexpr int NL = decltype(nl)::value;
        // with two tiles the fragments live only within the slice
        bf16x8_t bfl[2][kNJ], afl[2][kNI];
        bf16x8_t(&bf)[2][kNJ] = *(kRing == 3 ? &bf_ring : &bfl);
        bf16x8_t(&af)[2][kNI] = *(kRing == 3 ? &af_ring : &afl);
        load_a(t + kRing - 1, RA);
        load_w(t + 2, nxt);
        __builtin_amdgcn_sched_barrier(0);  // keep the loads at the top of the slice
        const int b0 = t % kRing, b1 = b0 == kRing - 1 ? 0 : b0 + 1, b2 = b1 == kRing - 1 ? 0 : b1 + 1;
        const uint8_t* Ac = smem + kATile * b0;
        const uint8_t* An = smem + kATile * b1;
        uint32_t snext[kNJ];  // three tiles: scale bytes of slice t + 1, decoded at the last step
        if constexpr (kRing == 3) {
#pragma unroll
            for (int j = 0; j < kNJ; ++j)
                snext[j] = wsc(nx1, j, t + 1);
        } else {
            // two tiles: this slice's first fragments, from the tile completed at
            // the previous barrier
#pragma unroll
            for (int j = 0; j < kNJ; ++j) {
                uint32_t st = wsc(cur, j, t);
                if (SLDS && t == 0 && r_tail)  // staged scales of blocks past K % 64
                    st = mask_partial(st, h);
                dcur[j] = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(st, 1.0f, false);
                bf[0][j] = __builtin_bit_cast(bf16x8_t, dequant8_bf16(word(cur, j, 0), dcur[j][0]));
            }
#pragma unroll
            for (int i = 0; i < NL; ++i)
                af[0][i] = afrag(Ac, i, 0);
        }
#pragma unroll
        for (int kk = 0; kk < kBK / 16; ++kk) {
            const int c = kk & 1, nx = c ^ 1;
            // fragments of the next MFMA step: step kk + 1 of this slice, or step 0
            // of slice t + 1 (tile b1 was complete at the previous barrier)
            const bool last = kk + 1 == kBK / 16;
            if (!last || kRing == 3) {
#pragma unroll
                for (int i = 0; i < NL; ++i)
                    af[nx][i] = last ? afrag(An, i, 0) : afrag(Ac, i, kk + 1);
                if (last) {
#pragma unroll
                    for (int j = 0; j < kNJ; ++j)
                        dcur[j] = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(snext[j], 1.0f, false);
                }
#pragma unroll
                for (int j = 0; j < kNJ; ++j)
                    bf[nx][j] = __builtin_bit_cast(
                        bf16x8_t, dequant8_bf16(last ? word(nx1, j, 0) : word(cur, j, kk + 1),
                                                dcur[j][last ? 0 : (kk + 1) >> 1]));
            }
#pragma unroll
            for (int i = 0; i < NL; ++i)
#pragma unroll
                for (int j = 0; j < kNJ; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(bf[c][j], af[c][i], acc[i][j], 0, 0, 0);
            if constexpr (SLDS) {
                // Issue order: the next step's activation fragment reads first,
                // then each MFMA followed by four VALU operations (the next
                // step's weight dequantization), so that the reads have a whole
                // step to land and the dequantization runs between MFMAs.  (The
                // per-slice scale loads of the other instantiation leave no
                // registers for this order.)
                const bool pre = !last || kRing == 3;
                if (pre)
                    __builtin_amdgcn_sched_group_barrier(0x100, NL, 0);  // LDS reads
#pragma unroll
                for (int m = 0; m < NL * kNJ; ++m) {
                    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // one MFMA
                    if (pre)
                        __builtin_amdgcn_sched_group_barrier(0x002, 4, 0);  // four VALU
                }
                __builtin_amdgcn_sched_barrier(0);
            }
        }
        // activations of slice t + kRing - 1 into the tile after this one's
        // successor (zeros past the last slice, into a tile nobody reads again)
        store_a(RA, t + kRing - 1, smem + kATile * (kRing == 3 ? b2 : b1));
        __syncthreads();
    };
    // three slices per trip so that the three code register sets rotate without copies
    auto run = [&](auto nl) __attribute__((always_inline)) {
        for (int t = 0; t < steps; t += 3) {
            step(nl, t, S0, S1, S2);
            if (t + 1 < steps)
                step(nl, t + 1, S1, S2, S0);
            if (t + 2 < steps)
                step(nl, t + 2, S2, S0, S1);
        }
    };
    const int64_t live_rows = row_end - row0;
    if (live_rows > 96)
        run(std::integral_constant<int, 4>{});
    else if (live_rows > 64)
        run(std::integral_constant<int, 3>{});
    else if (live_rows > 32)
        run(std::integral_constant<int, 2>{});
    else
        run(std::integral_constant<int, 1>{});

    // ---- epilogue: scale, RNE to bf16, stage through LDS, coalesced stores ----
    // The weights are the MFMA's row operand, so lane l of wave w holds
    // activation row 32 i + l % 32 and, in registers 4 g .. 4 g + 3, the four
    // consecutive columns 64 w + 32 j + 8 g + 4 h .. + 3: two packed conversions
    // and one 8-byte LDS write per group.  Each wave stages its own 128 x 64
    // block (rows of 68 bf16: 16 consecutive rows at one column cover all
    // banks) and writes it out in 128-byte row segments.  Only the wave itself
    // reads its block, and LDS operations of one wave complete in order, so no
    // barrier is needed (the loop's last barrier has retired every read of the
    // operand tiles this space overlays).
    const float s_e = A_FP4 ? w_tensor_scale[e] * a_tensor_scale[0] : w_tensor_scale[e];
    uint16_t* const Cs = reinterpret_cast<uint16_t*>(smem) + wave * (kBM * kCP);
#pragma unroll
    for (int i = 0; i < kNI; ++i)
#pragma unroll
        for (int j = 0; j < kNJ; ++j)
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                const f32x2_t p0 = {acc[i][j][4 * g] * s_e, acc[i][j][4 * g + 1] * s_e};
                const f32x2_t p1 = {acc[i][j][4 * g + 2] * s_e, acc[i][j][4 * g + 3] * s_e};
                const uint32_t w0 = __builtin_bit_cast(uint32_t, __builtin_convertvector(p0, bf16x2_t));
                const uint32_t w1 = __builtin_bit_cast(uint32_t, __builtin_convertvector(p1, bf16x2_t));
                *reinterpret_cast<uint2*>(Cs + (32 * i + (lane & 31)) * kCP + 32 * j + 8 * g + 4 * h) =
                    make_uint2(w0, w1);
            }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    // lane l writes 16 bytes of rows l / 8 + 8 it at columns 8 (l % 8) of the
    // wave's 64: all LDS reads first, then the stores
    const int64_t wc0 = col0 + 64 * wave;
    const int64_t rows_left = row_end - row0;
    const int r_l = lane >> 3, c_l = 8 * (lane & 7);
    uint4 v[kBM / 8];
#pragma unroll
    for (int it = 0; it < kBM / 8; ++it) {
        const uint16_t* s = Cs + (r_l + 8 * it) * kCP + c_l;
        const uint2 lo = *reinterpret_cast<const uint2*>(s);
        const uint2 hi = *reinterpret_cast<const uint2*>(s + 4);
        v[it] = make_uint4(lo.x, lo.y, hi.x, hi.y);
    }
    uint16_t* const dst0 = out + (row0 + r_l) * n + wc0 + c_l;
    if ((n % 8) == 0 && wc0 + 64 <= n) {
#pragma unroll
        for (int it = 0; it < kBM / 8; ++it)
            if (r_l + 8 * it < rows_left)
                *reinterpret_cast<uint4*>(dst0 + 8 * it * n) = v[it];
    } else {
        const int64_t gc = wc0 + c_l;
#pragma unroll
        for (int it = 0; it < kBM / 8; ++it) {
            if (r_l + 8 * it >= rows_left || gc >= n)
                continue;
            uint16_t* dst = dst0 + 8 * it * n;
            if ((n % 8) == 0 && gc + 8 <= n) {
                *reinterpret_cast<uint4*>(dst) = v[it];
            } else {
                const uint32_t w[4] = {v[it].x, v[it].y, v[it].z, v[it].w};
                for (int t = 0; t < 8 && gc + t < n; ++t)
                    dst[t] = (uint16_t)(w[t >> 1] >> (16 * (t & 1)));
            }
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
    // Scales staged in LDS: a tile's block of scales must fit and start on a
    // 16-byte boundary.  Weight tiles start at row e * n + 256 c; activation
    // tiles at any row, so their rows must be whole 16-byte units.
    const int64_t kb = k / 16;
    auto al16 = [](const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15) == 0; };
    bool slds = kb * kBN <= kWSTile && al16(w_scales) && (n * kb) % 16 == 0;
    if (A_FP4)
        slds = slds && kb * kBM <= kASTile && al16(a_scales) && kb % 16 == 0;
    // staged weight-scale rows rotated when K / 64 is a power of two (see lds_wscales)
    int sw_l2d = -1;
    if (k % 64 == 0 && k / 64 <= 32 && ((k / 64) & (k / 64 - 1)) == 0)
        for (sw_l2d = 0; (1 << sw_l2d) < k / 64; ++sw_l2d) {
        }
    if (slds)
        hipLaunchKernelGGL((grouped_gemm_nvfp4_kernel<A_FP4, true>), dim3((unsigned)grid),
                           dim3(kGThreads), 0, s, a, a_scales, a_tensor_scale, group_offsets,
                           num_groups, m_total, n, k, w_codes, w_scales, w_tensor_scale, out, n_tiles, sw_l2d);
    else
        hipLaunchKernelGGL((grouped_gemm_nvfp4_kernel<A_FP4, false>), dim3((unsigned)grid),
                           dim3(kGThreads), 0, s, a, a_scales, a_tensor_scale, group_offsets,
                           num_groups, m_total, n, k, w_codes, w_scales, w_tensor_scale, out, n_tiles, sw_l2d);
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
