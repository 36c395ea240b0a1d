// tq_quantize.hip - bandwidth-bound kernels of the FP4 path for gfx950:
// tensor amax, nearest / guided NVFP4 quantization (with the fused 1-bit hint),
// standalone hint extraction, dequantization and code-mismatch counting.
//
// Layout and arithmetic follow include/tq.h.  Each lane owns whole 16-element
// blocks, so a block's maximum, its E4M3 scale and its reciprocal stay in the
// lane's registers with no cross-lane reduction; a wave covers 64 consecutive
// blocks (2 KiB of bf16), its loads are 16-byte vectors and its stores are one
// 8-byte code word, one scale byte and one 16-bit hint word per lane.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "tq_device.hpp"
#include "tq_kernels.hpp"

namespace tq {

constexpr int kThreads = 256;

// Workgroups per launch of the streaming kernels (spread over the batch).
//
// The amax stream is read-only, with several 16-byte loads in flight per lane in a
// grid-stride loop, and each workgroup publishes its maximum with one device-scope
// atomic.  Such atomics on one address are serialised on MI355X (about 12 ns each,
// measured), so the number of workgroups per tensor matters:
//  - A launch of many tensors (at least one per CU) uses 256-thread workgroups,
//    about a thousand in all.  Their atomics go to different addresses.
//  - Fewer tensors use 1024-thread workgroups, about one per CU in all.  For one
//    tensor this measured 5.69 TB/s against 5.08 TB/s with 1024 workgroups of 256
//    (268 MB); for 25 MB it took 10.1 us against 18.7 us.
//
// The quantizers, which also write, run fastest with one work item per lane and no
// grid-stride reuse, because consecutive workgroups then cover consecutive memory
// (measured on MI355X: 5.3 -> 5.8 TB/s for the nearest quantizer between 128k
// workgroups and one block per lane).  Nontemporal loads for the read-once streams
// were measured and not kept.
//
// The mismatch count only reads, and ends each workgroup with two 64-bit atomics on
// its tensor's counters; atomics on one address serialize (about 8-12 ns each on
// MI355X).  Each lane keeps 8 pairs of 16-byte loads in flight and a tensor gets at
// most 512 workgroups: 3072 tensors of 1.57M codes went from 1111 to 771 us (78% of
// HBM peak) and one 134M-code tensor from 400 to 38 us against one pair per lane.
constexpr int64_t kAmaxGroups = 1024;      // 256-thread workgroups, many tensors
constexpr int64_t kAmaxWideGroups = 256;   // 1024-thread workgroups, fewer tensors
constexpr int64_t kAmaxWideBelowBatch = 256;
constexpr int kAmaxWideThreads = 1024;
constexpr int kAmaxUnroll = 4;
constexpr int64_t kQuantGroups = (int64_t)1 << 30;  // as many as there are work items
constexpr int kMismatchUnroll = 8;
constexpr unsigned kMismatchMaxGroups = 512;  // per tensor

// ---------------------------------------------------------------------------
// small fills (used instead of memset nodes, which misbehave under graph replay)
// ---------------------------------------------------------------------------

__global__ __launch_bounds__(kThreads) void fill_u32_kernel(uint32_t* __restrict__ p, uint32_t v,
                                                            int64_t n)
{
    for (int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x; i < n;
         i += (int64_t)gridDim.x * kThreads)
        p[i] = v;
}

void launch_fill_u32(uint32_t* p, uint32_t v, int64_t n, hipStream_t s)
{
    if (n <= 0)
        return;
    int64_t g = (n + kThreads - 1) / kThreads;
    if (g > 1024)
        g = 1024;
    hipLaunchKernelGGL(fill_u32_kernel, dim3((unsigned)g), dim3(kThreads), 0, s, p, v, n);
}

// ---------------------------------------------------------------------------
// tensor amax
// ---------------------------------------------------------------------------

__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v)
{
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) {
        uint32_t o = (uint32_t)__shfl_xor((int)v, off, 64);
        v = v > o ? v : o;
    }
    return v;
}

__device__ __forceinline__ uint32_t abs_bits_max(uint4 q, bool bf16, uint32_t m)
{
    uint32_t w[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        if (bf16) {
            uint32_t lo = (w[i] << 16) & 0x7FFF0000u;
            uint32_t hi = w[i] & 0x7FFF0000u;
            m = m > lo ? m : lo;
            m = m > hi ? m : hi;
        } else {
            uint32_t a = w[i] & 0x7FFFFFFFu;
            m = m > a ? m : a;
        }
    }
    return m;
}

// |x| of finite binary32 values orders like the unsigned integer of its bits,
// so the maximum is taken on bit patterns and published with an integer atomic.
template <bool BF16, int T>
__global__ __launch_bounds__(T) void amax_kernel(const uint4* __restrict__ x, int64_t vec_per_tensor,
                                                 int64_t batch, float* __restrict__ amax)
{
    __shared__ uint32_t red[T / 64];
    for (int64_t b = blockIdx.y; b < batch; b += gridDim.y) {
        const uint4* xb = x + b * vec_per_tensor;
        uint32_t m = 0;
        const int64_t stride = (int64_t)gridDim.x * T;
        int64_t i = (int64_t)blockIdx.x * T + threadIdx.x;
        // kAmaxUnroll independent 16-byte loads in flight per lane
        for (; i + (kAmaxUnroll - 1) * stride < vec_per_tensor; i += kAmaxUnroll * stride) {
            uint4 q[kAmaxUnroll];
#pragma unroll
            for (int u = 0; u < kAmaxUnroll; ++u)
                q[u] = xb[i + u * stride];
#pragma unroll
            for (int u = 0; u < kAmaxUnroll; ++u)
                m = abs_bits_max(q[u], BF16, m);
        }
        for (; i < vec_per_tensor; i += stride)
            m = abs_bits_max(xb[i], BF16, m);
        m = wave_max_u32(m);
        const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
        if (lane == 0)
            red[wave] = m;
        __syncthreads();
        if (threadIdx.x == 0) {
            uint32_t r = red[0];
#pragma unroll
            for (int w = 1; w < T / 64; ++w)
                r = r > red[w] ? r : red[w];
            if (r != 0)
                atomicMax(reinterpret_cast<unsigned int*>(amax + b), r);
        }
        __syncthreads();
    }
}

static unsigned grid_y(int64_t batch) { return (unsigned)(batch < 65535 ? batch : 65535); }

// Workgroups per tensor so that the whole launch has about `target` groups of
// `threads` lanes.
static unsigned groups_per_tensor(int64_t work_items, int64_t batch, int64_t target,
                                  int64_t threads = kThreads)
{
    int64_t need = (work_items + threads - 1) / threads;
    int64_t cap = target / (batch < 1 ? 1 : batch);
    if (cap < 1)
        cap = 1;
    int64_t g = need < cap ? need : cap;
    return (unsigned)(g < 1 ? 1 : g);
}

void launch_amax(const void* x, bool bf16, int64_t batch, int64_t per_tensor, float* amax,
                 hipStream_t s)
{
    launch_fill_u32(reinterpret_cast<uint32_t*>(amax), 0u, batch, s);
    const int64_t vec = per_tensor * (bf16 ? 2 : 4) / 16;
    if (vec == 0)
        return;
    const uint4* xv = static_cast<const uint4*>(x);
    if (batch < kAmaxWideBelowBatch) {
        dim3 grid(groups_per_tensor(vec, batch, kAmaxWideGroups, kAmaxWideThreads), grid_y(batch));
        if (bf16)
            hipLaunchKernelGGL((amax_kernel<true, kAmaxWideThreads>), grid, dim3(kAmaxWideThreads), 0, s,
                               xv, vec, batch, amax);
        else
            hipLaunchKernelGGL((amax_kernel<false, kAmaxWideThreads>), grid, dim3(kAmaxWideThreads), 0, s,
                               xv, vec, batch, amax);
        return;
    }
    dim3 grid(groups_per_tensor(vec, batch, kAmaxGroups), grid_y(batch));
    if (bf16)
        hipLaunchKernelGGL((amax_kernel<true, kThreads>), grid, dim3(kThreads), 0, s, xv, vec, batch, amax);
    else
        hipLaunchKernelGGL((amax_kernel<false, kThreads>), grid, dim3(kThreads), 0, s, xv, vec, batch, amax);
}

// ---------------------------------------------------------------------------
// nearest / guided quantization
// ---------------------------------------------------------------------------

enum { MODE_NEAREST = kModeNearest, MODE_NEAREST_HINT = kModeNearestHint, MODE_GUIDED = kModeGuided };

template <bool BF16>
__device__ __forceinline__ void load_block(const void* __restrict__ x, int64_t blk, float v[16])
{
    if (BF16) {
        const uint4* p = static_cast<const uint4*>(x) + 2 * blk;
        uint4 a = p[0], b = p[1];
        uint32_t w[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            v[2 * i] = bf16_lo(w[i]);
            v[2 * i + 1] = bf16_hi(w[i]);
        }
    } else {
        const float4* p = static_cast<const float4*>(x) + 4 * blk;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            float4 q = p[i];
            v[4 * i] = q.x;
            v[4 * i + 1] = q.y;
            v[4 * i + 2] = q.z;
            v[4 * i + 3] = q.w;
        }
    }
}

// One lane quantizes one 16-element block: amax -> E4M3 scale -> reciprocal ->
// 16 codes, packed 8 bytes; MODE_NEAREST_HINT also emits the 16 parity bits and
// MODE_GUIDED consumes them.  Nearest codes come from gfx950's packed FP4
// conversion (see pack8_nearest), guided codes from the bit-level bracket rule.
template <bool BF16, int MODE>
__global__ __launch_bounds__(kThreads) void quantize_kernel(
    const void* __restrict__ x, int64_t blocks_per_tensor, int64_t batch,
    const float* __restrict__ tensor_amax, uint2* __restrict__ codes,
    uint8_t* __restrict__ scales, float* __restrict__ tensor_scale,
    uint16_t* __restrict__ hints, int64_t total_blocks)
{
    // Consecutive workgroups are dealt to the 8 XCDs in turn.  For the nearest
    // modes, when the grid has a multiple of 8 workgroups, they are renumbered
    // so that each XCD streams a contiguous eighth of the launch (3.5% faster on
    // the MoE-weights workload; the guided mode, which also reads the hints,
    // ran 4.5% slower with it and keeps the plain order).  The renumbering is
    // scalar and 32-bit unless the grid has 2^32 workgroups or more.
    uint32_t bx = blockIdx.x, by = blockIdx.y;
    if constexpr (MODE != MODE_GUIDED) {
        const uint32_t gx = gridDim.x, gy = gridDim.y;
        const uint64_t G = (uint64_t)gx * gy;
        if ((G & 7) == 0) {
            if (gy == 1) {
                bx = (bx & 7) * (gx >> 3) + (bx >> 3);
            } else if (G <= 0xFFFFFFFFull) {
                const uint32_t L = by * gx + bx, R = (L & 7) * (uint32_t)(G >> 3) + (L >> 3);
                by = R / gx;
                bx = R - by * gx;
            } else {
                const uint64_t L = (uint64_t)by * gx + bx, R = (L & 7) * (G >> 3) + (L >> 3);
                by = (uint32_t)(R / gx);
                bx = (uint32_t)(R - (uint64_t)by * gx);
            }
        }
    }
    // block j of tensor b
    auto quantize_block = [&](int64_t b, int64_t j, float s_t) __attribute__((always_inline)) {
        const int64_t blk = b * blocks_per_tensor + j;
        float v[16];
        load_block<BF16>(x, blk, v);
        uint32_t hin = 0;
        if (MODE == MODE_GUIDED)
            hin = hints[blk];
        float A_b = 0.0f;
#pragma unroll
        for (int i = 0; i < 16; ++i)
            A_b = fmaxf(A_b, fabsf(v[i]));
        uint32_t e = 0;
        if (s_t != 0.0f)
            e = e4m3_encode((A_b / 6.0f) / s_t);
        const float dec = e4m3_decode(e);
        uint32_t lo = 0, hi = 0;
        if (dec != 0.0f) {
            const float r_b = 1.0f / (dec * s_t);
            float y[16];
#pragma unroll
            for (int i = 0; i < 16; ++i)
                y[i] = v[i] * r_b;
            if (MODE == MODE_GUIDED) {
                lo = pack8_guided(y, hin);
                hi = pack8_guided(y + 8, hin >> 8);
            } else {
                lo = pack8_nearest(y);
                hi = pack8_nearest(y + 8);
            }
        }
        codes[blk] = make_uint2(lo, hi);
        scales[blk] = (uint8_t)e;
        if (MODE == MODE_NEAREST_HINT) {
            hints[blk] = (uint16_t)(parity8(lo) | (parity8(hi) << 8));
            if ((total_blocks & 1) && blk == total_blocks - 1)
                hints[blk + 1] = 0;  // zero the unused half of the last word
        }
    };
    auto scale_of = [&](int64_t b) -> float {
        const float A_T = tensor_amax[b];
        return (A_T == 0.0f) ? 0.0f : A_T / 2688.0f;
    };
    // The launcher's usual grid: one workgroup row per tensor and one block per
    // lane, so no loop.
    if ((int64_t)gridDim.y == batch && (int64_t)gridDim.x * kThreads >= blocks_per_tensor) {
        const float s_t = scale_of(by);
        if (bx == 0 && threadIdx.x == 0)
            tensor_scale[by] = s_t;
        const int64_t j = (int64_t)bx * kThreads + threadIdx.x;
        if (j < blocks_per_tensor)
            quantize_block(by, j, s_t);
        return;
    }
    for (int64_t b = by; b < batch; b += gridDim.y) {
        const float s_t = scale_of(b);
        if (bx == 0 && threadIdx.x == 0)
            tensor_scale[b] = s_t;
        for (int64_t j = (int64_t)bx * kThreads + threadIdx.x; j < blocks_per_tensor;
             j += (int64_t)gridDim.x * kThreads)
            quantize_block(b, j, s_t);
    }
}

void launch_quantize(const void* x, bool bf16, int64_t batch, int64_t rows, int64_t cols,
                     const float* tensor_amax, uint8_t* codes, uint8_t* scales,
                     float* tensor_scale, uint32_t* hints, int mode, hipStream_t s)
{
    const int64_t bpt = rows * cols / 16;
    const int64_t total = bpt * batch;
    dim3 grid(groups_per_tensor(bpt, batch, kQuantGroups), grid_y(batch));
    uint2* c2 = reinterpret_cast<uint2*>(codes);
    uint16_t* h = reinterpret_cast<uint16_t*>(hints);
#define TQ_QLAUNCH(B, M)                                                                     \
    hipLaunchKernelGGL((quantize_kernel<B, M>), grid, dim3(kThreads), 0, s, x, bpt, batch,   \
                       tensor_amax, c2, scales, tensor_scale, h, total)
    if (bf16) {
        if (mode == MODE_NEAREST)
            TQ_QLAUNCH(true, MODE_NEAREST);
        else if (mode == MODE_NEAREST_HINT)
            TQ_QLAUNCH(true, MODE_NEAREST_HINT);
        else
            TQ_QLAUNCH(true, MODE_GUIDED);
    } else {
        if (mode == MODE_NEAREST)
            TQ_QLAUNCH(false, MODE_NEAREST);
        else if (mode == MODE_NEAREST_HINT)
            TQ_QLAUNCH(false, MODE_NEAREST_HINT);
        else
            TQ_QLAUNCH(false, MODE_GUIDED);
    }
#undef TQ_QLAUNCH
}

// Per-tensor scalars of empty tensors: amax (unless given) and tensor scale are 0.
__global__ void empty_tensor_scalars_kernel(float* amax, float* ts, int64_t batch, int write_amax)
{
    for (int64_t b = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; b < batch;
         b += (int64_t)gridDim.x * blockDim.x) {
        if (write_amax)
            amax[b] = 0.0f;
        ts[b] = 0.0f;
    }
}

void launch_empty_tensor_scalars(float* amax, float* ts, int64_t batch, bool write_amax,
                                 hipStream_t s)
{
    if (batch <= 0)
        return;
    hipLaunchKernelGGL(empty_tensor_scalars_kernel, dim3(1), dim3(kThreads), 0, s, amax, ts, batch,
                       write_amax ? 1 : 0);
}

// ---------------------------------------------------------------------------
// standalone hint extraction: word w <- parity bits of codes 32w .. 32w+31
// ---------------------------------------------------------------------------

// Gather bits 0, 4, 8, ..., 28 of w into bits 0..7.
__device__ __forceinline__ uint32_t gather_nibble_lsbs(uint32_t w)
{
    uint32_t x = w & 0x11111111u;
    x = (x | (x >> 3)) & 0x03030303u;
    x = (x | (x >> 6)) & 0x000F000Fu;
    x = (x | (x >> 12)) & 0x000000FFu;
    return x;
}

__global__ __launch_bounds__(kThreads) void extract_hint_kernel(const uint8_t* __restrict__ codes,
                                                                int64_t n,
                                                                uint32_t* __restrict__ hints,
                                                                int64_t words)
{
    for (int64_t w = (int64_t)blockIdx.x * kThreads + threadIdx.x; w < words;
         w += (int64_t)gridDim.x * kThreads) {
        uint32_t bits = 0;
        if (32 * w + 32 <= n) {
            uint4 q = reinterpret_cast<const uint4*>(codes)[w];
            bits = gather_nibble_lsbs(q.x) | (gather_nibble_lsbs(q.y) << 8) |
                   (gather_nibble_lsbs(q.z) << 16) | (gather_nibble_lsbs(q.w) << 24);
        } else {
            const int64_t nbytes = (n + 1) / 2;
            for (int j = 0; j < 16 && 16 * w + j < nbytes; ++j) {
                uint32_t byte = codes[16 * w + j];
                bits |= (byte & 1u) << (2 * j);
                bits |= ((byte >> 4) & 1u) << (2 * j + 1);
            }
            const int64_t valid = n - 32 * w;  // 1..31
            bits &= (1u << valid) - 1u;
        }
        hints[w] = bits;
    }
}

void launch_extract_hint(const uint8_t* codes, int64_t n, uint32_t* hints, hipStream_t s)
{
    const int64_t words = (n + 31) / 32;
    if (words == 0)
        return;
    int64_t g = (words + kThreads - 1) / kThreads;
    if (g > (1 << 30))
        g = 1 << 30;
    hipLaunchKernelGGL(extract_hint_kernel, dim3((unsigned)g), dim3(kThreads), 0, s, codes, n,
                       hints, words);
}

// ---------------------------------------------------------------------------
// dequantization: one lane per 16-element block
// ---------------------------------------------------------------------------

__global__ __launch_bounds__(kThreads) void dequantize_kernel(const uint2* __restrict__ codes,
                                                              const uint8_t* __restrict__ scales,
                                                              const float* __restrict__ ts,
                                                              int64_t blocks_per_tensor,
                                                              int64_t batch,
                                                              float4* __restrict__ out)
{
    for (int64_t b = blockIdx.y; b < batch; b += gridDim.y) {
        const float s_t = ts[b];
        for (int64_t j = (int64_t)blockIdx.x * kThreads + threadIdx.x; j < blocks_per_tensor;
             j += (int64_t)gridDim.x * kThreads) {
            const int64_t blk = b * blocks_per_tensor + j;
            const uint2 c = codes[blk];
            const float d = e4m3_decode(scales[blk]);
            float v[16];
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                const uint32_t code = ((i < 8 ? c.x : c.y) >> (4 * (i & 7))) & 15u;
                const float mag = (e2m1_value(code & 7u) * d) * s_t;
                v[i] = (code & 8u) ? -mag : mag;
            }
#pragma unroll
            for (int i = 0; i < 4; ++i)
                out[4 * blk + i] = make_float4(v[4 * i], v[4 * i + 1], v[4 * i + 2], v[4 * i + 3]);
        }
    }
}

void launch_dequantize(const uint8_t* codes, const uint8_t* scales, const float* ts, int64_t batch,
                       int64_t rows, int64_t cols, float* out, hipStream_t s)
{
    const int64_t bpt = rows * cols / 16;
    dim3 grid(groups_per_tensor(bpt, batch, kQuantGroups), grid_y(batch));
    hipLaunchKernelGGL(dequantize_kernel, grid, dim3(kThreads), 0, s,
                       reinterpret_cast<const uint2*>(codes), scales, ts, bpt, batch,
                       reinterpret_cast<float4*>(out));
}

// ---------------------------------------------------------------------------
// code mismatch counting
// ---------------------------------------------------------------------------

__device__ __forceinline__ int signed_pos(uint32_t c)
{
    const int m = (int)(c & 7u);
    return (c & 8u) ? -m : m;
}

// Mismatches of eight packed codes: a nibble differs iff any of its bits does
// (OR-folded onto the nibble's low bit, then counted); adjacency is checked only
// for the differing nibbles.
__device__ __forceinline__ void count_word(uint32_t a, uint32_t b, uint32_t& mism, uint32_t& adj)
{
    uint32_t f = a ^ b;
    f |= f >> 1;
    f |= f >> 2;
    f &= 0x11111111u;
    mism += (uint32_t)__popc(f);
    while (f) {
        const int sh = __ffs(f) - 1;  // 4 * nibble index
        f &= f - 1u;
        const int d = signed_pos((a >> sh) & 15u) - signed_pos((b >> sh) & 15u);
        adj += (d == 1 || d == -1) ? 1u : 0u;
    }
}

// Both counts over one 16-byte piece (32 codes); equal pieces cost one compare.
__device__ __forceinline__ void count_vec(uint4 qa, uint4 qb, uint32_t& mism, uint32_t& adj)
{
    if (((qa.x ^ qb.x) | (qa.y ^ qb.y) | (qa.z ^ qb.z) | (qa.w ^ qb.w)) == 0u)
        return;
    count_word(qa.x, qb.x, mism, adj);
    count_word(qa.y, qb.y, mism, adj);
    count_word(qa.z, qb.z, mism, adj);
    count_word(qa.w, qb.w, mism, adj);
}

__global__ __launch_bounds__(kThreads) void mismatch_kernel(const uint4* __restrict__ a,
                                                            const uint4* __restrict__ b,
                                                            int64_t vec_per_tensor, int64_t batch,
                                                            unsigned long long* __restrict__ counts)
{
    __shared__ uint32_t red[2][kThreads / 64];
    for (int64_t t = blockIdx.y; t < batch; t += gridDim.y) {
        uint32_t mism = 0, adj = 0;
        const uint4* ta = a + t * vec_per_tensor;
        const uint4* tb = b + t * vec_per_tensor;
        const int64_t stride = (int64_t)gridDim.x * kThreads, last = vec_per_tensor - 1;
        // All kMismatchUnroll pairs are issued before the first is compared.  Indices
        // past the end load the last pair (in bounds, unconditional, so that the loads
        // stay together for any size) and are not counted.
        for (int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x; i < vec_per_tensor;
             i += kMismatchUnroll * stride) {
            uint4 qa[kMismatchUnroll], qb[kMismatchUnroll];
#pragma unroll
            for (int u = 0; u < kMismatchUnroll; ++u) {
                const int64_t j = i + u * stride < last ? i + u * stride : last;
                qa[u] = ta[j];
                qb[u] = tb[j];
            }
#pragma unroll
            for (int u = 0; u < kMismatchUnroll; ++u)
                if (i + u * stride < vec_per_tensor)
                    count_vec(qa[u], qb[u], mism, adj);
        }
#pragma unroll
        for (int off = 32; off >= 1; off >>= 1) {
            mism += (uint32_t)__shfl_xor((int)mism, off, 64);
            adj += (uint32_t)__shfl_xor((int)adj, off, 64);
        }
        const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
        if (lane == 0) {
            red[0][wave] = mism;
            red[1][wave] = adj;
        }
        __syncthreads();
        if (threadIdx.x == 0) {
            unsigned long long m = 0, d = 0;
            for (int w = 0; w < kThreads / 64; ++w) {
                m += red[0][w];
                d += red[1][w];
            }
            if (m)
                atomicAdd(counts + 2 * t, m);
            if (d)
                atomicAdd(counts + 2 * t + 1, d);
        }
        __syncthreads();
    }
}

void launch_mismatch(const uint8_t* a, const uint8_t* b, int64_t batch, int64_t per_tensor,
                     uint64_t* counts, hipStream_t s)
{
    launch_fill_u32(reinterpret_cast<uint32_t*>(counts), 0u, 4 * batch, s);
    const int64_t vec = per_tensor / 32;
    if (vec == 0)
        return;
    const unsigned gx = groups_per_tensor((vec + kMismatchUnroll - 1) / kMismatchUnroll, batch, kQuantGroups);
    dim3 grid(gx < kMismatchMaxGroups ? gx : kMismatchMaxGroups, grid_y(batch));
    hipLaunchKernelGGL(mismatch_kernel, grid, dim3(kThreads), 0, s,
                       reinterpret_cast<const uint4*>(a), reinterpret_cast<const uint4*>(b), vec,
                       batch, reinterpret_cast<unsigned long long*>(counts));
}

}  // namespace tq
