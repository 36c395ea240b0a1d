// tq_api.cpp - the C ABI of libtq (include/tq.h): synchronous argument
// validation, then asynchronous kernel launches on the caller's stream.
// Nothing here allocates memory or keeps state.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/tq.h"
#include "tq_kernels.hpp"

namespace {

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

// n = a * b * c with overflow and sign checks.
bool product(int64_t a, int64_t b, int64_t c, int64_t* n)
{
    if (a < 0 || b < 0 || c < 0)
        return false;
    int64_t ab;
    if (__builtin_mul_overflow(a, b, &ab) || __builtin_mul_overflow(ab, c, n))
        return false;
    return *n <= (INT64_C(1) << 60);
}

hipStream_t as_stream(void* s) { return static_cast<hipStream_t>(s); }

// Clear a stale error left by earlier, unrelated runtime calls so that only this
// call's launches are judged.
void clear_error() { (void)hipGetLastError(); }

tq_status launch_status()
{
    hipError_t e = hipGetLastError();
    return e == hipSuccess ? TQ_OK : TQ_ERR_LAUNCH;
}

tq_status quantize_impl(const void* x, int32_t dtype, int64_t batch, int64_t rows, int64_t cols,
                        float* tensor_amax, const uint32_t* hints_in, uint8_t* codes,
                        uint8_t* scales, float* tensor_scale, uint32_t* hints_out, uint32_t flags,
                        void* stream, bool guided)
{
    if (dtype != TQ_F32 && dtype != TQ_BF16)
        return TQ_ERR_DTYPE;
    if (flags & ~static_cast<uint32_t>(TQ_AMAX_GIVEN))
        return TQ_ERR_FLAGS;
    int64_t n;
    if (!product(batch, rows, cols, &n) || cols % 16 != 0)
        return TQ_ERR_SHAPE;
    if (batch == 0)
        return TQ_OK;
    if (!tensor_amax || !tensor_scale)
        return TQ_ERR_NULL;
    const bool amax_given = (flags & TQ_AMAX_GIVEN) != 0;
    const bool bf16 = dtype == TQ_BF16;
    hipStream_t s = as_stream(stream);
    if (n == 0) {
        clear_error();
        tq::launch_empty_tensor_scalars(tensor_amax, tensor_scale, batch, !amax_given, s);
        return launch_status();
    }
    if (!x || !codes || !scales)
        return TQ_ERR_NULL;
    if (!aligned(x, 16) || !aligned(codes, 16))
        return TQ_ERR_ALIGN;
    if ((hints_in && !aligned(hints_in, 4)) || (hints_out && !aligned(hints_out, 4)))
        return TQ_ERR_ALIGN;
    clear_error();
    if (!amax_given)
        tq::launch_amax(x, bf16, batch, rows * cols, tensor_amax, s);
    int mode = tq::kModeNearest;
    uint32_t* hp = nullptr;
    if (guided && hints_in) {
        mode = tq::kModeGuided;
        hp = const_cast<uint32_t*>(hints_in);
    } else if (!guided && hints_out) {
        mode = tq::kModeNearestHint;
        hp = hints_out;
    }
    tq::launch_quantize(x, bf16, batch, rows, cols, tensor_amax, codes, scales, tensor_scale, hp,
                        mode, s);
    return launch_status();
}

}  // namespace

extern "C" {

TQ_API tq_status tq_tensor_amax(const void* x, int32_t dtype, int64_t batch, int64_t per_tensor,
                                float* amax, void* stream)
{
    if (dtype != TQ_F32 && dtype != TQ_BF16)
        return TQ_ERR_DTYPE;
    int64_t n;
    if (!product(batch, per_tensor, 1, &n) || per_tensor % 16 != 0)
        return TQ_ERR_SHAPE;
    if (batch == 0)
        return TQ_OK;
    if (!amax || (n > 0 && !x))
        return TQ_ERR_NULL;
    if (n > 0 && !aligned(x, 16))
        return TQ_ERR_ALIGN;
    clear_error();
    tq::launch_amax(x, dtype == TQ_BF16, batch, per_tensor, amax, as_stream(stream));
    return launch_status();
}

TQ_API tq_status tq_quantize(const void* x, int32_t dtype, int64_t batch, int64_t rows,
                             int64_t cols, float* tensor_amax, uint8_t* codes, uint8_t* scales,
                             float* tensor_scale, uint32_t* hints_out, uint32_t flags,
                             void* stream)
{
    return quantize_impl(x, dtype, batch, rows, cols, tensor_amax, nullptr, codes, scales,
                         tensor_scale, hints_out, flags, stream, false);
}

TQ_API tq_status tq_quantize_guided(const void* x, int32_t dtype, int64_t batch, int64_t rows,
                                    int64_t cols, float* tensor_amax, const uint32_t* hints,
                                    uint8_t* codes, uint8_t* scales, float* tensor_scale,
                                    uint32_t flags, void* stream)
{
    return quantize_impl(x, dtype, batch, rows, cols, tensor_amax, hints, codes, scales,
                         tensor_scale, nullptr, flags, stream, true);
}

TQ_API tq_status tq_extract_hint(const uint8_t* codes, int64_t n, uint32_t* hints, void* stream)
{
    if (n < 0 || n > (INT64_C(1) << 60))
        return TQ_ERR_SHAPE;
    if (n == 0)
        return TQ_OK;
    if (!codes || !hints)
        return TQ_ERR_NULL;
    if (!aligned(codes, 16) || !aligned(hints, 4))
        return TQ_ERR_ALIGN;
    clear_error();
    tq::launch_extract_hint(codes, n, hints, as_stream(stream));
    return launch_status();
}

TQ_API tq_status tq_requant_transpose_sr(const uint8_t* codes, const uint8_t* scales,
                                         const float* tensor_scale, int64_t batch, int64_t rows,
                                         int64_t cols, uint64_t seed, uint8_t* codes_t,
                                         uint8_t* scales_t, float* tensor_scale_t, void* stream)
{
    int64_t n;
    if (!product(batch, rows, cols, &n) || rows % 16 != 0 || cols % 16 != 0)
        return TQ_ERR_SHAPE;
    if (batch == 0)
        return TQ_OK;
    if (!tensor_scale || !tensor_scale_t)
        return TQ_ERR_NULL;
    if (n > 0) {
        if (!codes || !scales || !codes_t || !scales_t)
            return TQ_ERR_NULL;
        if (!aligned(codes, 16) || !aligned(codes_t, 16))
            return TQ_ERR_ALIGN;
    }
    clear_error();
    tq::launch_requant_transpose_sr(codes, scales, tensor_scale, batch, rows, cols, seed, codes_t,
                                    scales_t, tensor_scale_t, as_stream(stream));
    return launch_status();
}

// The grouped GEMM launches one workgroup per possible 128 x 256 output tile
// and indexes tiles in 32 bits: m_total fits the int32 group offsets and the
// tile count stays below 2^31.
static bool gemm_grid_ok(int64_t m_total, int64_t n, int32_t num_groups)
{
    if (m_total > INT32_MAX)
        return false;
    const int64_t tiles = ((m_total + 127) / 128 + num_groups) * ((n + 255) / 256);
    return tiles <= INT32_MAX - 8;
}

TQ_API tq_status tq_grouped_gemm_nvfp4(const uint16_t* a, const int32_t* group_offsets,
                                       int32_t num_groups, int64_t m_total, int64_t n, int64_t k,
                                       const uint8_t* w_codes, const uint8_t* w_scales,
                                       const float* w_tensor_scale, uint16_t* out, void* stream)
{
    if (num_groups < 1)
        return TQ_ERR_SHAPE;
    int64_t tmp;
    if (!product(m_total, k, 1, &tmp) || !product(m_total, n, 1, &tmp) ||
        !product(num_groups, n, k, &tmp) || k % 16 != 0 || k > (int64_t(1) << 22) || n % 2 != 0 ||
        !gemm_grid_ok(m_total, n, num_groups))
        return TQ_ERR_SHAPE;
    if (!group_offsets)
        return TQ_ERR_NULL;
    if (m_total == 0 || n == 0)
        return TQ_OK;
    if (!a || !out || !w_tensor_scale || (k > 0 && (!w_codes || !w_scales)))
        return TQ_ERR_NULL;
    if (!aligned(a, 16) || !aligned(out, 4) || (k > 0 && !aligned(w_codes, 16)))
        return TQ_ERR_ALIGN;
    clear_error();
    tq::launch_grouped_gemm_nvfp4(a, group_offsets, num_groups, m_total, n, k, w_codes, w_scales,
                                  w_tensor_scale, out, as_stream(stream));
    return launch_status();
}

TQ_API tq_status tq_quantize_mxfp8(const void* x, int32_t dtype, int64_t batch, int64_t rows,
                                   int64_t cols, uint8_t* codes, uint8_t* scales, void* stream)
{
    if (dtype != TQ_F32 && dtype != TQ_BF16)
        return TQ_ERR_DTYPE;
    int64_t n;
    if (!product(batch, rows, cols, &n) || cols % 32 != 0)
        return TQ_ERR_SHAPE;
    if (n == 0)
        return TQ_OK;
    if (!x || !codes || !scales)
        return TQ_ERR_NULL;
    if (!aligned(x, 16) || !aligned(codes, 16))
        return TQ_ERR_ALIGN;
    clear_error();
    tq::launch_quantize_mxfp8(x, dtype == TQ_BF16, n, codes, scales, as_stream(stream));
    return launch_status();
}

TQ_API tq_status tq_requant_transpose_mxfp8_sr(const uint8_t* codes, const uint8_t* scales,
                                               const float* tensor_scale, int64_t batch,
                                               int64_t rows, int64_t cols, uint64_t seed,
                                               uint8_t* codes_t, uint8_t* scales_t,
                                               float* tensor_scale_t, void* stream)
{
    int64_t n;
    if (!product(batch, rows, cols, &n) || rows % 32 != 0 || cols % 16 != 0)
        return TQ_ERR_SHAPE;
    if (batch == 0)
        return TQ_OK;
    if (!tensor_scale || !tensor_scale_t)
        return TQ_ERR_NULL;
    if (n > 0) {
        if (!codes || !scales || !codes_t || !scales_t)
            return TQ_ERR_NULL;
        if (!aligned(codes, 16) || !aligned(codes_t, 16))
            return TQ_ERR_ALIGN;
    }
    clear_error();
    tq::launch_requant_transpose_mxfp8_sr(codes, scales, tensor_scale, batch, rows, cols, seed,
                                          codes_t, scales_t, tensor_scale_t, as_stream(stream));
    return launch_status();
}

TQ_API tq_status tq_quantize_tile16(const void* x, int32_t dtype, int64_t batch, int64_t rows,
                                    int64_t cols, float* tensor_amax, uint8_t* codes,
                                    uint8_t* scales, float* tensor_scale, uint32_t flags,
                                    void* stream)
{
    if (dtype != TQ_F32 && dtype != TQ_BF16)
        return TQ_ERR_DTYPE;
    if (flags & ~static_cast<uint32_t>(TQ_AMAX_GIVEN))
        return TQ_ERR_FLAGS;
    int64_t n;
    if (!product(batch, rows, cols, &n) || rows % 16 != 0 || cols % 16 != 0)
        return TQ_ERR_SHAPE;
    if (batch == 0)
        return TQ_OK;
    if (!tensor_amax || !tensor_scale)
        return TQ_ERR_NULL;
    const bool amax_given = (flags & TQ_AMAX_GIVEN) != 0;
    hipStream_t s = as_stream(stream);
    if (n == 0) {
        clear_error();
        tq::launch_empty_tensor_scalars(tensor_amax, tensor_scale, batch, !amax_given, s);
        return launch_status();
    }
    if (!x || !codes || !scales)
        return TQ_ERR_NULL;
    if (!aligned(x, 16) || !aligned(codes, 16))
        return TQ_ERR_ALIGN;
    clear_error();
    if (!amax_given)
        tq::launch_amax(x, dtype == TQ_BF16, batch, rows * cols, tensor_amax, s);
    tq::launch_quantize_tile16(x, dtype == TQ_BF16, batch, rows, cols, tensor_amax, codes, scales,
                               tensor_scale, s);
    return launch_status();
}

TQ_API tq_status tq_transpose_tile16(const uint8_t* codes, const uint8_t* scales,
                                     const float* tensor_scale, int64_t batch, int64_t rows,
                                     int64_t cols, uint8_t* codes_t, uint8_t* scales_t,
                                     float* tensor_scale_t, void* stream)
{
    int64_t n;
    if (!product(batch, rows, cols, &n) || rows % 16 != 0 || cols % 16 != 0)
        return TQ_ERR_SHAPE;
    if (batch == 0)
        return TQ_OK;
    if (!tensor_scale || !tensor_scale_t)
        return TQ_ERR_NULL;
    if (n > 0) {
        if (!codes || !scales || !codes_t || !scales_t)
            return TQ_ERR_NULL;
        if (!aligned(codes, 8) || !aligned(codes_t, 8))
            return TQ_ERR_ALIGN;
    }
    clear_error();
    tq::launch_transpose_tile16(codes, scales, tensor_scale, batch, rows, cols, codes_t, scales_t,
                                tensor_scale_t, as_stream(stream));
    return launch_status();
}

TQ_API tq_status tq_grouped_gemm_w4a4(const uint8_t* a_codes, const uint8_t* a_scales,
                                      const float* a_tensor_scale, const int32_t* group_offsets,
                                      int32_t num_groups, int64_t m_total, int64_t n, int64_t k,
                                      const uint8_t* w_codes, const uint8_t* w_scales,
                                      const float* w_tensor_scale, uint16_t* out, void* stream)
{
    if (num_groups < 1)
        return TQ_ERR_SHAPE;
    int64_t tmp;
    if (!product(m_total, k, 1, &tmp) || !product(m_total, n, 1, &tmp) ||
        !product(num_groups, n, k, &tmp) || k % 16 != 0 || k > (int64_t(1) << 22) || n % 2 != 0 ||
        !gemm_grid_ok(m_total, n, num_groups))
        return TQ_ERR_SHAPE;
    if (!group_offsets)
        return TQ_ERR_NULL;
    if (m_total == 0 || n == 0)
        return TQ_OK;
    if (!out || !w_tensor_scale || !a_tensor_scale ||
        (k > 0 && (!a_codes || !a_scales || !w_codes || !w_scales)))
        return TQ_ERR_NULL;
    if (!aligned(out, 4) || (k > 0 && (!aligned(a_codes, 16) || !aligned(w_codes, 16))))
        return TQ_ERR_ALIGN;
    clear_error();
    tq::launch_grouped_gemm_w4a4(a_codes, a_scales, a_tensor_scale, group_offsets, num_groups,
                                 m_total, n, k, w_codes, w_scales, w_tensor_scale, out,
                                 as_stream(stream));
    return launch_status();
}

TQ_API tq_status tq_dequantize(const uint8_t* codes, const uint8_t* scales,
                               const float* tensor_scale, int64_t batch, int64_t rows,
                               int64_t cols, float* out, void* stream)
{
    int64_t n;
    if (!product(batch, rows, cols, &n) || cols % 16 != 0)
        return TQ_ERR_SHAPE;
    if (n == 0)
        return TQ_OK;
    if (!codes || !scales || !tensor_scale || !out)
        return TQ_ERR_NULL;
    if (!aligned(codes, 16) || !aligned(out, 16))
        return TQ_ERR_ALIGN;
    clear_error();
    tq::launch_dequantize(codes, scales, tensor_scale, batch, rows, cols, out, as_stream(stream));
    return launch_status();
}

TQ_API tq_status tq_code_mismatch(const uint8_t* codes_a, const uint8_t* codes_b, int64_t batch,
                                  int64_t per_tensor, uint64_t* counts, void* stream)
{
    int64_t n;
    if (!product(batch, per_tensor, 1, &n) || per_tensor % 32 != 0)
        return TQ_ERR_SHAPE;
    if (batch == 0)
        return TQ_OK;
    if (!counts || (n > 0 && (!codes_a || !codes_b)))
        return TQ_ERR_NULL;
    if (n > 0 && (!aligned(codes_a, 16) || !aligned(codes_b, 16)))
        return TQ_ERR_ALIGN;
    if (!aligned(counts, 8))
        return TQ_ERR_ALIGN;
    clear_error();
    tq::launch_mismatch(codes_a, codes_b, batch, per_tensor, counts, as_stream(stream));
    return launch_status();
}

TQ_API int32_t tq_hint_first_layer(int32_t num_layers)
{
    return num_layers > 0 ? num_layers / 2 : 0;
}

TQ_API const char* tq_status_string(tq_status s)
{
    switch (s) {
    case TQ_OK: return "TQ_OK";
    case TQ_ERR_NULL: return "TQ_ERR_NULL: a required pointer is NULL";
    case TQ_ERR_SHAPE: return "TQ_ERR_SHAPE: invalid or overflowing size";
    case TQ_ERR_DTYPE: return "TQ_ERR_DTYPE: unknown dtype";
    case TQ_ERR_ALIGN: return "TQ_ERR_ALIGN: misaligned pointer";
    case TQ_ERR_LAUNCH: return "TQ_ERR_LAUNCH: kernel launch failed";
    case TQ_ERR_DEVICE: return "TQ_ERR_DEVICE: HIP device error";
    case TQ_ERR_FLAGS: return "TQ_ERR_FLAGS: unknown flag bits";
    default: return "unknown tq_status";
    }
}

TQ_API int32_t tq_version(void) { return 0x000100; }

}  // extern "C"
