// tq_kernels.hpp - host-side launchers of the libtq kernels (one per kernel file).
// Arguments are already validated by the C-ABI layer (tq_api.cpp).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace tq {

// quantize modes
enum { kModeNearest = 0, kModeNearestHint = 1, kModeGuided = 2 };

void launch_fill_u32(uint32_t* p, uint32_t v, int64_t n, hipStream_t s);
void launch_amax(const void* x, bool bf16, int64_t batch, int64_t per_tensor, float* amax,
                 hipStream_t s);
void launch_quantize(const void* x, bool bf16, int64_t batch, int64_t rows, int64_t cols,
                     const float* tensor_amax, uint8_t* codes, uint8_t* scales,
                     float* tensor_scale, uint32_t* hints, int mode, hipStream_t s);
void launch_empty_tensor_scalars(float* amax, float* ts, int64_t batch, bool write_amax,
                                 hipStream_t s);
void launch_extract_hint(const uint8_t* codes, int64_t n, uint32_t* hints, hipStream_t s);
void launch_dequantize(const uint8_t* codes, const uint8_t* scales, const float* ts, int64_t batch,
                       int64_t rows, int64_t cols, float* out, hipStream_t s);
void launch_mismatch(const uint8_t* a, const uint8_t* b, int64_t batch, int64_t per_tensor,
                     uint64_t* counts, hipStream_t s);
void launch_requant_transpose_sr(const uint8_t* codes, const uint8_t* scales,
                                 const float* tensor_scale, int64_t batch, int64_t rows,
                                 int64_t cols, uint64_t seed, uint8_t* codes_t, uint8_t* scales_t,
                                 float* tensor_scale_t, hipStream_t s);
void launch_quantize_tile16(const void* x, bool bf16, int64_t batch, int64_t rows, int64_t cols,
                            const float* tensor_amax, uint8_t* codes, uint8_t* scales,
                            float* tensor_scale, hipStream_t s);
void launch_transpose_tile16(const uint8_t* codes, const uint8_t* scales, const float* tensor_scale,
                             int64_t batch, int64_t rows, int64_t cols, uint8_t* codes_t,
                             uint8_t* scales_t, float* tensor_scale_t, hipStream_t s);
void launch_quantize_mxfp8(const void* x, bool bf16, int64_t n, uint8_t* codes, uint8_t* scales,
                           hipStream_t s);
void launch_requant_transpose_mxfp8_sr(const uint8_t* codes, const uint8_t* scales,
                                       const float* tensor_scale, int64_t batch, int64_t rows,
                                       int64_t cols, uint64_t seed, uint8_t* codes_t,
                                       uint8_t* scales_t, float* tensor_scale_t, hipStream_t s);
void launch_grouped_gemm_nvfp4(const uint16_t* a, const int32_t* group_offsets, int num_groups,
                               int64_t m_total, int64_t n, int64_t k, const uint8_t* w_codes,
                               const uint8_t* w_scales, const float* w_tensor_scale, uint16_t* out,
                               hipStream_t s);
void launch_grouped_gemm_w4a4(const uint8_t* a_codes, const uint8_t* a_scales,
                              const float* a_tensor_scale, const int32_t* group_offsets,
                              int num_groups, int64_t m_total, int64_t n, int64_t k,
                              const uint8_t* w_codes, const uint8_t* w_scales,
                              const float* w_tensor_scale, uint16_t* out, hipStream_t s);

}  // namespace tq
