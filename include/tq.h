/*
 * tq.h - C ABI of libtq: block-scaled FP4 (NVFP4-style) quantization, rollout-guided
 * rounding from a 1-bit hint, a stochastic-rounding transpose-requantize and an
 * NVFP4-weight grouped GEMM, as hand-written HIP kernels for MI355X (gfx950).
 *
 * Sources, cited by page title and passage:
 *   [TRACE] "TRACE" explainer on FP4 RL rollouts (blog.ontle.kr/blog/286)
 *   [RLQ]   "RL에서 양자화를 사용하는 방법" (ai-systems-engineering.com)
 *   [TML]   "싱킹 머신스 랩, 4비트 학습 기법 공개" (metallab.ai)
 *
 * ---------------------------------------------------------------------------------
 * Conventions (all entry points)
 *
 *  Pointers    Tensor arguments are DEVICE pointers (hipMalloc memory, or the data
 *              pointer of a torch CUDA tensor) on the current HIP device.  Host
 *              pointers are never accepted.
 *  Stream      `stream` is a hipStream_t passed as void*; NULL means the null
 *              stream.  Each call validates its arguments, enqueues its kernels on
 *              `stream` and returns without synchronising.  Results are visible
 *              after the stream is synchronised; asynchronous device faults surface
 *              there, not in the return value.
 *  Ownership   The caller owns and sizes every buffer.  The library allocates no
 *              memory and keeps no state besides cached device properties; calls
 *              are reentrant and thread-safe.  Calls writing the same outputs on
 *              different streams race.
 *  Errors      Validation is synchronous and happens before anything is
 *              enqueued: a failing check returns its code and launches nothing.  A
 *              launch the runtime rejects returns TQ_ERR_LAUNCH.  No C++ exception
 *              crosses the ABI.
 *  Sizes       All sizes are element counts (int64); zero-sized work returns TQ_OK
 *              after writing only the per-tensor scalars that are defined for it.
 *
 * Data layout (NVFP4 tensor = codes + block scales + tensor scale; [TML] summary
 * box and forward/backward-mismatch paragraph: 16 consecutive values share one
 * 8-bit scale, 4.5 bits per value; [RLQ] Fig. 2 paragraph: value = code x scale):
 *
 *  x           [batch][rows][cols] row-major, fp32 or bf16 (TQ_F32 / TQ_BF16).
 *  codes       [batch][rows][cols/2] bytes.  A 4-bit code is 8*s + m: sign s (bit 3),
 *              E2M1 magnitude index m (bits 0..2) on the grid
 *              {0, 0.5, 1, 1.5, 2, 3, 4, 6}.  Element 2j sits in the low nibble of
 *              byte j.  Zero is always +0 (code 0).
 *  scales      [batch][rows][cols/16] E4M3FN bytes (bias 7, max 448), one per 16
 *              consecutive elements of a row; never NaN.
 *  tensor_scale[batch] fp32.  Value of element i of block b of tensor t:
 *              (+-G[m]) * dec(scales[b]) * tensor_scale[t].
 *  hints       1 bit per element, bit i in word i/32 at position i%32 (LSB first),
 *              over the flattened [batch][rows][cols] index.  Trailing bits of the
 *              last word are 0.
 *
 * Alignment: x, a and codes arguments must be 16-byte aligned; hints 4-byte aligned.
 * ---------------------------------------------------------------------------------
 */
#ifndef TQ_H
#define TQ_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#if defined(__GNUC__)
#define TQ_API __attribute__((visibility("default")))
#else
#define TQ_API
#endif

typedef int32_t tq_status;

enum {
    TQ_OK = 0,
    TQ_ERR_NULL = 1,   /* a required pointer is NULL */
    TQ_ERR_SHAPE = 2,  /* negative size, a dimension not a multiple of 16, overflow */
    TQ_ERR_DTYPE = 3,  /* dtype is neither TQ_F32 nor TQ_BF16 */
    TQ_ERR_ALIGN = 4,  /* pointer misaligned for the kernel's vector accesses */
    TQ_ERR_LAUNCH = 5, /* the HIP runtime rejected a kernel launch */
    TQ_ERR_DEVICE = 6, /* no usable HIP device, or a device query failed */
    TQ_ERR_FLAGS = 7   /* unknown bits in `flags` */
};

enum { TQ_F32 = 0, TQ_BF16 = 1 };

/* flags: tensor_amax[] is an input (computed elsewhere) instead of an output. */
enum { TQ_AMAX_GIVEN = 1u << 0 };

/*
 * tq_tensor_amax - per-tensor maximum of |x|: the first step of the two-level scale.
 * [RLQ] "RL에서 양자화를 사용하는 방법", the paragraph on the shared convention of
 * Fig. 2: both engines must agree not only on the codes but on the scale that
 * turns a stored code into a value.  Here that scale is the product of the E4M3
 * block scale and a per-tensor fp32 scale s_t = A_T / 2688 (2688 = 6 * 448, the
 * largest E2M1 magnitude times the largest E4M3 value), and A_T is this maximum.
 *   x          [batch][per_tensor] fp32 or bf16, 16-byte aligned.
 *   amax       [batch] fp32 output; amax[t] = max_i |x[t][i]| (0 for empty tensors).
 * per_tensor must be a multiple of 16.  Inputs must be finite.
 */
TQ_API tq_status tq_tensor_amax(const void* x, int32_t dtype, int64_t batch,
                                int64_t per_tensor, float* amax, void* stream);

/*
 * tq_quantize - nearest-rounding NVFP4 quantizer (the rollout side, and the
 * trainer side without guidance).  [TML] forward/backward-mismatch paragraph
 * (16-value groups, one scale each); [TRACE] rounding-boundary analogy (the
 * default rule rounds to the nearest bin); [RLQ] Fig. 2 paragraph (code x scale).
 *
 * Per tensor t: A_T = max|x| (computed into tensor_amax[t], or read from it with
 * TQ_AMAX_GIVEN); s_t = A_T / 2688 (0 if A_T = 0), written to tensor_scale[t].
 * Per block of 16 along a row: A_b = max|x|, d_b = (A_b / 6) / s_t,
 * e_b = E4M3 round-to-nearest-even of d_b, saturating at 448.  dec(e_b) = 0 gives
 * 16 zero codes; else r_b = 1 / (dec(e_b) * s_t).  Per element y = x * r_b and
 * m = nearest E2M1 index of |y| (ties to the even index; |y| > 5 gives 6.0).
 * Every step is one IEEE binary32 operation rounded to nearest even.
 *
 *   x            [batch][rows][cols], dtype TQ_F32 or TQ_BF16, 16-byte aligned.
 *   tensor_amax  [batch] fp32, output (input with TQ_AMAX_GIVEN).
 *   codes        [batch][rows][cols/2] u8 output, 16-byte aligned.
 *   scales       [batch][rows][cols/16] u8 output.
 *   tensor_scale [batch] fp32 output.
 *   hints_out    nullable; if given, [ceil(batch*rows*cols/32)] u32 output holding
 *                the parity (m & 1) of every code: the compact hint of [TRACE]'s
 *                compact-guidance paragraph, fused into the same pass.
 * Requires cols % 16 == 0.  Inputs must be finite, and A_T must be 0 or >= 2^-100.
 */
TQ_API tq_status tq_quantize(const void* x, int32_t dtype, int64_t batch, int64_t rows,
                             int64_t cols, float* tensor_amax, uint8_t* codes,
                             uint8_t* scales, float* tensor_scale, uint32_t* hints_out,
                             uint32_t flags, void* stream);

/*
 * tq_extract_hint - the 1-bit compact hint from stored codes.  [TRACE]
 * compact-guidance paragraph: mismatched codes are almost always one bin apart,
 * so a part of the mantissa suffices; this library sends one bit, the E2M1
 * mantissa bit (m & 1) of each rollout code.
 *   codes  [ceil(n/2)] u8 (element 2j in the low nibble), 16-byte aligned.
 *   hints  [ceil(n/32)] u32 output, 4-byte aligned; bits past n are 0.
 */
TQ_API tq_status tq_extract_hint(const uint8_t* codes, int64_t n, uint32_t* hints,
                                 void* stream);

/*
 * tq_quantize_guided - TRACE rollout-guided rounding on the trainer's tensor.
 * [TRACE] paragraph after the rounding analogy: the training side, near a
 * boundary, takes the bin the rollout actually chose instead of the nearest one,
 * which never makes the mismatch at that element worse than nearest rounding.
 *
 * Scales exactly as tq_quantize on x (the hint carries no scale).  Per element,
 * with a = |y|: a >= 6 gives m = 7; otherwise lo = the largest grid index with
 * G[lo] <= a; a == G[lo] gives m = lo; otherwise m = lo if (lo & 1) equals the
 * element's hint bit, else lo + 1.  The chosen code always brackets the value.
 *   hints  nullable: NULL gives exactly tq_quantize (callers pass NULL for layers
 *          below tq_hint_first_layer()).  Layout as in tq_quantize.
 * Other arguments, flags and requirements as in tq_quantize.
 */
TQ_API tq_status tq_quantize_guided(const void* x, int32_t dtype, int64_t batch,
                                    int64_t rows, int64_t cols, float* tensor_amax,
                                    const uint32_t* hints, uint8_t* codes, uint8_t* scales,
                                    float* tensor_scale, uint32_t flags, void* stream);

/*
 * tq_requant_transpose_sr - dequantize -> transpose -> requantize with stochastic
 * rounding, for the backward pass.  [TML] forward/backward-mismatch paragraph:
 * transposing changes which 16 values share a scale, so the values go back to
 * higher precision, are transposed, and are quantized again with stochastic
 * rounding (2.25 -> 2 with probability 3/4, -> 3 with 1/4, keeping the mean).
 *
 * Input: batch NVFP4 tensors of rows x cols (blocks along cols).  Output: the
 * cols x rows transposes, blocks of 16 along the new rows (down 16 input rows).
 * u = +-G[m] * dec(e) (exact, tensor scale left out); per new block
 * A' = max|u|, e' = E4M3(A'/6) (round to nearest even), r' = 1 / dec(e');
 * y = u * r'; between the grid points lo <= |y| < lo+1 round up iff
 * k < 256 * (|y| - G[lo]) / (G[lo+1] - G[lo]), k the element's random byte;
 * |y| >= 6 gives 6.  tensor_scale_t = tensor_scale.
 * Random byte of output element i (linear index over [batch][cols][rows]): byte
 * i mod 16, little-endian, of Philox4x32-10 with counter (i/16 mod 2^32, i/16 >> 32,
 * 0, 0) and key (seed mod 2^32, seed >> 32).
 *
 *   codes, scales, tensor_scale   input NVFP4 tensors ([batch][rows][cols/2], ...).
 *   codes_t  [batch][cols][rows/2] u8 output, 16-byte aligned.
 *   scales_t [batch][cols][rows/16] u8 output.
 *   tensor_scale_t [batch] fp32 output.
 * Requires rows % 16 == 0 and cols % 16 == 0; codes 16-byte aligned.
 */
TQ_API tq_status tq_requant_transpose_sr(const uint8_t* codes, const uint8_t* scales,
                                         const float* tensor_scale, int64_t batch,
                                         int64_t rows, int64_t cols, uint64_t seed,
                                         uint8_t* codes_t, uint8_t* scales_t,
                                         float* tensor_scale_t, void* stream);

/*
 * tq_grouped_gemm_nvfp4 - MoE expert GEMM with NVFP4 weights and bf16 activations.
 * [TML] summary box and the paragraph on where 4-bit compute is used: the MoE
 * layers' forward runs with NVFP4 operands.
 *
 * For group e and rows off[e] <= i < off[e+1]:
 *   out[i][c] = bf16_rne( s_e * sum_k a[i][k] * W_e[c][k] ),
 * W_e[c][k] = +-G[m] * dec(e_b), dequantized exactly to bf16 in on-chip memory,
 * products accumulated in fp32 by bf16 MFMA, s_e = w_tensor_scale[e] applied once.
 *
 *   a              [m_total][k] bf16 (raw 16-bit patterns), 16-byte aligned.
 *   group_offsets  [num_groups+1] int32, device memory.
 *   w_codes        [num_groups][n][k/2] u8 (k contiguous), 16-byte aligned.
 *   w_scales       [num_groups][n][k/16] u8.
 *   w_tensor_scale [num_groups] fp32.
 *   out            [m_total][n] bf16 output, 4-byte aligned.
 * Requires k % 16 == 0, 0 <= k <= 2^22, n % 2 == 0, num_groups >= 1,
 * m_total < 2^31 and (ceil(m_total/128) + num_groups) * ceil(n/256) < 2^31 - 8
 * (the output tile count; else TQ_ERR_SHAPE).  Device-side preconditions
 * (not checked): group_offsets nondecreasing with [0] = 0 and
 * [num_groups] = m_total; scale bytes are non-negative E4M3 (0x00..0x7E,
 * as tq_quantize writes them).
 * Rows outside every group are left unwritten.
 */
TQ_API tq_status tq_grouped_gemm_nvfp4(const uint16_t* a, const int32_t* group_offsets,
                                       int32_t num_groups, int64_t m_total, int64_t n,
                                       int64_t k, const uint8_t* w_codes,
                                       const uint8_t* w_scales, const float* w_tensor_scale,
                                       uint16_t* out, void* stream);

/*
 * MXFP8 ([TML] summary box: the backward runs in MXFP8 with requantization and
 * stochastic rounding; format-comparison paragraph: 8.25 bits per value, i.e.
 * an 8-bit scale per 32 8-bit values).  Elements are E4M3FN bytes (sign in bit 7,
 * zero always 0x00, never NaN, |value| <= 448); a block of 32 consecutive values
 * along a row shares one E8M0 scale byte E, value 2^(E - 127).  The shared
 * exponent of a block with maximum magnitude A > 0 is floor(log2 A) - 8 (the
 * exponent of E4M3's largest normal), clamped to [-127, 127]; A = 0 gives E = 0
 * and zero elements.
 *
 * tq_quantize_mxfp8 - nearest MXFP8: element = E4M3 round-to-nearest-even of
 * x * 2^-se, saturating at 448.
 *   x       [batch][rows][cols] fp32 or bf16, 16-byte aligned.
 *   codes   [batch][rows][cols] E4M3 bytes, 16-byte aligned.
 *   scales  [batch][rows][cols/32] E8M0 bytes.
 * Requires cols % 32 == 0.
 */
TQ_API tq_status tq_quantize_mxfp8(const void* x, int32_t dtype, int64_t batch, int64_t rows,
                                   int64_t cols, uint8_t* codes, uint8_t* scales, void* stream);

/*
 * tq_requant_transpose_mxfp8_sr - the backward copy of an NVFP4 forward tensor:
 * dequantize exactly (u = +-G[m] * dec(e), tensor scale kept aside), transpose,
 * and requantize to MXFP8 along the new rows (blocks of 32 down 32 original rows)
 * with stochastic rounding on the E4M3 grid: y = u * 2^-se (exact); with lo <= |y|
 * < hi the bracketing E4M3 values, round up iff k < 256 (|y| - lo) / (hi - lo),
 * k the element's random byte from the Philox4x32-10 stream of
 * tq_requant_transpose_sr (same counter, key and byte layout, output index
 * i = (b * cols + j) * rows + r); |y| >= 448 gives 448.  The tensor scale is
 * copied: value = E4M3 * 2^se * tensor_scale_t.
 *   codes, scales, tensor_scale  NVFP4 input [batch][rows][cols] (as tq_quantize).
 *   codes_t   [batch][cols][rows] E4M3 bytes; scales_t [batch][cols][rows/32] E8M0;
 *   tensor_scale_t [batch].
 * Requires rows % 32 == 0 and cols % 16 == 0; codes and codes_t 16-byte aligned.
 */
TQ_API tq_status tq_requant_transpose_mxfp8_sr(const uint8_t* codes, const uint8_t* scales,
                                               const float* tensor_scale, int64_t batch,
                                               int64_t rows, int64_t cols, uint64_t seed,
                                               uint8_t* codes_t, uint8_t* scales_t,
                                               float* tensor_scale_t, void* stream);

/*
 * tq_quantize_tile16 - nearest NVFP4 quantization with one E4M3 scale per 16 x 16
 * tile instead of per 16 consecutive values ([TML] forward/backward-mismatch
 * paragraph: the tile alternative, which a transpose leaves intact, and its
 * drawback that one large value can zero the rest of its 256-value tile).
 *
 * Steps as tq_quantize with the block maximum taken over the tile:
 *   s_t = A_T/2688; per tile A = max|x| over its 256 values,
 *   e = enc(fl(fl(A/6)/s_t)), r = fl(1/fl(dec(e) s_t)); per element the nearest
 *   E2M1 code of fl(x r), zero as +0; a tile whose scale decodes to 0 is all 0.
 *
 *   x            [batch][rows][cols] fp32 or bf16, 16-byte aligned.
 *   codes        [batch][rows][cols/2] (as tq_quantize), 16-byte aligned.
 *   scales       [batch][rows/16][cols/16] E4M3 tile scales.
 *   tensor_amax, tensor_scale, flags as tq_quantize.
 * Requires rows % 16 == 0 and cols % 16 == 0 (else TQ_ERR_SHAPE).
 */
TQ_API tq_status tq_quantize_tile16(const void* x, int32_t dtype, int64_t batch, int64_t rows,
                                    int64_t cols, float* tensor_amax, uint8_t* codes,
                                    uint8_t* scales, float* tensor_scale, uint32_t flags,
                                    void* stream);

/*
 * tq_transpose_tile16 - transpose of a 16x16-tile NVFP4 tensor.  Every value keeps
 * its tile, so codes and tile scales are moved and nothing is requantized: the
 * result equals tq_quantize_tile16 of the transposed input, bit for bit.
 *
 *   codes/scales/tensor_scale  input as written by tq_quantize_tile16.
 *   codes_t   [batch][cols][rows/2], 8-byte aligned (codes too).
 *   scales_t  [batch][cols/16][rows/16].
 *   tensor_scale_t [batch] = tensor_scale.
 * Requires rows % 16 == 0 and cols % 16 == 0.
 */
TQ_API tq_status tq_transpose_tile16(const uint8_t* codes, const uint8_t* scales,
                                     const float* tensor_scale, int64_t batch, int64_t rows,
                                     int64_t cols, uint8_t* codes_t, uint8_t* scales_t,
                                     float* tensor_scale_t, void* stream);

/*
 * tq_grouped_gemm_w4a4 - MoE expert GEMM with NVFP4 weights AND NVFP4 activations
 * ([TRACE] results-table paragraph: the compared FP4 rollouts quantize weights,
 * activations and KV cache; [TML] summary box: the MoE forward runs in NVFP4).
 *
 * As tq_grouped_gemm_nvfp4, with the activations one NVFP4 tensor (as written by
 * tq_quantize with batch 1, rows m_total, cols k):
 *   out[i][c] = bf16_rne( (s_a * s_e) * sum_k A~[i][k] * W~_e[c][k] ),
 * A~[i][k] = +-G[m] * dec(a_scales[i][k/16]), s_a = a_tensor_scale[0]; both operands
 * are dequantized exactly to bf16 in on-chip memory and multiplied by bf16 MFMA
 * with fp32 accumulation.
 *
 *   a_codes        [m_total][k/2] u8, 16-byte aligned.
 *   a_scales       [m_total][k/16] u8 E4M3 (0x00..0x7E).
 *   a_tensor_scale [1] fp32.
 *   other arguments as tq_grouped_gemm_nvfp4.
 * Requirements and errors as tq_grouped_gemm_nvfp4.
 */
TQ_API tq_status tq_grouped_gemm_w4a4(const uint8_t* a_codes, const uint8_t* a_scales,
                                      const float* a_tensor_scale, const int32_t* group_offsets,
                                      int32_t num_groups, int64_t m_total, int64_t n, int64_t k,
                                      const uint8_t* w_codes, const uint8_t* w_scales,
                                      const float* w_tensor_scale, uint16_t* out, void* stream);

/*
 * tq_dequantize - NVFP4 -> fp32: out = (+-G[m] * dec(e)) * tensor_scale ([RLQ]
 * Fig. 2 paragraph: code x scale).  Shapes as in tq_quantize; out [batch][rows][cols]
 * fp32, 16-byte aligned.  Requires cols % 16 == 0.
 */
TQ_API tq_status tq_dequantize(const uint8_t* codes, const uint8_t* scales,
                               const float* tensor_scale, int64_t batch, int64_t rows,
                               int64_t cols, float* out, void* stream);

/*
 * tq_code_mismatch - per-tensor mismatch statistics between two code arrays
 * ([TRACE] compact-guidance paragraph: mismatches counted per element, nearly
 * all one bin apart).  counts[2t] = #{i : a_i != b_i};
 * counts[2t+1] = #{i : signed grid positions differ by exactly one}.
 *   codes_a, codes_b [batch][per_tensor/2] u8, 16-byte aligned.
 *   counts           [batch][2] u64 output (overwritten).
 * per_tensor must be a multiple of 32.
 */
TQ_API tq_status tq_code_mismatch(const uint8_t* codes_a, const uint8_t* codes_b,
                                  int64_t batch, int64_t per_tensor, uint64_t* counts,
                                  void* stream);

/* First layer that receives hints: floor(num_layers / 2) ([TRACE] compact-guidance
 * paragraph: only the latter half of the layers). Host-only, no device work. */
TQ_API int32_t tq_hint_first_layer(int32_t num_layers);

/* Static string naming a status code. */
TQ_API const char* tq_status_string(tq_status s);

/* Library version, e.g. 0x000100 for 0.1.0. */
TQ_API int32_t tq_version(void);

#ifdef __cplusplus
}
#endif

#endif /* TQ_H */
