/*
 * tq_oracle.c - plain CPU oracle for the block-scaled FP4 path.
 *
 * TEST INFRASTRUCTURE ONLY.  The test suite, the package smoke check and the
 * benchmark's CPU-baseline leg are the only callers.  The product library
 * never links, loads or calls this file, and this file includes nothing of the
 * product's sources.
 *
 * The oracle is deliberately slow and literal: each function follows one
 * definition, in the order the sources give it, with no blocking, fusion or
 * reordering.  Sources are cited by page title and passage:
 *
 *   [TRACE] "TRACE" explainer on FP4 RL rollouts (blog.ontle.kr/blog/286)
 *   [RLQ]   "RL에서 양자화를 사용하는 방법" (ai-systems-engineering.com),
 *           sections "같은 가중치에서도 확률이 달라진다" and
 *           "학습과 추론을 구성하는 두 가지 방법" (Fig. 1, Fig. 2)
 *   [TML]   "싱킹 머신스 랩, 4비트 학습 기법 공개" (metallab.ai), summary box
 *           and the format-comparison and forward/backward-mismatch paragraphs
 *
 * Where the pages are silent the readings are fixed here once (E2M1 element
 * grid, E4M3 block scale, fp32 tensor scale, operation order, tie rules,
 * stochastic-rounding random bits); they are listed with the design notes.
 *
 * Arithmetic rules.  Every `float` operation below is a single IEEE-754
 * binary32 operation, round to nearest even: the file is compiled with
 * -ffp-contract=off (no fused multiply-add) on x86-64 SSE (no excess
 * precision), subnormals kept.  Comparisons against the E2M1/E4M3 grids are
 * made in double, where each difference used is exact (see the guards).
 * Floating point decides integer codes here, so those decisions are taken in
 * binary32, the precision of the device kernels.
 */
#include <math.h>
#include <stddef.h>
#include <stdint.h>
#include <string.h>

/* ------------------------------------------------------------------------ */
/* Number formats                                                           */
/* ------------------------------------------------------------------------ */

/* E2M1 magnitudes.  [TML] format-comparison paragraph: 4 bits give 16 codes;
 * the grid itself is the usual E2M1 set.  A 4-bit code is 8*s + m: sign s in
 * bit 3, magnitude index m in bits 0..2; m's lowest bit is the mantissa bit. */
static const double E2M1_GRID[8] = {0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0};

double tqo_e2m1_value(int code)
{
    double v = E2M1_GRID[code & 7];
    return (code & 8) ? -v : v;
}

/* E4M3FN decode: sign, 4 exponent bits (bias 7), 3 mantissa bits, no
 * infinities; exponent 15 with mantissa 7 is NaN; exponent 0 holds the
 * subnormals M * 2^-9.  Largest finite value 448. */
double tqo_e4m3_value(uint8_t b)
{
    int s = b >> 7, E = (b >> 3) & 15, M = b & 7;
    double v;
    if (E == 15 && M == 7)
        return NAN;
    if (E == 0)
        v = ldexp((double)M, -9);
    else
        v = ldexp(1.0 + M / 8.0, E - 7);
    return s ? -v : v;
}

/* E4M3 encode of a finite d >= 0: the finite non-negative E4M3 value nearest
 * to d, ties to the even code (= even mantissa); d >= 448 saturates to 0x7E.
 * Guard: d <= 2^-10 is at or below the midpoint between 0 and the smallest
 * positive value 2^-9, so it encodes to 0 (the tie goes to even code 0).  For
 * the remaining d (2^-10 < d < 448) every difference d - v below spans at most
 * 42 bits and is exact in double, so the argmin is exact. */
uint8_t tqo_e4m3_encode(float d)
{
    if (!(d > 0x1p-10f))
        return 0;
    if (d >= 448.0f)
        return 0x7E;
    int best = 0;
    double bestdist = fabs((double)d);
    for (int c = 1; c <= 0x7E; ++c) {
        double dist = fabs((double)d - tqo_e4m3_value((uint8_t)c));
        if (dist < bestdist || (dist == bestdist && (c & 1) == 0)) {
            best = c;
            bestdist = dist;
        }
    }
    return (uint8_t)best;
}

/* Nearest E2M1 magnitude index for a >= 0, ties to the even index.
 * [TRACE] rounding-boundary analogy: the default rule is "the nearest bin".
 * Guards: a <= 0.25 (midpoint of 0 and 0.5, tie to even index 0) gives 0;
 * a >= 6 gives 7 (6 is the largest grid point: saturation).  In between,
 * a - G[j] is exact in double, so the argmin is exact. */
int tqo_e2m1_nearest(float a)
{
    if (!(a > 0.25f))
        return 0;
    if (a >= 6.0f)
        return 7;
    int best = 0;
    double bestdist = fabs((double)a);
    for (int j = 1; j < 8; ++j) {
        double dist = fabs((double)a - E2M1_GRID[j]);
        if (dist < bestdist || (dist == bestdist && (j & 1) == 0)) {
            best = j;
            bestdist = dist;
        }
    }
    return best;
}

/* Largest grid index j with G[j] <= a (a >= 0): the lower end of the bracket
 * that holds a. */
int tqo_e2m1_floor(float a)
{
    int lo = 0;
    for (int j = 1; j < 8; ++j)
        if (E2M1_GRID[j] <= (double)a)
            lo = j;
    return lo;
}

static float bf16_to_float(uint16_t h)
{
    uint32_t u = (uint32_t)h << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return f;
}

/* Element i of an input tensor, dtype 0 = fp32, 1 = bf16 (exact widening). */
static float load_x(const void *x, int dtype, int64_t i)
{
    if (dtype == 0)
        return ((const float *)x)[i];
    return bf16_to_float(((const uint16_t *)x)[i]);
}

static void put_code(uint8_t *codes, int64_t i, int code)
{
    uint8_t *p = &codes[i >> 1];
    if (i & 1)
        *p = (uint8_t)((*p & 0x0F) | (code << 4));
    else
        *p = (uint8_t)((*p & 0xF0) | code);
}

int tqo_get_code(const uint8_t *codes, int64_t i)
{
    return (i & 1) ? (codes[i >> 1] >> 4) : (codes[i >> 1] & 0x0F);
}

/* ------------------------------------------------------------------------ */
/* Tensor amax (per tensor of the batch)                                    */
/* ------------------------------------------------------------------------ */

void tqo_tensor_amax(const void *x, int dtype, int64_t batch, int64_t per_tensor, float *amax)
{
    for (int64_t b = 0; b < batch; ++b) {
        float m = 0.0f;
        for (int64_t i = 0; i < per_tensor; ++i) {
            float v = fabsf(load_x(x, dtype, b * per_tensor + i));
            if (v > m)
                m = v;
        }
        amax[b] = m;
    }
}

/* ------------------------------------------------------------------------ */
/* Q: nearest quantizer and G: guided quantizer                             */
/* ------------------------------------------------------------------------ */

/*
 * Shared steps 1-2 (per tensor and per block), then per element either the
 * nearest rule (Q) or the guided rule (G).
 *
 * [TML] forward/backward-mismatch paragraph: 16 consecutive values share one
 * scale.  [TML] summary box: 4.5 bits per value, i.e. one 8-bit scale per 16
 * 4-bit values.  [RLQ] Fig. 2 paragraph: a stored code times its scale is the
 * value, on both engines.  [TRACE] rounding-boundary analogy: nearest is the
 * default rule; TRACE instead takes the bin the rollout took.
 *
 * Step 1. A_T = max|x| over the tensor (or given).  s_t = A_T / 2688 where
 *         2688 = 6 * 448 (largest E2M1 times largest E4M3); A_T = 0 gives
 *         s_t = 0, all scale bytes 0 and all codes 0.
 * Step 2. Per block of 16 along the row: A_b = max|x|, d_b = (A_b / 6) / s_t,
 *         e_b = enc(d_b).  dec(e_b) = 0 gives 16 zero codes.  Otherwise
 *         S_b = dec(e_b) * s_t and r_b = 1 / S_b.
 * Step 3. y = x * r_b, a = |y|.
 *         Q: m = nearest index (ties to even, saturate at 6).
 *         G: a >= 6 gives m = 7; else lo = floor index; a on the grid gives
 *            m = lo; else m = lo if (lo & 1) equals the hint bit, else lo + 1.
 *         Sign s = 1 iff y < 0 and m != 0 (zero is canonical +0).
 *
 * hints == NULL with guided == 1 is identical to Q (no hint: nearest).
 * amax_given != 0: tensor_amax[] is an input.
 */
static void quantize_common(const void *x, int dtype, int64_t batch, int64_t rows, int64_t cols,
                            int amax_given, float *tensor_amax, const uint32_t *hints,
                            int guided, uint8_t *codes, uint8_t *scales, float *tensor_scale)
{
    const int64_t per_tensor = rows * cols;
    const int64_t blocks_per_row = cols / 16;
    for (int64_t b = 0; b < batch; ++b) {
        /* step 1 */
        float A_T;
        if (amax_given) {
            A_T = tensor_amax[b];
        } else {
            A_T = 0.0f;
            for (int64_t i = 0; i < per_tensor; ++i) {
                float v = fabsf(load_x(x, dtype, b * per_tensor + i));
                if (v > A_T)
                    A_T = v;
            }
            tensor_amax[b] = A_T;
        }
        float s_t = (A_T == 0.0f) ? 0.0f : A_T / 2688.0f;
        tensor_scale[b] = s_t;

        for (int64_t r = 0; r < rows; ++r) {
            for (int64_t blk = 0; blk < blocks_per_row; ++blk) {
                const int64_t base = b * per_tensor + r * cols + blk * 16;
                /* step 2 */
                float A_b = 0.0f;
                for (int t = 0; t < 16; ++t) {
                    float v = fabsf(load_x(x, dtype, base + t));
                    if (v > A_b)
                        A_b = v;
                }
                uint8_t e_b = 0;
                if (s_t != 0.0f) {
                    float d_b = (A_b / 6.0f) / s_t;
                    e_b = tqo_e4m3_encode(d_b);
                }
                scales[(b * rows + r) * blocks_per_row + blk] = e_b;
                float dec_e = (float)tqo_e4m3_value(e_b);
                if (dec_e == 0.0f) {
                    for (int t = 0; t < 16; ++t)
                        put_code(codes, base + t, 0);
                    continue;
                }
                float S_b = dec_e * s_t;
                float r_b = 1.0f / S_b;
                /* step 3 */
                for (int t = 0; t < 16; ++t) {
                    const int64_t i = base + t;
                    float y = load_x(x, dtype, i) * r_b;
                    float a = fabsf(y);
                    int m;
                    if (!guided || hints == NULL) {
                        m = tqo_e2m1_nearest(a);
                    } else {
                        int h = (int)((hints[i >> 5] >> (i & 31)) & 1u);
                        if (a >= 6.0f) {
                            m = 7;
                        } else {
                            int lo = tqo_e2m1_floor(a);
                            if (E2M1_GRID[lo] == (double)a)
                                m = lo;
                            else
                                m = ((lo & 1) == h) ? lo : lo + 1;
                        }
                    }
                    int s = (y < 0.0f && m != 0) ? 1 : 0;
                    put_code(codes, i, 8 * s + m);
                }
            }
        }
    }
}

/* Q, optionally also writing the rollout hint stream (see tqo_extract_hint). */
void tqo_quantize(const void *x, int dtype, int64_t batch, int64_t rows, int64_t cols,
                  int amax_given, float *tensor_amax, uint8_t *codes, uint8_t *scales,
                  float *tensor_scale)
{
    quantize_common(x, dtype, batch, rows, cols, amax_given, tensor_amax, NULL, 0, codes, scales,
                    tensor_scale);
}

void tqo_quantize_guided(const void *x, int dtype, int64_t batch, int64_t rows, int64_t cols,
                         int amax_given, float *tensor_amax, const uint32_t *hints,
                         uint8_t *codes, uint8_t *scales, float *tensor_scale)
{
    quantize_common(x, dtype, batch, rows, cols, amax_given, tensor_amax, hints, 1, codes, scales,
                    tensor_scale);
}

/* ------------------------------------------------------------------------ */
/* H: compact hint                                                           */
/* ------------------------------------------------------------------------ */

/* [TRACE] compact-guidance paragraph: mismatched values are almost always one
 * bin apart, so part of the mantissa bits suffices.  Reading: one bit per
 * element, the E2M1 mantissa bit m & 1 of the rollout's code (its parity),
 * packed least-significant-bit first into 32-bit words; bits past n are 0. */
void tqo_extract_hint(const uint8_t *codes, int64_t n, uint32_t *hints)
{
    int64_t words = (n + 31) / 32;
    for (int64_t w = 0; w < words; ++w)
        hints[w] = 0;
    for (int64_t i = 0; i < n; ++i) {
        uint32_t bit = (uint32_t)(tqo_get_code(codes, i) & 1);
        hints[i >> 5] |= bit << (i & 31);
    }
}

/* [TRACE] compact-guidance paragraph: hints go only to the latter half of the
 * layers.  Reading: layers l >= floor(L / 2). */
int tqo_hint_first_layer(int num_layers)
{
    return num_layers / 2;
}

/* ------------------------------------------------------------------------ */
/* Dequantization                                                            */
/* ------------------------------------------------------------------------ */

/* [RLQ] Fig. 2 paragraph: value = code x scale.  Here
 * v = +-((G[m] * dec(e_b)) * s_t); the inner product is exact in binary32. */
void tqo_dequantize(const uint8_t *codes, const uint8_t *scales, const float *tensor_scale,
                    int64_t batch, int64_t rows, int64_t cols, float *out)
{
    for (int64_t b = 0; b < batch; ++b)
        for (int64_t r = 0; r < rows; ++r)
            for (int64_t c = 0; c < cols; ++c) {
                int64_t i = (b * rows + r) * cols + c;
                int code = tqo_get_code(codes, i);
                float g = (float)E2M1_GRID[code & 7];
                float d = (float)tqo_e4m3_value(scales[(b * rows + r) * (cols / 16) + c / 16]);
                float v = (g * d) * tensor_scale[b];
                out[i] = (code & 8) ? -v : v;
            }
}

/* ------------------------------------------------------------------------ */
/* Philox4x32-10 (Salmon, Moraes, Dror, Shaw, "Parallel Random Numbers: As   */
/* Easy as 1, 2, 3", SC'11), written from the paper's definition.           */
/* ------------------------------------------------------------------------ */

void tqo_philox4x32_10(const uint32_t ctr_in[4], const uint32_t key_in[2], uint32_t out[4])
{
    const uint32_t M0 = 0xD2511F53u, M1 = 0xCD9E8D57u; /* round multipliers */
    const uint32_t W0 = 0x9E3779B9u, W1 = 0xBB67AE85u; /* Weyl key increments */
    uint32_t c0 = ctr_in[0], c1 = ctr_in[1], c2 = ctr_in[2], c3 = ctr_in[3];
    uint32_t k0 = key_in[0], k1 = key_in[1];
    for (int round = 0; round < 10; ++round) {
        if (round > 0) {
            k0 += W0;
            k1 += W1;
        }
        uint64_t p0 = (uint64_t)M0 * c0;
        uint64_t p1 = (uint64_t)M1 * c2;
        uint32_t hi0 = (uint32_t)(p0 >> 32), lo0 = (uint32_t)p0;
        uint32_t hi1 = (uint32_t)(p1 >> 32), lo1 = (uint32_t)p1;
        uint32_t n0 = hi1 ^ c1 ^ k0;
        uint32_t n1 = lo1;
        uint32_t n2 = hi0 ^ c3 ^ k1;
        uint32_t n3 = lo0;
        c0 = n0;
        c1 = n1;
        c2 = n2;
        c3 = n3;
    }
    out[0] = c0;
    out[1] = c1;
    out[2] = c2;
    out[3] = c3;
}

/* Random byte of output element i for stream `seed`: one Philox call per
 * 16-element output block beta = i / 16 with counter (beta lo, beta hi, 0, 0)
 * and key (seed lo, seed hi); byte i mod 16 of w0|w1|w2|w3, little-endian. */
int tqo_sr_byte(uint64_t seed, uint64_t i)
{
    uint64_t beta = i / 16;
    uint32_t ctr[4] = {(uint32_t)beta, (uint32_t)(beta >> 32), 0u, 0u};
    uint32_t key[2] = {(uint32_t)seed, (uint32_t)(seed >> 32)};
    uint32_t w[4];
    tqo_philox4x32_10(ctr, key, w);
    unsigned j = (unsigned)(i & 15);
    return (int)((w[j >> 2] >> (8 * (j & 3))) & 0xFFu);
}

/* ------------------------------------------------------------------------ */
/* S: dequantize -> transpose -> requantize with stochastic rounding         */
/* ------------------------------------------------------------------------ */

/* Stochastic rounding of a >= 0 with random byte k: [TML] forward/backward-
 * mismatch paragraph (2.25 goes to 2 three times in four and to 3 once, so
 * the mean is kept).  Reading: between the two grid points bracketing a, go
 * up with probability p = (a - G[lo]) / (G[lo+1] - G[lo]), realised as
 * "up iff k < 256 p"; on-grid values and a >= 6 are deterministic. */
int tqo_sr_index(float a, int k)
{
    if (a >= 6.0f)
        return 7;
    int lo = tqo_e2m1_floor(a);
    if (E2M1_GRID[lo] == (double)a)
        return lo;
    double delta = E2M1_GRID[lo + 1] - E2M1_GRID[lo];
    double p256 = 256.0 * (((double)a - E2M1_GRID[lo]) / delta); /* exact */
    return ((double)k < p256) ? lo + 1 : lo;
}

/*
 * Input: `batch` NVFP4 tensors of rows x cols (blocks of 16 along cols).
 * Output: the transposed tensors, cols x rows, blocks of 16 along the new
 * rows (i.e. down 16 original rows), same tensor scale.
 * [TML] forward/backward-mismatch paragraph: the transpose changes which 16
 * values share a scale, so the values are taken back to higher precision,
 * transposed, and requantized with stochastic rounding.
 *
 * 1. u = +-G[m] * dec(e): exact, in the tensor-scale-normalised domain.
 * 2. Per new block: A' = max|u|, d' = A' / 6, e' = enc(d'); dec(e') = 0 gives
 *    zero codes, else r' = 1 / dec(e').
 * 3. y = u * r', m = SR index of |y| with the element's random byte, sign as Q.
 * 4. The tensor scale is copied.
 * Random byte: element (b, j, r) of the output has linear index
 * i = (b * cols + j) * rows + r.  `first` is the index of tensor 0 of this call
 * within a larger batch, so one tensor of a batch can be recomputed alone: the
 * random bytes use i + first * cols * rows, the outputs are written from 0.
 */
void tqo_requant_transpose_sr(const uint8_t *codes, const uint8_t *scales,
                              const float *tensor_scale, int64_t batch, int64_t rows,
                              int64_t cols, uint64_t seed, uint8_t *codes_t, uint8_t *scales_t,
                              float *tensor_scale_t, int64_t first)
{
    const int64_t per_tensor = rows * cols;
    for (int64_t b = 0; b < batch; ++b) {
        tensor_scale_t[b] = tensor_scale[b];
        for (int64_t j = 0; j < cols; ++j) {          /* output row = input column */
            for (int64_t t = 0; t < rows / 16; ++t) { /* new block along the output row */
                float u[16];
                float A = 0.0f;
                for (int q = 0; q < 16; ++q) {
                    int64_t r = 16 * t + q; /* input row */
                    int64_t src = b * per_tensor + r * cols + j;
                    int code = tqo_get_code(codes, src);
                    float g = (float)E2M1_GRID[code & 7];
                    float d = (float)tqo_e4m3_value(scales[(b * rows + r) * (cols / 16) + j / 16]);
                    float v = g * d;
                    u[q] = (code & 8) ? -v : v;
                    if (fabsf(u[q]) > A)
                        A = fabsf(u[q]);
                }
                float d_new = A / 6.0f;
                uint8_t e_new = tqo_e4m3_encode(d_new);
                scales_t[(b * cols + j) * (rows / 16) + t] = e_new;
                float dec_new = (float)tqo_e4m3_value(e_new);
                for (int q = 0; q < 16; ++q) {
                    int64_t i = (b * cols + j) * rows + 16 * t + q; /* output linear index */
                    int64_t gi = ((first + b) * cols + j) * rows + 16 * t + q; /* in the whole batch */
                    int m = 0;
                    float y = 0.0f;
                    if (dec_new != 0.0f) {
                        float rr = 1.0f / dec_new;
                        y = u[q] * rr;
                        m = tqo_sr_index(fabsf(y), tqo_sr_byte(seed, (uint64_t)gi));
                    }
                    int s = (y < 0.0f && m != 0) ? 1 : 0;
                    put_code(codes_t, i, 8 * s + m);
                }
            }
        }
    }
}

/* ------------------------------------------------------------------------ */
/* M: grouped GEMM with NVFP4 expert weights, in double                       */
/* ------------------------------------------------------------------------ */

/*
 * [TML] summary box and the paragraph on where 4-bit compute goes: the MoE
 * layers' forward runs with NVFP4 operands.  For row i in group e
 * (off[e] <= i < off[e+1]) and column c:
 *   ref[i][c]    = sum_k A[i][k] * W_e[c][k]
 *   abssum[i][c] = sum_k |A[i][k] * W_e[c][k]|
 * with W_e[c][k] = +-G[m] * dec(e_b) * s_t,e evaluated in double (exact) and
 * A read from bf16.  Rows are given explicitly (row_ids, nrows) so a sample of
 * a large problem can be checked; rows outside every group are left as 0.
 */
void tqo_grouped_gemm(const uint16_t *a, const int32_t *group_offsets, int32_t num_groups,
                      int64_t n, int64_t k, const uint8_t *w_codes, const uint8_t *w_scales,
                      const float *w_tensor_scale, const int64_t *row_ids, int64_t nrows,
                      double *ref, double *abssum)
{
    for (int64_t q = 0; q < nrows; ++q) {
        const int64_t i = row_ids[q];
        int e = -1;
        for (int g = 0; g < num_groups; ++g)
            if (group_offsets[g] <= i && i < group_offsets[g + 1]) {
                e = g;
                break;
            }
        for (int64_t c = 0; c < n; ++c) {
            double acc = 0.0, aacc = 0.0;
            if (e >= 0) {
                for (int64_t kk = 0; kk < k; ++kk) {
                    double av = (double)bf16_to_float(a[i * k + kk]);
                    int64_t wi = ((int64_t)e * n + c) * k + kk;
                    int code = tqo_get_code(w_codes, wi);
                    double wv = tqo_e2m1_value(code) *
                                tqo_e4m3_value(w_scales[((int64_t)e * n + c) * (k / 16) + kk / 16]) *
                                (double)w_tensor_scale[e];
                    acc += av * wv;
                    aacc += fabs(av * wv);
                }
            }
            ref[q * n + c] = acc;
            abssum[q * n + c] = aacc;
        }
    }
}

/* W4A4 grouped GEMM: activations NVFP4 as well ([TRACE] results-table
 * paragraph: weights, activations and KV cache all FP4 in the compared
 * rollouts; [TML] summary box: 4-bit forward).  The activations are one NVFP4
 * tensor [m_total][k] (codes, block scales along k, one fp32 tensor scale);
 * each side is dequantized exactly, the product is accumulated in double:
 *   ref[q][c] = sum_k (G[a] dec(sa) s_a) (G[w] dec(sw) s_e). */
void tqo_grouped_gemm_w4a4(const uint8_t *a_codes, const uint8_t *a_scales,
                           const float *a_tensor_scale, const int32_t *group_offsets,
                           int32_t num_groups, int64_t n, int64_t k, const uint8_t *w_codes,
                           const uint8_t *w_scales, const float *w_tensor_scale,
                           const int64_t *row_ids, int64_t nrows, double *ref, double *abssum)
{
    for (int64_t q = 0; q < nrows; ++q) {
        const int64_t i = row_ids[q];
        int e = -1;
        for (int g = 0; g < num_groups; ++g)
            if (group_offsets[g] <= i && i < group_offsets[g + 1]) {
                e = g;
                break;
            }
        for (int64_t c = 0; c < n; ++c) {
            double acc = 0.0, aacc = 0.0;
            if (e >= 0) {
                for (int64_t kk = 0; kk < k; ++kk) {
                    double av = tqo_e2m1_value(tqo_get_code(a_codes, i * k + kk)) *
                                tqo_e4m3_value(a_scales[i * (k / 16) + kk / 16]) *
                                (double)a_tensor_scale[0];
                    int64_t wi = ((int64_t)e * n + c) * k + kk;
                    double wv = tqo_e2m1_value(tqo_get_code(w_codes, wi)) *
                                tqo_e4m3_value(w_scales[((int64_t)e * n + c) * (k / 16) + kk / 16]) *
                                (double)w_tensor_scale[e];
                    acc += av * wv;
                    aacc += fabs(av * wv);
                }
            }
            ref[q * n + c] = acc;
            abssum[q * n + c] = aacc;
        }
    }
}

/* ------------------------------------------------------------------------ */
/* MXFP8: E4M3 elements, one E8M0 scale per 32 values                        */
/* ------------------------------------------------------------------------ */

/* [TML] summary box and format-comparison paragraph: the backward runs in
 * MXFP8 at 8.25 bits per value, i.e. an 8-bit scale per 32 8-bit values.
 * Readings (the usual MX convention): elements E4M3FN, the scale a power of
 * two stored as a biased exponent byte E (value 2^(E-127)), the shared
 * exponent of a block with maximum magnitude A > 0 being floor(log2 A) - 8
 * (8 = exponent of E4M3's largest normal, 448 = 1.75 * 2^8), clamped to
 * [-127, 127]; A = 0 gives E = 0 and zero elements. */
double tqo_e8m0_value(uint8_t e)
{
    return ldexp(1.0, (int)e - 127);
}

static int mx_shared_exp(float A)
{
    int ex;
    frexp((double)A, &ex); /* A = f * 2^ex, f in [0.5, 1): floor(log2 A) = ex - 1 */
    int se = (ex - 1) - 8;
    if (se < -127)
        se = -127;
    if (se > 127)
        se = 127;
    return se;
}

/* E4M3 byte (sign | magnitude code) of y: nearest, ties to even, saturating at
 * 448, zero as +0. */
static uint8_t e4m3_signed_nearest(float y)
{
    uint8_t m = tqo_e4m3_encode(fabsf(y));
    return (uint8_t)((y < 0.0f && m != 0) ? (0x80 | m) : m);
}

/* Nearest MXFP8 quantization of `batch` tensors [rows][cols] (cols % 32 == 0):
 * codes [batch][rows][cols] E4M3 bytes, scales [batch][rows][cols/32] E8M0. */
void tqo_quantize_mxfp8(const void *x, int dtype, int64_t batch, int64_t rows, int64_t cols,
                        uint8_t *codes, uint8_t *scales)
{
    const int64_t nb = cols / 32;
    for (int64_t b = 0; b < batch; ++b)
        for (int64_t r = 0; r < rows; ++r)
            for (int64_t k = 0; k < nb; ++k) {
                const int64_t base = (b * rows + r) * cols + 32 * k;
                float A = 0.0f;
                for (int t = 0; t < 32; ++t) {
                    float v = fabsf(load_x(x, dtype, base + t));
                    if (v > A)
                        A = v;
                }
                const int64_t si = (b * rows + r) * nb + k;
                if (A == 0.0f) {
                    scales[si] = 0;
                    for (int t = 0; t < 32; ++t)
                        codes[base + t] = 0;
                    continue;
                }
                const int se = mx_shared_exp(A);
                scales[si] = (uint8_t)(se + 127);
                for (int t = 0; t < 32; ++t) {
                    /* exact scaling by a power of two (ldexpf), then E4M3 nearest */
                    float y = ldexpf(load_x(x, dtype, base + t), -se);
                    codes[base + t] = e4m3_signed_nearest(y);
                }
            }
}

/* E4M3 stochastic rounding of a >= 0 with random byte k: between the two E4M3
 * values bracketing a, up iff k < 256 (a - lo) / (hi - lo) (the rule of
 * tqo_sr_index on the E4M3 grid); values on the grid are kept and a >= 448
 * gives 448. */
int tqo_e4m3_sr(float a, int k)
{
    if (a >= 448.0f)
        return 0x7E;
    /* lo = largest code with value <= a: the finite codes 0x00..0x7E increase in
     * value with the code, so bisect over them */
    int lo = 0, hi_c = 0x7E;
    while (lo < hi_c) {
        int mid = (lo + hi_c + 1) / 2;
        if (tqo_e4m3_value((uint8_t)mid) <= (double)a)
            lo = mid;
        else
            hi_c = mid - 1;
    }
    double vlo = tqo_e4m3_value((uint8_t)lo);
    if (vlo == (double)a)
        return lo;
    double vhi = tqo_e4m3_value((uint8_t)(lo + 1));
    double p256 = 256.0 * (((double)a - vlo) / (vhi - vlo)); /* exact */
    return ((double)k < p256) ? lo + 1 : lo;
}

/* Backward copy for MXFP8: an NVFP4 tensor [rows][cols] is dequantized exactly
 * (u = +-G[m] dec(e), tensor scale kept aside), transposed, and requantized to
 * MXFP8 along the new rows (blocks of 32 down the old rows) with stochastic
 * rounding ([TML] summary box: MXFP8 backward with requantization and
 * stochastic rounding; forward/backward-mismatch paragraph).  Per new block:
 * se = shared exponent of max|u|, y = u * 2^-se (exact), code = sign | E4M3 SR
 * of |y| with the element's random byte (the stream of tqo_sr_byte at output
 * index i = (b * cols + j) * rows + r, offset by first * cols * rows as in
 * tqo_requant_transpose_sr).  The tensor scale is copied.
 * Requires rows % 32 == 0, cols % 16 == 0.  codes_t [batch][cols][rows],
 * scales_t [batch][cols][rows/32]. */
void tqo_requant_transpose_mxfp8_sr(const uint8_t *codes, const uint8_t *scales,
                                    const float *tensor_scale, int64_t batch, int64_t rows,
                                    int64_t cols, uint64_t seed, uint8_t *codes_t,
                                    uint8_t *scales_t, float *tensor_scale_t, int64_t first)
{
    const int64_t per_tensor = rows * cols;
    for (int64_t b = 0; b < batch; ++b) {
        tensor_scale_t[b] = tensor_scale[b];
        for (int64_t j = 0; j < cols; ++j)
            for (int64_t t = 0; t < rows / 32; ++t) {
                float u[32];
                float A = 0.0f;
                for (int q = 0; q < 32; ++q) {
                    int64_t r = 32 * t + q;
                    int code = tqo_get_code(codes, b * per_tensor + r * cols + j);
                    float v = (float)E2M1_GRID[code & 7] *
                              (float)tqo_e4m3_value(scales[(b * rows + r) * (cols / 16) + j / 16]);
                    u[q] = (code & 8) ? -v : v;
                    if (fabsf(u[q]) > A)
                        A = fabsf(u[q]);
                }
                const int64_t si = (b * cols + j) * (rows / 32) + t;
                const int64_t o = (b * cols + j) * rows + 32 * t;
                const int64_t go = ((first + b) * cols + j) * rows + 32 * t; /* in the whole batch */
                if (A == 0.0f) {
                    scales_t[si] = 0;
                    for (int q = 0; q < 32; ++q)
                        codes_t[o + q] = 0;
                    continue;
                }
                const int se = mx_shared_exp(A);
                scales_t[si] = (uint8_t)(se + 127);
                for (int q = 0; q < 32; ++q) {
                    float y = ldexpf(u[q], -se);
                    int m = tqo_e4m3_sr(fabsf(y), tqo_sr_byte(seed, (uint64_t)(go + q)));
                    codes_t[o + q] = (uint8_t)((y < 0.0f && m != 0) ? (0x80 | m) : m);
                }
            }
    }
}

/* ------------------------------------------------------------------------ */
/* 16x16-tile scaling                                                        */
/* ------------------------------------------------------------------------ */

/* [TML] forward/backward-mismatch paragraph: the 16x16-tile alternative gives
 * one scale to a tile of 16 rows x 16 columns (256 values), so a transpose
 * keeps every value's group; a single large value can zero the rest of its
 * tile.  Steps as Q, with the block maximum taken over the tile: s_t =
 * A_T/2688; per tile d = fl(fl(A_tile/6)/s_t) -> E4M3 e; S = fl(dec(e) s_t),
 * r = fl(1/S); per element the nearest E2M1 code of fl(x r).
 * codes [batch][rows][cols/2] as Q; scales [batch][rows/16][cols/16]. */
void tqo_quantize_tile16(const void *x, int dtype, int64_t batch, int64_t rows, int64_t cols,
                         int amax_given, float *tensor_amax, uint8_t *codes, uint8_t *scales,
                         float *tensor_scale)
{
    const int64_t per_tensor = rows * cols;
    const int64_t tr = rows / 16, tc = cols / 16;
    for (int64_t b = 0; b < batch; ++b) {
        float A_T;
        if (amax_given) {
            A_T = tensor_amax[b];
        } else {
            A_T = 0.0f;
            for (int64_t i = 0; i < per_tensor; ++i) {
                float v = fabsf(load_x(x, dtype, b * per_tensor + i));
                if (v > A_T)
                    A_T = v;
            }
            tensor_amax[b] = A_T;
        }
        float s_t = (A_T == 0.0f) ? 0.0f : A_T / 2688.0f;
        tensor_scale[b] = s_t;
        for (int64_t ti = 0; ti < tr; ++ti) {
            for (int64_t tj = 0; tj < tc; ++tj) {
                float A = 0.0f;
                for (int u = 0; u < 16; ++u)
                    for (int v = 0; v < 16; ++v) {
                        float a = fabsf(load_x(x, dtype, b * per_tensor + (16 * ti + u) * cols + 16 * tj + v));
                        if (a > A)
                            A = a;
                    }
                uint8_t e = 0;
                if (s_t != 0.0f)
                    e = tqo_e4m3_encode((A / 6.0f) / s_t);
                scales[(b * tr + ti) * tc + tj] = e;
                float dec = (float)tqo_e4m3_value(e);
                float r = dec == 0.0f ? 0.0f : 1.0f / (dec * s_t);
                for (int u = 0; u < 16; ++u)
                    for (int v = 0; v < 16; ++v) {
                        int64_t i = b * per_tensor + (16 * ti + u) * cols + 16 * tj + v;
                        int code = 0;
                        if (dec != 0.0f) {
                            float y = load_x(x, dtype, i) * r;
                            int m = tqo_e2m1_nearest(fabsf(y));
                            code = ((y < 0.0f && m != 0) ? 8 : 0) + m;
                        }
                        put_code(codes, i, code);
                    }
            }
        }
    }
}

/* Transpose of a 16x16-tile NVFP4 tensor: every value keeps its tile, so codes
 * and tile scales are moved, nothing is requantized.  codes_t [batch][cols][rows/2],
 * scales_t [batch][cols/16][rows/16], tensor scale copied. */
void tqo_transpose_tile16(const uint8_t *codes, const uint8_t *scales, const float *tensor_scale,
                          int64_t batch, int64_t rows, int64_t cols, uint8_t *codes_t,
                          uint8_t *scales_t, float *tensor_scale_t)
{
    const int64_t tr = rows / 16, tc = cols / 16;
    for (int64_t b = 0; b < batch; ++b) {
        tensor_scale_t[b] = tensor_scale[b];
        for (int64_t r = 0; r < rows; ++r)
            for (int64_t c = 0; c < cols; ++c)
                put_code(codes_t, (b * cols + c) * rows + r,
                         tqo_get_code(codes, (b * rows + r) * cols + c));
        for (int64_t ti = 0; ti < tr; ++ti)
            for (int64_t tj = 0; tj < tc; ++tj)
                scales_t[(b * tc + tj) * tr + ti] = scales[(b * tr + ti) * tc + tj];
    }
}

/* ------------------------------------------------------------------------ */
/* Mismatch statistics                                                       */
/* ------------------------------------------------------------------------ */

/* [TRACE] compact-guidance paragraph: mismatches are counted per element and
 * are almost always one bin apart.  counts[2b] = #{i : a_i != b_i};
 * counts[2b+1] = #{i : |ord(a_i) - ord(b_i)| == 1} with ord(code) the signed
 * grid position (-m for negative codes, +m otherwise). */
void tqo_code_mismatch(const uint8_t *codes_a, const uint8_t *codes_b, int64_t batch,
                       int64_t per_tensor, uint64_t *counts)
{
    for (int64_t b = 0; b < batch; ++b) {
        uint64_t mism = 0, adj = 0;
        for (int64_t t = 0; t < per_tensor; ++t) {
            int64_t i = b * per_tensor + t;
            int ca = tqo_get_code(codes_a, i), cb = tqo_get_code(codes_b, i);
            if (ca != cb) {
                ++mism;
                int oa = (ca & 8) ? -(ca & 7) : (ca & 7);
                int ob = (cb & 8) ? -(cb & 7) : (cb & 7);
                if (oa - ob == 1 || ob - oa == 1)
                    ++adj;
            }
        }
        counts[2 * b] = mism;
        counts[2 * b + 1] = adj;
    }
}

/* ------------------------------------------------------------------------ */
/* Array forms of the scalar rules (plain loops, used by dense pin sweeps)   */
/* ------------------------------------------------------------------------ */

void tqo_e4m3_encode_array(const float *d, int64_t n, uint8_t *out)
{
    for (int64_t i = 0; i < n; ++i)
        out[i] = tqo_e4m3_encode(d[i]);
}

void tqo_e2m1_nearest_array(const float *a, int64_t n, uint8_t *out)
{
    for (int64_t i = 0; i < n; ++i)
        out[i] = (uint8_t)tqo_e2m1_nearest(a[i]);
}
