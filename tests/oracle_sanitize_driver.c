/* Test driver: calls every routine of oracle/tq_oracle.c on small shapes,
 * with each buffer allocated at exactly the size its layout gives, so that a
 * build with AddressSanitizer and UndefinedBehaviorSanitizer reports any read or
 * write outside a buffer and any undefined operation.  Test infrastructure
 * only: it links the oracle, and nothing else, and prints "ok" at the end. */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

double tqo_e2m1_value(int code);
double tqo_e4m3_value(uint8_t b);
uint8_t tqo_e4m3_encode(float d);
int tqo_e2m1_nearest(float a);
int tqo_e2m1_floor(float a);
int tqo_get_code(const uint8_t *codes, int64_t i);
void tqo_tensor_amax(const void *x, int dtype, int64_t batch, int64_t per_tensor, float *amax);
void tqo_quantize(const void *x, int dtype, int64_t batch, int64_t rows, int64_t cols, int amax_given,
                  float *tensor_amax, uint8_t *codes, uint8_t *scales, float *tensor_scale);
void tqo_quantize_guided(const void *x, int dtype, int64_t batch, int64_t rows, int64_t cols,
                         int amax_given, float *tensor_amax, const uint32_t *hints, uint8_t *codes,
                         uint8_t *scales, float *tensor_scale);
void tqo_extract_hint(const uint8_t *codes, int64_t n, uint32_t *hints);
int tqo_hint_first_layer(int num_layers);
void tqo_dequantize(const uint8_t *codes, const uint8_t *scales, const float *tensor_scale,
                    int64_t batch, int64_t rows, int64_t cols, float *out);
void tqo_philox4x32_10(const uint32_t ctr_in[4], const uint32_t key_in[2], uint32_t out[4]);
int tqo_sr_byte(uint64_t seed, uint64_t i);
int tqo_sr_index(float a, int k);
void tqo_requant_transpose_sr(const uint8_t *codes, const uint8_t *scales, const float *tensor_scale,
                              int64_t batch, int64_t rows, int64_t cols, uint64_t seed,
                              uint8_t *codes_t, uint8_t *scales_t, float *tensor_scale_t, int64_t first);
void tqo_grouped_gemm(const uint16_t *a, const int32_t *group_offsets, int32_t num_groups, int64_t n,
                      int64_t k, const uint8_t *w_codes, const uint8_t *w_scales,
                      const float *w_tensor_scale, const int64_t *row_ids, int64_t nrows,
                      double *ref, double *abssum);
void tqo_grouped_gemm_w4a4(const uint8_t *a_codes, const uint8_t *a_scales,
                           const float *a_tensor_scale, const int32_t *group_offsets,
                           int32_t num_groups, int64_t n, int64_t k, const uint8_t *w_codes,
                           const uint8_t *w_scales, const float *w_tensor_scale,
                           const int64_t *row_ids, int64_t nrows, double *ref, double *abssum);
double tqo_e8m0_value(uint8_t e);
void tqo_quantize_mxfp8(const void *x, int dtype, int64_t batch, int64_t rows, int64_t cols,
                        uint8_t *codes, uint8_t *scales);
int tqo_e4m3_sr(float a, int k);
void tqo_requant_transpose_mxfp8_sr(const uint8_t *codes, const uint8_t *scales,
                                    const float *tensor_scale, int64_t batch, int64_t rows,
                                    int64_t cols, uint64_t seed, uint8_t *codes_t,
                                    uint8_t *scales_t, float *tensor_scale_t, int64_t first);
void tqo_quantize_tile16(const void *x, int dtype, int64_t batch, int64_t rows, int64_t cols,
                         int amax_given, float *tensor_amax, uint8_t *codes, uint8_t *scales,
                         float *tensor_scale);
void tqo_transpose_tile16(const uint8_t *codes, const uint8_t *scales, const float *tensor_scale,
                          int64_t batch, int64_t rows, int64_t cols, uint8_t *codes_t,
                          uint8_t *scales_t, float *tensor_scale_t);
void tqo_code_mismatch(const uint8_t *codes_a, const uint8_t *codes_b, int64_t batch,
                       int64_t per_tensor, uint64_t *counts);
void tqo_e4m3_encode_array(const float *d, int64_t n, uint8_t *out);
void tqo_e2m1_nearest_array(const float *a, int64_t n, uint8_t *out);

static uint64_t rng_state = 0x9E3779B97F4A7C15ull;
static uint32_t rnd(void)
{
    rng_state ^= rng_state << 13;
    rng_state ^= rng_state >> 7;
    rng_state ^= rng_state << 17;
    return (uint32_t)(rng_state >> 11);
}

/* a buffer of exactly n bytes (never 0), filled with a byte pattern */
static void *buf(size_t n)
{
    unsigned char *p = malloc(n ? n : 1);
    if (!p) {
        fprintf(stderr, "out of memory\n");
        exit(2);
    }
    for (size_t i = 0; i < n; ++i)
        p[i] = (unsigned char)rnd();
    return p;
}

/* n random finite floats: mixed magnitudes, some zeros, some exact grid points */
static float *floats(int64_t n)
{
    float *x = buf((size_t)n * sizeof(float));
    for (int64_t i = 0; i < n; ++i) {
        const uint32_t r = rnd();
        float v = (float)((int32_t)(r & 0xFFFF) - 32768) / 4096.0f;
        if ((r >> 16) % 13 == 0)
            v = 0.0f;
        else if ((r >> 16) % 11 == 0)
            v = (float)((r >> 20) % 7) * 0.5f;
        else if ((r >> 16) % 7 == 0)
            v *= 1e-30f;
        x[i] = v;
    }
    return x;
}

/* bf16 bit patterns of floats (truncation is enough for a driver) */
static uint16_t *bf16_of(const float *x, int64_t n)
{
    uint16_t *b = buf((size_t)n * 2);
    for (int64_t i = 0; i < n; ++i) {
        uint32_t u;
        memcpy(&u, &x[i], 4);
        b[i] = (uint16_t)(u >> 16);
    }
    return b;
}

static void quantizers(int dtype, int64_t B, int64_t R, int64_t C)
{
    const int64_t n = B * R * C;
    float *xf = floats(n);
    void *x = dtype == 0 ? (void *)xf : (void *)bf16_of(xf, n);
    float *amax = buf((size_t)B * 4), *ts = buf((size_t)B * 4), *deq = buf((size_t)n * 4);
    uint8_t *codes = buf((size_t)n / 2), *scales = buf((size_t)n / 16);
    uint8_t *codes_g = buf((size_t)n / 2), *scales_g = buf((size_t)n / 16);
    uint32_t *hints = buf((size_t)((n + 31) / 32) * 4);
    uint64_t *counts = buf((size_t)B * 2 * 8);
    tqo_tensor_amax(x, dtype, B, R * C, amax);
    tqo_quantize(x, dtype, B, R, C, 0, amax, codes, scales, ts);
    tqo_quantize(x, dtype, B, R, C, 1, amax, codes, scales, ts);
    tqo_extract_hint(codes, n, hints);
    tqo_quantize_guided(x, dtype, B, R, C, 1, amax, hints, codes_g, scales_g, ts);
    tqo_quantize_guided(x, dtype, B, R, C, 0, amax, NULL, codes_g, scales_g, ts);
    tqo_dequantize(codes, scales, ts, B, R, C, deq);
    tqo_code_mismatch(codes, codes_g, B, R * C, counts);
    if (R % 16 == 0) {
        uint8_t *ct = buf((size_t)n / 2), *st = buf((size_t)n / 16);
        float *tst = buf((size_t)B * 4);
        tqo_requant_transpose_sr(codes, scales, ts, B, R, C, 7u, ct, st, tst, 0);
        tqo_requant_transpose_sr(codes, scales, ts, B, R, C, 0x10000000Bull, ct, st, tst, 3);
        uint8_t *q16 = buf((size_t)n / 2), *s16 = buf((size_t)(R / 16) * (C / 16) * B);
        uint8_t *q16t = buf((size_t)n / 2), *s16t = buf((size_t)(R / 16) * (C / 16) * B);
        tqo_quantize_tile16(x, dtype, B, R, C, 1, amax, q16, s16, ts);
        tqo_transpose_tile16(q16, s16, ts, B, R, C, q16t, s16t, tst);
        free(ct), free(st), free(tst), free(q16), free(s16), free(q16t), free(s16t);
        if (R % 32 == 0) {
            uint8_t *mc = buf((size_t)n), *ms = buf((size_t)n / 32);
            tqo_requant_transpose_mxfp8_sr(codes, scales, ts, B, R, C, 5u, mc, ms, ts, 2);
            free(mc), free(ms);
        }
    }
    if (C % 32 == 0) {
        uint8_t *mc = buf((size_t)n), *ms = buf((size_t)n / 32);
        tqo_quantize_mxfp8(x, dtype, B, R, C, mc, ms);
        free(mc), free(ms);
    }
    if (dtype == 1)
        free(x);
    free(xf), free(amax), free(ts), free(deq), free(codes), free(scales), free(codes_g),
        free(scales_g), free(hints), free(counts);
}

static void gemms(void)
{
    /* groups of 2, 0 and 3 rows; n = 6, k = 48 */
    const int32_t G = 3, off[4] = {0, 2, 2, 5};
    const int64_t M = 5, N = 6, K = 48;
    float *af = floats(M * K);
    uint16_t *a = bf16_of(af, M * K);
    float *wf = floats(G * N * K);
    uint8_t *wc = buf((size_t)G * N * K / 2), *ws = buf((size_t)G * N * K / 16);
    float *wamax = buf((size_t)G * 4), *wts = buf((size_t)G * 4);
    tqo_quantize(wf, 0, G, N, K, 0, wamax, wc, ws, wts);
    int64_t *rows = buf((size_t)M * 8);
    for (int64_t i = 0; i < M; ++i)
        rows[i] = M - 1 - i;
    double *ref = buf((size_t)M * N * 8), *asum = buf((size_t)M * N * 8);
    tqo_grouped_gemm(a, off, G, N, K, wc, ws, wts, rows, M, ref, asum);
    uint8_t *ac = buf((size_t)M * K / 2), *as = buf((size_t)M * K / 16);
    float *aamax = buf(4), *ats = buf(4);
    tqo_quantize(af, 0, 1, M, K, 0, aamax, ac, as, ats);
    tqo_grouped_gemm_w4a4(ac, as, ats, off, G, N, K, wc, ws, wts, rows, M, ref, asum);
    free(af), free(a), free(wf), free(wc), free(ws), free(wamax), free(wts), free(rows), free(ref),
        free(asum), free(ac), free(as), free(aamax), free(ats);
}

int main(void)
{
    quantizers(0, 1, 1, 16);
    quantizers(0, 2, 3, 32);
    quantizers(1, 1, 5, 48);
    quantizers(0, 2, 32, 48);
    quantizers(1, 3, 16, 64);
    quantizers(1, 1, 64, 32);
    gemms();
    /* scalar routines over their whole input ranges */
    for (int c = 0; c < 16; ++c)
        (void)tqo_e2m1_value(c);
    for (int b = 0; b < 256; ++b) {
        (void)tqo_e4m3_value((uint8_t)b);
        (void)tqo_e8m0_value((uint8_t)b);
        (void)tqo_sr_index(2.25f, b);
        (void)tqo_e4m3_sr(0.3f + 0.01f * (float)b, b);
    }
    float *d = floats(4096);
    for (int64_t i = 0; i < 4096; ++i)
        d[i] = d[i] < 0 ? -d[i] : d[i];
    uint8_t *e = buf(4096);
    tqo_e4m3_encode_array(d, 4096, e);
    tqo_e2m1_nearest_array(d, 4096, e);
    for (int64_t i = 0; i < 4096; ++i) {
        (void)tqo_e4m3_encode(d[i]);
        (void)tqo_e2m1_nearest(d[i]);
        (void)tqo_e2m1_floor(d[i]);
    }
    (void)tqo_get_code(e, 4095);
    uint32_t ctr[4] = {1, 2, 3, 4}, key[2] = {5, 6}, out[4];
    tqo_philox4x32_10(ctr, key, out);
    (void)tqo_sr_byte(0xFFFFFFFFFFFFFFFFull, 0xFFFFFFFFFull);
    (void)tqo_hint_first_layer(48);
    free(d), free(e);
    printf("ok\n");
    return 0;
}
