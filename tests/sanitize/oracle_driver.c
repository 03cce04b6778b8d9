/* Drives the oracle's C functions (oracle/fp4q_oracle.c) under the address
 * and undefined-behaviour sanitizers on heap buffers of exactly the sizes
 * each call needs: every layout, rounding, block size and scale format on
 * ragged and empty shapes, bf16 and fp32 inputs with a row stride, SR index
 * origins, both decodes, the GEMM loops and the probe-matched GEMM; plus
 * every code of each codec and a sweep of binary32 inputs through the
 * encoders. Exits non-zero on a failed consistency check; the sanitizers
 * abort on any out-of-bounds access or undefined operation. */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

double oracle_e2m1_decode(int code);
double oracle_ue5m3_decode(int code);
int oracle_ue5m3_encode(float raw, int *flags);
double oracle_e4m3_decode(int code);
int oracle_e4m3_encode(float raw, int *flags);
int oracle_e2m1_encode_rne(float v, int negative);
int oracle_e2m1_encode_sr(float v, int negative, uint32_t w);
uint32_t oracle_sr_word(uint64_t seed, uint32_t subseq, uint64_t i);
float oracle_amax(const void *x, int dtype, int64_t rows, int64_t cols, int64_t ld);
float oracle_tensor_scale(float amax, float T);
int oracle_quantize_fmt(const void *x, int dtype, int64_t rows, int64_t cols, int64_t ld, float amax_held,
                        float T, int layout, int block, int scale_fmt, int rnd, uint64_t seed, uint32_t subseq,
                        int64_t idx_row0, int64_t idx_col0, int64_t idx_cols, uint8_t *codes, uint8_t *scales,
                        float *enc_scale_out, uint8_t *codes_t, uint8_t *scales_t, int32_t *diag);
void oracle_decode_f64_fmt(const uint8_t *codes, const uint8_t *scales, int64_t rows, int64_t cols, int layout,
                           int block, int scale_fmt, double *out);
void oracle_dequant_f32_fmt(const uint8_t *codes, const uint8_t *scales, int64_t rows, int64_t cols, int layout,
                            int block, int scale_fmt, float S, float *out);
void oracle_gemm_f64_loops(const double *a, const double *b, int64_t m, int64_t n, int64_t k, double sa,
                           double sb, double *y);
int oracle_gemm_probe(const double *a, const double *b, int64_t m, int64_t n, int64_t k, float sa, float sb,
                      int snap_log2, float *y);

static int fails = 0;
#define CHECK(c, ...) do { if (!(c)) { fprintf(stderr, __VA_ARGS__); fputc('\n', stderr); fails++; } } while (0)

static uint64_t rs = 88172645463325252ull;
static uint64_t rnd64(void) { rs ^= rs << 13; rs ^= rs >> 7; rs ^= rs << 17; return rs; }
static float rndf(float scale) {
    const double u = (double)(rnd64() >> 11) / 9007199254740992.0;
    const double t = tan(3.14159265 * (u - 0.5)); /* heavy tails */
    return (float)(scale * t);
}

/* one quantization on exactly sized buffers; the decoded operand is checked
 * against the source's sign pattern */
static void quantize_case(int64_t rows, int64_t cols, int64_t pad, int dtype, int layout, int block, int fmt,
                          int rnd, int transposed) {
    const int es = dtype == 0 ? 4 : 2;
    const int64_t ld = cols + pad;
    uint8_t *x = malloc((size_t)(rows * ld * es) + 1);
    for (int64_t i = 0; i < rows * ld; ++i) {
        float v = rndf(1.0f);
        if (es == 4) memcpy(x + i * 4, &v, 4);
        else { uint32_t u; memcpy(&u, &v, 4); uint16_t h = (uint16_t)(u >> 16); memcpy(x + i * 2, &h, 2); }
    }
    const int col = layout == 1;
    const int64_t orows = col ? cols : rows, ocols = col ? rows : cols;
    const size_t ncodes = (size_t)(orows * (ocols / 2));
    const size_t nscales = layout == 2 ? (size_t)((rows / block) * (cols / block)) : (size_t)(orows * (ocols / block));
    uint8_t *codes = malloc(ncodes + 1), *scales = malloc(nscales + 1);
    uint8_t *codes_t = NULL, *scales_t = NULL;
    if (layout == 2 && transposed) {
        codes_t = malloc(ncodes + 1);
        scales_t = malloc(nscales + 1);
    }
    float S;
    int32_t diag[2];
    const float amax = oracle_amax(x, dtype, rows, cols, ld);
    int rc = oracle_quantize_fmt(x, dtype, rows, cols, ld, amax, 448.0f, layout, block, fmt, rnd, 0x1234567ull, 5,
                                 3, 7, cols + 11, codes, scales, &S, codes_t, scales_t, diag);
    CHECK(rc == 0, "quantize rc %d (%lld x %lld layout %d block %d)", rc, (long long)rows, (long long)cols, layout,
          block);
    if (rc == 0 && rows > 0 && cols > 0) {
        double *dec = malloc((size_t)(orows * ocols) * sizeof(double) + 1);
        float *deq = malloc((size_t)(orows * ocols) * sizeof(float) + 1);
        const int qlayout = layout == 2 ? 2 : 0;
        oracle_decode_f64_fmt(codes, scales, orows, ocols, qlayout, block, fmt, dec);
        oracle_dequant_f32_fmt(codes, scales, orows, ocols, qlayout, block, fmt, S, deq);
        if (codes_t) {
            oracle_decode_f64_fmt(codes_t, scales_t, cols, rows, 2, block, fmt, dec);
        }
        free(dec);
        free(deq);
    }
    free(x); free(codes); free(scales); free(codes_t); free(scales_t);
}

int main(void) {
    /* every code of each codec */
    for (int c = 0; c < 16; ++c) CHECK(fabs(oracle_e2m1_decode(c)) <= 6.0, "e2m1 %d", c);
    for (int c = 0; c < 256; ++c) { (void)oracle_ue5m3_decode(c); (void)oracle_e4m3_decode(c); }
    /* encoders over a sweep of binary32 values, special values included */
    const float specials[] = {0.0f, -0.0f, 1e-45f, -1e-45f, 1e-38f, 0.25f, 0.75f, 5.0f, 6.0f, 7.0f, 61440.0f,
                              1e30f, INFINITY, -INFINITY, NAN};
    for (size_t i = 0; i < sizeof specials / sizeof specials[0]; ++i) {
        int f;
        (void)oracle_ue5m3_encode(fabsf(specials[i]), &f);
        (void)oracle_e4m3_encode(fabsf(specials[i]), &f);
        (void)oracle_e2m1_encode_rne(specials[i], signbit(specials[i]) != 0);
        (void)oracle_e2m1_encode_sr(specials[i], signbit(specials[i]) != 0, 0u);
        (void)oracle_e2m1_encode_sr(specials[i], signbit(specials[i]) != 0, 0xFFFFFFFFu);
    }
    for (uint32_t u = 0; u < 0x7F800000u; u += 0x1FF7u) {
        float v; memcpy(&v, &u, 4);
        int f;
        int c = oracle_ue5m3_encode(v, &f);
        CHECK(c >= 1 && c <= 0xF7, "ue5m3 code %d", c);
        (void)oracle_e4m3_encode(v, &f);
        c = oracle_e2m1_encode_rne(v, 0);
        CHECK(c >= 0 && c <= 7, "rne code %d", c);
        c = oracle_e2m1_encode_sr(v, 1, u * 2654435761u);
        CHECK(c >= 8 && c <= 15, "sr code %d", c);
    }
    (void)oracle_sr_word(~0ull, ~0u, ~0ull);
    CHECK(oracle_tensor_scale(0.0f, 448.0f) == 1.0f, "tensor scale of a zero amax");
    CHECK(oracle_tensor_scale(INFINITY, 448.0f) == 1.0f, "tensor scale of an infinite amax");
    (void)oracle_tensor_scale(1e-45f, 2048.0f);

    /* quantize: layouts x roundings x blocks x formats x dtypes on ragged and empty shapes */
    const int64_t shapes[][2] = {{0, 64}, {1, 32}, {33, 96}, {64, 160}, {96, 64}, {32, 0}};
    for (size_t s = 0; s < sizeof shapes / sizeof shapes[0]; ++s)
        for (int layout = 0; layout < 3; ++layout)
            for (int block = 16; block <= 32; block += 16)
                for (int fmt = 0; fmt < 2; ++fmt)
                    for (int rnd = 0; rnd < 2; ++rnd)
                        for (int dtype = 0; dtype < 2; ++dtype) {
                            int64_t r = shapes[s][0], c = shapes[s][1];
                            if (layout != 1 && c % block) continue;
                            if (layout != 0 && r % block) continue;
                            if (layout == 1 && c % 2) continue;
                            quantize_case(r, c, dtype ? 8 : 3, dtype, layout, block, fmt, rnd, 1);
                        }

    /* GEMM loops and the probe-matched GEMM on lattice values (decoded codes) */
    const int64_t m = 17, n = 9, k = 200;
    double *a = malloc((size_t)(m * k) * sizeof(double)), *b = malloc((size_t)(n * k) * sizeof(double));
    for (int64_t i = 0; i < m * k; ++i) a[i] = oracle_e2m1_decode((int)(rnd64() & 15)) * ldexp(1.0, (int)(rnd64() % 20) - 10);
    for (int64_t i = 0; i < n * k; ++i) b[i] = oracle_e2m1_decode((int)(rnd64() & 15)) * ldexp(1.0, (int)(rnd64() % 20) - 10);
    double *y = malloc((size_t)(m * n) * sizeof(double));
    float *yp = malloc((size_t)(m * n) * sizeof(float));
    oracle_gemm_f64_loops(a, b, m, n, k, 448.0, 3.0, y);
    for (int snap = 0; snap <= 10; snap += 10) CHECK(oracle_gemm_probe(a, b, m, n, k, 448.0f, 3.0f, snap, yp) == 0, "probe");
    CHECK(oracle_gemm_probe(a, b, m, n, 0, 1.0f, 1.0f, 0, yp) == 0, "probe K = 0");
    free(a); free(b); free(y); free(yp);

    printf("oracle driver: %s\n", fails ? "FAILED" : "ok");
    return fails != 0;
}
