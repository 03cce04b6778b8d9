/*
 * fp4q oracle: a plain, slow, scalar CPU implementation of the block-scaled
 * FP4 codec (E2M1 payloads, unsigned-E5M3 block scales, FP32 tensor scale)
 * and of the dequantized-operand linear layer built on it.
 *
 * TEST INFRASTRUCTURE ONLY. The test suite, the package smoke check and the
 * benchmark's CPU-baseline leg are the only users. It shares no source with
 * the HIP library and is never a fallback for it.
 *
 * Arithmetic rules: a step stated as a binary32 operation is written as one C
 * float operation (this file is compiled with -ffp-contract=off and without
 * fast-math, so nothing is fused or reassociated). Every rounding decision
 * (nearest code, tie to even, stochastic choice) is written as a plain search
 * over the decoded codebook, not as bit manipulation.
 *
 * Sources, cited by page title and section:
 *   [UE5M3] "UE5M3 FP4 Block Scaling for Stable Language Model Pretraining"
 *   [RPS]   "Rounding in Preconditioner Space: Redesigning 4-bit AdamW
 *            Optimizer-State Quantization"
 *   [GWS]   "Gaussian Weight Sampling for Scalable, Efficient and Stable
 *            Pseudo-Quantization Training"
 * Readings taken where the pages are silent are marked READING.
 */
#include <fenv.h>
#include <float.h>
#include <math.h>
#include <stdint.h>
#include <string.h>

#define ORACLE_F32 0
#define ORACLE_BF16 1

#define ORACLE_ROW16 0
#define ORACLE_COL16 1
#define ORACLE_TILE16 2

#define ORACLE_RNE 0
#define ORACLE_SR 1

int oracle_abi_version(void) { return 1; }

/* ------------------------------------------------------------------------
 * E2M1 payload. [UE5M3] §3 (FP4 microscaling): 1 sign, 2 exponent and 1
 * mantissa bit, no Inf or NaN. [RPS] App. A.1 prints the normalised E2M1
 * codebook; times 6 its normal magnitudes are 1, 1.5, 2, 3, 4, 6.
 * READING: exponent field 0 is the subnormal binade holding 0 and 0.5, as in
 * the NVFP4/MXFP4 E2M1 the UE5M3 page builds on (the bitsandbytes codebook on
 * the optimizer page differs only there).
 * ---------------------------------------------------------------------- */
static double e2m1_magnitude(int mag3)
{
    int e = (mag3 >> 1) & 3;
    int m = mag3 & 1;
    if (e == 0)
        return 0.5 * m;
    return (1.0 + 0.5 * m) * ldexp(1.0, e - 1);
}

double oracle_e2m1_decode(int code)
{
    double v = e2m1_magnitude(code & 7);
    return (code & 8) ? -v : v;
}

/* ------------------------------------------------------------------------
 * UE5M3 block scale. [UE5M3] §4.1: the sign bit of a non-negative scale is
 * reused as a fifth exponent bit, three fraction bits stay. The page prints
 * 2^-14 as the smallest normal and 2^-17 as the smallest subnormal, which
 * fixes an exponent bias of 15; §5.2 prints 61,440 as the largest scale,
 * which is only true if exponent field 31 holds no finite value (Inf for a
 * zero fraction, NaN otherwise).
 * ---------------------------------------------------------------------- */
double oracle_ue5m3_decode(int code)
{
    int e = (code >> 3) & 31;
    int m = code & 7;
    if (e == 31)
        return m == 0 ? INFINITY : NAN;
    if (e == 0)
        return m * ldexp(1.0, -17);
    return (1.0 + m / 8.0) * ldexp(1.0, e - 15);
}

#define UE5M3_MAX_FINITE_CODE 0xF7
/* The value an unbounded exponent would place just above 61,440. */
#define UE5M3_BEYOND_MAX 65536.0

/*
 * Nearest UE5M3 code to raw >= 0, ties to the even code, before any repair.
 * Returns 0xF8 when raw rounds above the largest finite value (the nearest
 * point of the codebook extended by 2^16 is 2^16), i.e. when it would
 * overflow. Differences are taken in double: every candidate and raw are
 * binary32 numbers, so the comparison order is exact wherever a tie or a near
 * tie can occur.
 */
static int ue5m3_nearest_prerepair(float raw)
{
    double x = raw;
    if (x > UE5M3_BEYOND_MAX)
        return 0xF8;
    int best = 0;
    double bestd = fabs(x);
    for (int c = 1; c <= 0xF8; ++c) {
        double v = (c == 0xF8) ? UE5M3_BEYOND_MAX : oracle_ue5m3_decode(c);
        double d = fabs(x - v);
        if (d < bestd || (d == bestd && (c & 1) == 0)) {
            best = c;
            bestd = d;
        }
    }
    return best;
}

/*
 * Scale encode with repair. READING of [UE5M3] §5.3, which counts scale
 * codes that were zero-rounded or saturated before repair: a scale that
 * rounds to zero for a non-zero block becomes the smallest positive code
 * 0x01; a scale
 * that rounds above the largest finite value becomes 0xF7 (61,440).
 * flags bit 0: zero-rounded before repair, bit 1: saturated before repair.
 */
int oracle_ue5m3_encode(float raw, int *flags)
{
    int c = ue5m3_nearest_prerepair(raw);
    int f = 0;
    if (c == 0) {
        c = 0x01;
        f |= 1;
    } else if (c == 0xF8) {
        c = UE5M3_MAX_FINITE_CODE;
        f |= 2;
    }
    if (flags)
        *flags = f;
    return c;
}

/* Pre-repair code, exposed for the codebook tests. */
int oracle_ue5m3_nearest(float raw) { return ue5m3_nearest_prerepair(raw); }

/* ------------------------------------------------------------------------
 * E4M3 block scale, NVFP4's ([UE5M3] §3; §4.1 compares it with UE5M3): one
 * sign bit, four exponent bits with bias 7, three fraction bits; exponent
 * field 15 with fraction 7 is NaN, so the largest finite value is 448 and the
 * smallest subnormal 2^-9 (the ratios 61,440 / 448 ~ 137 and 2^-9 / 2^-17 =
 * 256 that §4.1 prints). Block scales are non-negative: codes 0x00..0x7E.
 * Encode and repair follow the UE5M3 rules above: nearest with ties to the
 * even code, a scale rounding to zero becomes 0x01 (2^-9), one rounding
 * above 448 (the next point of an unbounded codebook being 480) becomes
 * 0x7E.
 * ---------------------------------------------------------------------- */
double oracle_e4m3_decode(int code)
{
    int sgn = (code >> 7) & 1;
    int e = (code >> 3) & 15;
    int m = code & 7;
    if (e == 15 && m == 7)
        return NAN;
    double v = (e == 0) ? m * ldexp(1.0, -9) : (1.0 + m / 8.0) * ldexp(1.0, e - 7);
    return sgn ? -v : v;
}

#define E4M3_MAX_FINITE_CODE 0x7E
#define E4M3_BEYOND_MAX 480.0

static int e4m3_nearest_prerepair(float raw)
{
    double x = raw;
    if (x > E4M3_BEYOND_MAX)
        return 0x7F;
    int best = 0;
    double bestd = fabs(x);
    for (int c = 1; c <= 0x7F; ++c) {
        double v = (c == 0x7F) ? E4M3_BEYOND_MAX : oracle_e4m3_decode(c);
        double d = fabs(x - v);
        if (d < bestd || (d == bestd && (c & 1) == 0)) {
            best = c;
            bestd = d;
        }
    }
    return best;
}

int oracle_e4m3_encode(float raw, int *flags)
{
    int c = e4m3_nearest_prerepair(raw);
    int f = 0;
    if (c == 0) {
        c = 0x01;
        f |= 1;
    } else if (c == 0x7F) {
        c = E4M3_MAX_FINITE_CODE;
        f |= 2;
    }
    if (flags)
        *flags = f;
    return c;
}

#define ORACLE_UE5M3 0
#define ORACLE_E4M3 1

static double scale_decode(int fmt, int code)
{
    return fmt == ORACLE_E4M3 ? oracle_e4m3_decode(code) : oracle_ue5m3_decode(code);
}

static int scale_encode(int fmt, float raw, int *flags)
{
    return fmt == ORACLE_E4M3 ? oracle_e4m3_encode(raw, flags) : oracle_ue5m3_encode(raw, flags);
}

/* ------------------------------------------------------------------------
 * E2M1 payload rounding.
 * RNE: [UE5M3] §2 (saved activations rounded to nearest even) and [RPS] App. A.2
 * (RTN with a predetermined tie rule; here: the even code). Values beyond
 * the largest magnitude saturate to 6 ([UE5M3] §3: oversized values
 * saturate). READING: a NaN scaled value, which only arises as 0 * Inf when
 * the per-block multiplier overflows, encodes as zero. The sign bit is the
 * input's sign bit (so -0 and negative underflow give code 0x8).
 * ---------------------------------------------------------------------- */
int oracle_e2m1_encode_rne(float v, int negative)
{
    int s = negative ? 8 : 0;
    if (isnan(v))
        return s;
    double a = fabs((double)v);
    if (a > 6.0)
        return s | 7;
    int best = 0;
    double bestd = a;
    for (int q = 1; q < 8; ++q) {
        double d = fabs(a - e2m1_magnitude(q));
        if (d < bestd || (d == bestd && (q & 1) == 0)) {
            best = q;
            bestd = d;
        }
    }
    return s | best;
}

/*
 * SR: [UE5M3] §5.2 (unbiased randomized choice between adjacent representable
 * values; too few random bits can bias it) and [RPS] App. A.2 Definition 5
 * (the lower endpoint is taken with probability 1 - p, p the position of the
 * input between the endpoints; inputs on a level stay; inputs outside the
 * range go to the nearer endpoint).
 * READING: 32 random bits per element; the value rounds up in magnitude iff
 * the word w < ceil(p * 2^32), p = (a - lo) / (hi - lo) computed in binary32
 * (exact here: a - lo is exact because lo <= a < hi <= 2 lo or lo = 0, and
 * hi - lo is a power of two).
 */
int oracle_e2m1_encode_sr(float v, int negative, uint32_t w)
{
    int s = negative ? 8 : 0;
    if (isnan(v))
        return s;
    float a = fabsf(v);
    if (a >= 6.0f)
        return s | 7;
    int q = 0;
    while (!((double)a < e2m1_magnitude(q + 1)))
        ++q;
    float lo = (float)e2m1_magnitude(q);
    float hi = (float)e2m1_magnitude(q + 1);
    float p = (a - lo) / (hi - lo);
    double threshold = ceil((double)p * 4294967296.0);
    int up = (double)w < threshold;
    return s | (up ? q + 1 : q);
}

/* ------------------------------------------------------------------------
 * Philox4x32-10, the counter-based generator [GWS] §3.4 names (Salmon et al.,
 * "Parallel random numbers: as easy as 1, 2, 3", SC'11). Ten rounds; each
 * round multiplies counter words 0 and 2 by two fixed 32-bit multipliers,
 * takes the 64-bit products apart and mixes the high halves with the other
 * two words and the key; the key advances by two Weyl constants between
 * rounds. The constants are the published ones for this variant.
 * ---------------------------------------------------------------------- */
void oracle_philox4x32_10(const uint32_t ctr_in[4], const uint32_t key_in[2], uint32_t out[4])
{
    const uint64_t mul0 = 0xD2511F53u, mul1 = 0xCD9E8D57u;
    const uint32_t weyl0 = 0x9E3779B9u, weyl1 = 0xBB67AE85u;
    uint32_t c0 = ctr_in[0], c1 = ctr_in[1], c2 = ctr_in[2], c3 = ctr_in[3];
    uint32_t k0 = key_in[0], k1 = key_in[1];
    for (int round = 0; round < 10; ++round) {
        if (round > 0) {
            k0 += weyl0;
            k1 += weyl1;
        }
        uint64_t p0 = mul0 * (uint64_t)c0;
        uint64_t p1 = mul1 * (uint64_t)c2;
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

/*
 * The random word of source element i (row-major linear index in the logical
 * [rows, cols] tensor, independent of the stored layout and of ld).
 * READING of "keyed (seed, element index)": key = the 64-bit seed split in
 * two words, counter = (i/4 low word, i/4 high word, subseq, 0), word i mod 4.
 */
uint32_t oracle_sr_word(uint64_t seed, uint32_t subseq, uint64_t i)
{
    uint64_t j = i / 4;
    uint32_t ctr[4] = {(uint32_t)j, (uint32_t)(j >> 32), subseq, 0};
    uint32_t key[2] = {(uint32_t)seed, (uint32_t)(seed >> 32)};
    uint32_t out[4];
    oracle_philox4x32_10(ctr, key, out);
    return out[i % 4];
}

/* ------------------------------------------------------------------------
 * Inputs: binary32, or bfloat16 given as its 16 raw bits (widened exactly).
 * ---------------------------------------------------------------------- */
static float load_elem(const void *x, int dtype, int64_t ld, int64_t r, int64_t c)
{
    if (dtype == ORACLE_F32)
        return ((const float *)x)[r * ld + c];
    uint32_t bits = (uint32_t)((const uint16_t *)x)[r * ld + c] << 16;
    float f;
    memcpy(&f, &bits, 4);
    return f;
}

/*
 * Tensor amax ([UE5M3] §5.1: the operand's tensor maximum that is sampled
 * and held): the largest |x| over the tensor.
 */
float oracle_amax(const void *x, int dtype, int64_t rows, int64_t cols, int64_t ld)
{
    float m = 0.0f;
    for (int64_t r = 0; r < rows; ++r)
        for (int64_t c = 0; c < cols; ++c) {
            float a = fabsf(load_elem(x, dtype, ld, r, c));
            if (a > m)
                m = a;
        }
    return m;
}

/*
 * FP32 tensor (encode) scale. [UE5M3] §3 (NVFP4's FP32 tensor scale) and
 * §5.2 (NVIDIA's fixed 448 becomes a tunable target T: a block whose amax
 * equals the held tensor amax A gets block scale T). READING:
 * S = RN(RN(6 T) / A); S = 1 when A is zero or not finite; when the quotient
 * overflows, S is the largest finite binary32 value.
 */
float oracle_tensor_scale(float amax, float T)
{
    if (!(amax > 0.0f) || isinf(amax))
        return 1.0f;
    float six_t = 6.0f * T;
    float s = six_t / amax;
    if (isinf(s))
        s = 3.40282346638528859812e+38f;
    return s;
}

/*
 * Quantize one logical [rows, cols] tensor.
 *   layout ROW16  : blocks of 16 consecutive elements of a row.
 *                   codes [rows][cols/2], scales [rows][cols/16].
 *   layout COL16  : blocks of 16 consecutive elements of a column; stored as
 *                   ROW16 of the transpose: codes [cols][rows/2],
 *                   scales [cols][rows/16].
 *   layout TILE16 : 16 x 16 tiles; codes [rows][cols/2], scales
 *                   [rows/16][cols/16]; optionally also the transpose
 *                   (codes_t [cols][rows/2], scales_t [cols/16][rows/16]),
 *                   the same codes and scales transposed.
 * Packing: byte k of a stored row holds its elements 2k (bits 3:0) and
 * 2k+1 (bits 7:4).
 * Variants (block size 32, E4M3 scales: the page's block-32 run and NVFP4's
 * scale format, [UE5M3] §3 and §7.3) go through oracle_quantize_fmt: blocks
 * of `block` elements (a row or column segment, or block x block tiles) and
 * the scale format's encode/decode; shapes scale by `block` instead of 16.
 * Per block ([UE5M3] §3-§5; READING for the binary32 order of operations):
 *   bamax = max |x| over the block
 *   bamax == 0 : scale code 0, every payload code is the element's sign bit
 *   otherwise  : raw = RN(RN(bamax / 6) * S); code = UE5M3 nearest + repair;
 *                dec = decode(code); r = RN(S / dec); v = RN(x * r);
 *                payload = E2M1 RNE or SR of v.
 * SR words are indexed by the element's row-major position in the full
 * logical tensor: (idx_row0 + r) * idx_cols + idx_col0 + c, so a region of a
 * larger tensor can be quantized on its own (idx_row0 = idx_col0 = 0 and
 * idx_cols = cols for a whole tensor).
 * diag (optional): [0] blocks zero-rounded before repair, [1] saturated.
 * ROW16 needs cols % 16 == 0, COL16 rows % 16 == 0, TILE16 both.
 * Returns 0, or -1 on a shape error.
 */
static void put_code(uint8_t *codes, int64_t stride_bytes, int64_t row, int64_t col, int code)
{
    uint8_t *b = codes + row * stride_bytes + col / 2;
    if (col & 1)
        *b = (uint8_t)((*b & 0x0F) | (code << 4));
    else
        *b = (uint8_t)((*b & 0xF0) | code);
}

int oracle_quantize_fmt(const void *x, int dtype, int64_t rows, int64_t cols, int64_t ld,
                        float amax_held, float T, int layout, int block, int scale_fmt, int rnd,
                        uint64_t seed, uint32_t subseq, int64_t idx_row0, int64_t idx_col0,
                        int64_t idx_cols, uint8_t *codes, uint8_t *scales, float *enc_scale_out,
                        uint8_t *codes_t, uint8_t *scales_t, int32_t *diag)
{
    /* The blocked dimension(s) must hold whole blocks; the other may be
     * ragged (any length, including 0). */
    if (rows < 0 || cols < 0 || ld < cols || (block != 16 && block != 32))
        return -1;
    if (scale_fmt != ORACLE_UE5M3 && scale_fmt != ORACLE_E4M3)
        return -1;
    if ((layout != ORACLE_COL16 && cols % block) || (layout != ORACLE_ROW16 && rows % block))
        return -1;
    float S = oracle_tensor_scale(amax_held, T);
    if (enc_scale_out)
        *enc_scale_out = S;
    int32_t nzero = 0, nsat = 0;

    /* Block extent: br x bc elements starting at (r0, c0). */
    int64_t br = (layout == ORACLE_ROW16) ? 1 : block;
    int64_t bc = (layout == ORACLE_COL16) ? 1 : block;
    for (int64_t r0 = 0; r0 < rows; r0 += br) {
        for (int64_t c0 = 0; c0 < cols; c0 += bc) {
            float bamax = 0.0f;
            for (int64_t r = r0; r < r0 + br; ++r)
                for (int64_t c = c0; c < c0 + bc; ++c) {
                    float a = fabsf(load_elem(x, dtype, ld, r, c));
                    if (a > bamax)
                        bamax = a;
                }
            int scode = 0;
            float r_mul = 0.0f;
            if (bamax > 0.0f) {
                float d6 = bamax / 6.0f;
                float raw = d6 * S;
                int flags = 0;
                scode = scale_encode(scale_fmt, raw, &flags);
                nzero += flags & 1;
                nsat += (flags >> 1) & 1;
                float dec = (float)scale_decode(scale_fmt, scode);
                r_mul = S / dec;
            }
            for (int64_t r = r0; r < r0 + br; ++r)
                for (int64_t c = c0; c < c0 + bc; ++c) {
                    float xv = load_elem(x, dtype, ld, r, c);
                    int neg = signbit(xv) != 0;
                    int q;
                    if (bamax == 0.0f) {
                        q = neg ? 8 : 0;
                    } else {
                        float v = xv * r_mul;
                        if (rnd == ORACLE_SR)
                            q = oracle_e2m1_encode_sr(v, neg, oracle_sr_word(seed, subseq,
                                    (uint64_t)((idx_row0 + r) * idx_cols + idx_col0 + c)));
                        else
                            q = oracle_e2m1_encode_rne(v, neg);
                    }
                    if (layout == ORACLE_COL16) {
                        put_code(codes, rows / 2, c, r, q);
                    } else {
                        put_code(codes, cols / 2, r, c, q);
                        if (layout == ORACLE_TILE16 && codes_t)
                            put_code(codes_t, rows / 2, c, r, q);
                    }
                }
            if (layout == ORACLE_ROW16)
                scales[r0 * (cols / block) + c0 / block] = (uint8_t)scode;
            else if (layout == ORACLE_COL16)
                scales[c0 * (rows / block) + r0 / block] = (uint8_t)scode;
            else {
                scales[(r0 / block) * (cols / block) + c0 / block] = (uint8_t)scode;
                if (scales_t)
                    scales_t[(c0 / block) * (rows / block) + r0 / block] = (uint8_t)scode;
            }
        }
    }
    if (diag) {
        diag[0] = nzero;
        diag[1] = nsat;
    }
    return 0;
}

int oracle_quantize(const void *x, int dtype, int64_t rows, int64_t cols, int64_t ld,
                    float amax_held, float T, int layout, int rnd, uint64_t seed, uint32_t subseq,
                    int64_t idx_row0, int64_t idx_col0, int64_t idx_cols,
                    uint8_t *codes, uint8_t *scales, float *enc_scale_out,
                    uint8_t *codes_t, uint8_t *scales_t, int32_t *diag)
{
    return oracle_quantize_fmt(x, dtype, rows, cols, ld, amax_held, T, layout, 16, ORACLE_UE5M3,
                               rnd, seed, subseq, idx_row0, idx_col0, idx_cols, codes, scales,
                               enc_scale_out, codes_t, scales_t, diag);
}

/*
 * Decoded operand of a stored quantized tensor ([UE5M3] §6: the emulated
 * GEMM contracts decoded operands): out[r][c] = e2m1(code) * dec(scale),
 * exact in double (at most 6 significant bits). layout is ROW16 or TILE16
 * (a COL16 result is stored as ROW16 of the transpose).
 */
static double decoded(const uint8_t *codes, const uint8_t *scales, int64_t cols, int layout,
                      int block, int scale_fmt, int64_t r, int64_t c)
{
    uint8_t byte = codes[r * (cols / 2) + c / 2];
    int q = (c & 1) ? (byte >> 4) : (byte & 0x0F);
    int sc = (layout == ORACLE_TILE16) ? scales[(r / block) * (cols / block) + c / block]
                                       : scales[r * (cols / block) + c / block];
    return oracle_e2m1_decode(q) * scale_decode(scale_fmt, sc);
}

void oracle_decode_f64_fmt(const uint8_t *codes, const uint8_t *scales, int64_t rows, int64_t cols,
                           int layout, int block, int scale_fmt, double *out)
{
    for (int64_t r = 0; r < rows; ++r)
        for (int64_t c = 0; c < cols; ++c)
            out[r * cols + c] = decoded(codes, scales, cols, layout, block, scale_fmt, r, c);
}

void oracle_decode_f64(const uint8_t *codes, const uint8_t *scales, int64_t rows, int64_t cols,
                       int layout, double *out)
{
    oracle_decode_f64_fmt(codes, scales, rows, cols, layout, 16, ORACLE_UE5M3, out);
}

/*
 * Dequantize to binary32 ([UE5M3] §6): x_hat = RN((e2m1 * dec) / S), one
 * rounding of an exact product. (A bfloat16 output is this value rounded
 * once more, to bfloat16, by the caller.)
 */
void oracle_dequant_f32_fmt(const uint8_t *codes, const uint8_t *scales, int64_t rows, int64_t cols,
                            int layout, int block, int scale_fmt, float S, float *out)
{
    for (int64_t r = 0; r < rows; ++r)
        for (int64_t c = 0; c < cols; ++c)
            out[r * cols + c] =
                (float)decoded(codes, scales, cols, layout, block, scale_fmt, r, c) / S;
}

void oracle_dequant_f32(const uint8_t *codes, const uint8_t *scales, int64_t rows, int64_t cols,
                        int layout, float S, float *out)
{
    oracle_dequant_f32_fmt(codes, scales, rows, cols, layout, 16, ORACLE_UE5M3, S, out);
}

/*
 * Brute-force GEMM of decoded operands for small cases:
 * Y[i][j] = (sum_k A[i][k] B[j][k]) / (Sa Sb), all in double.
 */
void oracle_gemm_f64_loops(const double *a, const double *b, int64_t m, int64_t n, int64_t k,
                           double sa, double sb, double *y)
{
    for (int64_t i = 0; i < m; ++i)
        for (int64_t j = 0; j < n; ++j) {
            double acc = 0.0;
            for (int64_t t = 0; t < k; ++t)
                acc += a[i * k + t] * b[j * k + t];
            y[i * n + j] = acc / (sa * sb);
        }
}

/*
 * Probe-matched GEMM numerics ([UE5M3] §6 and Appendix B: the page's model
 * of native FP4 GEMM outputs). For each output element the contraction is
 * cut into consecutive slices of 64 along K; each slice's dot product of the
 * decoded operands is formed exactly and rounded once to binary32; the slice
 * partials are added in ascending slice order with binary32 additions
 * rounded toward zero; optionally the accumulator is snapped to the nearest
 * multiple of 2^-snap_log2 (ties to even: 1024 * c rounded, divided by 1024
 * for snap_log2 = 10); then it is multiplied by the tensor-scale product.
 * READING: the slice sum is rounded to nearest (once), the first partial
 * starts the sum, alpha = 1 / (Sa Sb) is formed in double and applied as one
 * binary32 multiply when it is a normal binary32 (else the product is formed
 * in double and rounded once), a shorter last slice when K % 64 != 0.
 *
 * Decoded operands (e2m1 * scale) are multiples of 2^-18 below 2^19, so
 * each is an integer n * 2^-18 with |n| < 2^37 and the slice sums are exact
 * in 128-bit integers (|sum| < 64 * 2^74).
 */
static float i128_scaled_rn(__int128 s, int e)
{
    if (s == 0) return 0.0f;
    const int neg = s < 0;
    const unsigned __int128 u = neg ? -(unsigned __int128)s : (unsigned __int128)s;
    int top = 0;
    for (unsigned __int128 t = u; t > 1; t >>= 1) ++top;
    uint64_t kept;
    int sh = 0;
    if (top <= 23) {
        kept = (uint64_t)u;
    } else {
        sh = top - 23;
        const unsigned __int128 one = 1;
        const unsigned __int128 rem = u & ((one << sh) - 1);
        const unsigned __int128 half = one << (sh - 1);
        kept = (uint64_t)(u >> sh);
        if (rem > half || (rem == half && (kept & 1u))) ++kept; /* ties to even */
    }
    const float f = ldexpf((float)kept, sh + e); /* kept <= 2^24: exact */
    return neg ? -f : f;
}

int oracle_gemm_probe(const double *a, const double *b, int64_t m, int64_t n, int64_t k,
                      float sa, float sb, int snap_log2, float *y)
{
    const double unit = 262144.0; /* 2^18 */
    const double alpha_d = 1.0 / ((double)sa * (double)sb);
    const float alpha = (float)alpha_d;
    const int alpha_normal = alpha >= FLT_MIN && alpha <= FLT_MAX;
    const int prev = fegetround();
    for (int64_t i = 0; i < m; ++i)
        for (int64_t j = 0; j < n; ++j) {
            float acc = 0.0f;
            for (int64_t g0 = 0; g0 < k; g0 += 64) {
                const int64_t g1 = g0 + 64 < k ? g0 + 64 : k;
                __int128 sum = 0;
                for (int64_t t = g0; t < g1; ++t) {
                    const double va = a[i * k + t] * unit, vb = b[j * k + t] * unit;
                    const int64_t na = (int64_t)va, nb = (int64_t)vb;
                    if ((double)na != va || (double)nb != vb) return 1; /* not on the lattice */
                    sum += (__int128)na * (__int128)nb;
                }
                const float p = i128_scaled_rn(sum, -36);
                fesetround(FE_TOWARDZERO);
                volatile float t = acc + p;
                acc = t;
                fesetround(FE_TONEAREST);
            }
            if (snap_log2 > 0) acc = ldexpf(nearbyintf(ldexpf(acc, snap_log2)), -snap_log2);
            y[i * n + j] = alpha_normal ? acc * alpha : (float)((double)acc * alpha_d);
        }
    fesetround(prev);
    return 0;
}
