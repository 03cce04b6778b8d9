/*
 * fp4q: block-scaled FP4 (E2M1 payload, UE5M3 block scale, FP32 tensor
 * scale) quantization and the emulated FP4 linear layer, as described in
 * "UE5M3 FP4 Block Scaling for Stable Language Model Pretraining", for AMD
 * Instinct MI355X (gfx950). C ABI of libfp4q.so.
 *
 * Conventions for every entry point:
 *  - Data pointers are DEVICE pointers (HIP memory of the current device)
 *    unless stated otherwise; fp4q_qtensor structs themselves are read on the
 *    host during the call. The caller allocates and owns every buffer; the
 *    library allocates nothing and keeps no state.
 *  - `stream` is a hipStream_t (NULL = the default stream). Work is enqueued
 *    on it and the call returns without synchronizing. Inputs must stay valid
 *    and outputs untouched until the stream has passed the work.
 *  - Arguments are validated before anything is enqueued; on any error
 *    nothing is enqueued and a status code is returned. FP4Q_E_HIP means a
 *    launch was rejected by the runtime; faults inside kernels surface at the
 *    caller's next synchronization, as for any HIP work.
 *  - Inputs must be finite (the held amax may be anything: see below).
 *  - Matrices are row-major. A quantized operand stores two 4-bit codes per
 *    byte: element 2k of a row in bits 3:0 of byte k, element 2k+1 in bits
 *    7:4. A code is sign (bit 3) | E2M1 magnitude (bits 2:0), magnitudes
 *    {0, 0.5, 1, 1.5, 2, 3, 4, 6}. A scale byte is a UE5M3 code: exponent
 *    bits 7:3 (bias 15), fraction bits 2:0; 0x01 = 2^-17 .. 0xF7 = 61440.
 */
#ifndef FP4Q_H
#define FP4Q_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define FP4Q_ABI_VERSION 3

typedef enum {
    FP4Q_OK = 0,
    FP4Q_E_NULL = 1,   /* a required pointer is NULL */
    FP4Q_E_SHAPE = 2,  /* negative size, block dimension not a multiple of 16,
                          ld < cols, mismatched GEMM shapes, or a grid too large */
    FP4Q_E_ALIGN = 3,  /* a pointer or row stride breaks the alignment rules */
    FP4Q_E_DTYPE = 4,  /* unknown dtype */
    FP4Q_E_ARG = 5,    /* unknown layout / rounding, bad target, bad buffer combination */
    FP4Q_E_HIP = 6     /* the HIP runtime rejected a launch */
} fp4q_status;

typedef enum { FP4Q_F32 = 0, FP4Q_BF16 = 1 } fp4q_dtype;

/* Payload rounding: round to nearest, ties to the even code (activations and
 * weights, §2 and §5 of the page), or stochastic rounding with one
 * Philox4x32-10 word per element (upstream gradients, §5.2). */
typedef enum { FP4Q_RNE = 0, FP4Q_SR = 1 } fp4q_round;

/* Block geometry (§3 and §5 of the page: 1D blocks of 16 along the
 * contraction axis for activations and gradients, 2D 16x16 for weights).
 * The names give the default block of 16; with a block size B of 32 (the
 * page's block-32 run, §7.3) every 16 below reads B. */
typedef enum {
    FP4Q_ROW16 = 0,     /* blocks of 16 along a row; codes [R][C/2], scales [R][C/16] */
    FP4Q_COL16 = 1,     /* blocks of 16 down a column, stored as ROW16 of the
                           transpose: codes [C][R/2], scales [C][R/16] */
    FP4Q_TILE16x16 = 2  /* 16x16 tiles; codes [R][C/2], scales [R/16][C/16] */
} fp4q_layout;

/* Block-scale format: UE5M3 (the page's, §4.1) or E4M3 (NVFP4's, §3; codes
 * 0x00..0x7E: 2^-9 .. 448, the same code's UE5M3 value times 256). */
typedef enum { FP4Q_UE5M3 = 0, FP4Q_E4M3 = 1 } fp4q_scale_fmt;

/* Memory packing of an operand's codes and scales. The pages fix what a
 * code and a scale are, not where they live. Within a row this library
 * stores two E2M1 codes per byte (element 2j in bits 3:0 and 2j+1 in bits
 * 7:4 of byte j) and one scale byte per block, in either packing:
 *  FP4Q_PACK_ROWS: row-major, as the shapes in fp4q_layout give them.
 *  FP4Q_PACK_K64: the contraction axis cut into tiles of 64 elements; tile t
 *    holds every row's 32 code bytes back to back, then the next tile:
 *    byte j of row r at (j / 32) * (R * 32) + r * 32 + j % 32 for an operand
 *    of R rows. Scales likewise with 64 / B bytes per row and tile: scale j
 *    of scale row s at (j / n) * (SR * n) + s * n + j % n, n = 64 / B, SR the
 *    number of scale rows. The buffer sizes equal the row-major ones. A
 *    GEMM workgroup then reads its rows' slice of one k tile as one
 *    contiguous run, and the COL16 output of a quantize is written in
 *    contiguous runs too. Needs the contraction length (cols of the
 *    operand) to be a multiple of 64. */
typedef enum { FP4Q_PACK_ROWS = 0, FP4Q_PACK_K64 = 1 } fp4q_pack;

/* One quantized operand as the GEMMs read it: `rows` x `cols` logical
 * elements, contiguous along `cols` (the contraction). layout is FP4Q_ROW16
 * (scales [rows][cols/B]; also what FP4Q_COL16 produces for the transpose)
 * or FP4Q_TILE16x16 (scales [rows/B][cols/B]), B = block (16 or 32);
 * scale_fmt an fp4q_scale_fmt. enc_scale points to the device fp32 tensor
 * scale S written by fp4q_quantize. codes must be 8-byte aligned and scales
 * 4-byte aligned. pack is an fp4q_pack; the two operands of a GEMM must share
 * it, and FP4Q_PACK_K64 needs cols % 64 == 0. */
typedef struct {
    const uint8_t *codes;
    const uint8_t *scales;
    const float *enc_scale;
    int64_t rows;
    int64_t cols;
    int32_t layout;
    int32_t block;
    int32_t scale_fmt;
    int32_t pack;
} fp4q_qtensor;

int fp4q_abi_version(void);
const char *fp4q_status_str(fp4q_status s);

/*
 * Tensor amax (§5.1 of the page: each operand's tensor maximum is sampled
 * and held). amax_out (device, one fp32) receives max |x| over the [rows,
 * cols] tensor x of dtype xt with row stride ld elements; 0 for an empty
 * tensor. Exact and order-independent (a maximum of sign-cleared bit
 * patterns). x must be 16-byte aligned and cols * sizeof(elem) and
 * ld * sizeof(elem) multiples of 16.
 */
fp4q_status fp4q_amax(const void *x, fp4q_dtype xt, int64_t rows, int64_t cols, int64_t ld,
                      float *amax_out, void *stream);

/*
 * Quantize x ([rows, cols], dtype xt, row stride ld) to E2M1 codes with UE5M3
 * block scales (§3-§5 of the page).
 *  amax_held (device, one fp32, 4-byte aligned): the held tensor amax A.
 *    The tensor scale is S = RN(RN(6 * target) / A), S = 1 if A is 0 or not
 *    finite, and the largest finite fp32 if the quotient overflows; target
 *    is the UE5M3 target T of §5.2 (448 default; finite and > 0). S is
 *    written to *enc_scale_out (device, optional).
 *  Per block: bamax = max |x|; if 0, scale code 0 and sign-only codes. Else
 *    raw = RN(RN(bamax / 6) * S), scale = nearest UE5M3 (ties to even), with
 *    repair: a scale rounding to 0 becomes 0x01, one rounding above 61440
 *    becomes 0xF7 (§5.3); r = RN(S / dec); payload of x is E2M1 of RN(x * r),
 *    saturating at 6, by RNE or SR (rnd). SR rounds |v| up to the next
 *    magnitude iff w < ceil(p * 2^32), p its position between the two
 *    neighbours and w = word (i mod 4) of Philox4x32-10 with key = seed and
 *    counter (i/4 low, i/4 high, subseq, 0), i the row-major index of the
 *    element in the logical [rows, cols] tensor (so ROW16 and COL16 of one
 *    tensor draw the same word per element).
 *  layout: FP4Q_ROW16 needs cols % 16 == 0; FP4Q_COL16 rows % 16 == 0 and
 *    cols % 8 == 0; FP4Q_TILE16x16 rows % 16 == 0 and cols % 16 == 0.
 *  codes / scales: outputs in the layout's shape (see fp4q_layout).
 *  codes_t / scales_t: both or neither; not with FP4Q_COL16.
 *    FP4Q_TILE16x16: the transposed copy (codes [cols][rows/2], scales
 *      [cols/16][rows/16]) that dgrad reads.
 *    FP4Q_ROW16: the COL16 quantization of the same tensor (codes
 *      [cols][rows/2], scales [cols][rows/16]; needs rows % 16 == 0),
 *      produced in the same pass: one read of x and, for SR, one Philox word
 *      per element serving both orientations (fwd/dgrad and wgrad operands).
 *  diag (device, optional, two int32): receives the number of blocks whose
 *    scale was zero-rounded and saturated before repair.
 *  Alignment: x 16-byte aligned, ld * sizeof(elem) a multiple of 16; codes
 *    (and codes_t) 8-byte aligned.
 */
fp4q_status fp4q_quantize(const void *x, fp4q_dtype xt, int64_t rows, int64_t cols, int64_t ld,
                          const float *amax_held, float target, fp4q_layout layout,
                          fp4q_round rnd, uint64_t seed, uint32_t subseq, uint8_t *codes,
                          uint8_t *scales, float *enc_scale_out, uint8_t *codes_t,
                          uint8_t *scales_t, int32_t *diag, void *stream);

/*
 * fp4q_quantize with a block size (16 or 32) and a scale format
 * (fp4q_scale_fmt): the page's block-32 variant and NVFP4's E4M3 scales
 * (§3, §7.3). Every rule above carries over with B = block in place of 16
 * (shapes, divisibility, the TILE transposed copy with B x B tiles, the ROW
 * plus COL single pass); for E4M3 the nearest-code encode saturates once raw
 * exceeds 464 (to 0x7E = 448) and a zero-rounded scale repairs to 0x01
 * (2^-9). pack (an fp4q_pack) applies to every output (codes, scales and
 * the codes_t / scales_t pair); FP4Q_PACK_K64 needs the contraction length
 * of each output to be a multiple of 64: cols for FP4Q_ROW16 and
 * FP4Q_TILE16x16, rows for FP4Q_COL16 and for the codes_t outputs.
 * fp4q_quantize is this call with block 16, FP4Q_UE5M3 and FP4Q_PACK_ROWS.
 */
fp4q_status fp4q_quantize_fmt(const void *x, fp4q_dtype xt, int64_t rows, int64_t cols,
                              int64_t ld, const float *amax_held, float target,
                              fp4q_layout layout, int32_t block, fp4q_scale_fmt scale_fmt,
                              int32_t pack, fp4q_round rnd, uint64_t seed, uint32_t subseq,
                              uint8_t *codes, uint8_t *scales, float *enc_scale_out,
                              uint8_t *codes_t, uint8_t *scales_t, int32_t *diag,
                              void *stream);

/*
 * Dequantize q into out ([q->rows, q->cols], row-major, dtype ot):
 * x_hat = RN_fp32((e2m1 * dec) / S), then RNE to bf16 for FP4Q_BF16 (§6 of
 * the page: the emulation decodes operands exactly; S is removed after).
 * q->cols % q->block == 0 (% 64 for FP4Q_PACK_K64); out 16-byte aligned.
 */
fp4q_status fp4q_dequant(const fp4q_qtensor *q, void *out, fp4q_dtype ot, void *stream);

/*
 * The emulated FP4 linear layer (§6 of the page): the contraction of the
 * decoded operands (exact in binary16 after a power-of-two scaling, which
 * alpha undoes) in f16 MFMA with fp32 accumulation, times
 * alpha = 1 / (Sa Sb) (computed in double), rounded once to fp32 and then,
 * for a bf16 output, once more (RNE). Outputs are row-major and contiguous.
 *  fwd:   y[M, N]  = Xq[M, K] . Wq[N, K]^T      xq: X ROW16; wq: W TILE16x16
 *  dgrad: dx[M, K] = dYq[M, N] . Wq[N, K]       dyq: dY ROW16 [M, N];
 *                                               wqt: the transposed W copy [K, N]
 *  wgrad: dw[N, K] = dYq^T[N, M] . Xq[M, K]     dyqt: dY COL16 ([N, M] stored);
 *                                               xqt:  X COL16 ([K, M] stored)
 * In each, both operands must have equal `cols` (the contraction length,
 * a multiple of 16 and of each operand's block size) and `rows` a multiple of
 * the block size when their layout is TILE. The two operands may use
 * different block sizes and scale formats; they must share the packing
 * (FP4Q_E_ARG otherwise). The output (device) is aligned to its element
 * size (FP4Q_E_ALIGN otherwise).
 */
fp4q_status fp4q_linear_fwd(const fp4q_qtensor *xq, const fp4q_qtensor *wq, void *y,
                            fp4q_dtype yt, void *stream);
fp4q_status fp4q_linear_dgrad(const fp4q_qtensor *dyq, const fp4q_qtensor *wqt, void *dx,
                              fp4q_dtype dxt, void *stream);
fp4q_status fp4q_linear_wgrad(const fp4q_qtensor *dyqt, const fp4q_qtensor *xqt, void *dw,
                              fp4q_dtype dwt, void *stream);

/*
 * The probe-matched GEMM numerics of the UE5M3 page (§6 and Appendix B: its
 * model of native FP4 GEMM outputs), as an alternative accumulation for any
 * of the three products above: y[M, N] = A[M, K] . B[N, K]^T with a = A
 * (fwd: X ROW16, dgrad: dY ROW16, wgrad: dY COL16) and b = B (W TILE16x16,
 * W's transposed copy, X COL16), contiguous along K as for the other calls.
 * For each output the contraction is cut into consecutive 64-wide slices of
 * K; each slice's dot product of the decoded operands is formed with fp32
 * MFMA accumulation, the slice sums are added in slice order with fp32
 * additions rounded toward zero; if snap_log2 > 0 the sum is rounded to the
 * nearest multiple of
 * 2^-snap_log2 (ties to even; 10 gives the page's 1/1024 grid); then
 * y = RN_out(RN(sum * alpha)), alpha = 1 / (Sa Sb) as in the calls above.
 * Exactness: the matrix core aligns each MFMA's products and accumulator to
 * the largest and keeps 24 bits below its leading bit (lower bits are
 * dropped, not rounded). So y equals the page's model (each slice sum
 * formed exactly and rounded once to binary32) bit for bit for every output
 * whose slices all meet this condition: the slice's products are integer
 * multiples of a common 2^g and their absolute sum is below 2^(g+24). That
 * holds for nearly every output of quantized activations, weights and
 * gradients (scales within a slice spanning a few binades); where a slice's
 * products span more than the 24-bit window, the slice sum may differ from
 * the exactly rounded one by a few units in its last place.
 * snap_log2 in [0, 30]; yt FP4Q_F32 or FP4Q_BF16; y aligned to its element
 * size.
 */
fp4q_status fp4q_linear_probe(const fp4q_qtensor *a, const fp4q_qtensor *b, void *y,
                              fp4q_dtype yt, int32_t snap_log2, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* FP4Q_H */
