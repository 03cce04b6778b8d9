// Host-side launch functions of the HIP kernels (internal to libfp4q.so).
// Arguments are validated by the C ABI layer before any of these is called.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fp4q {

// max |x| over a [rows, cols] bf16 (es = 2) or fp32 (es = 4) tensor with row
// stride ld (elements); writes the fp32 result to *out (zeroed first).
hipError_t launch_amax(const void* x, int es, int64_t rows, int64_t cols, int64_t ld,
                       float* out, hipStream_t s);

struct QuantArgs {
  const void* x;
  int es;  // 2: bf16, 4: fp32
  int64_t rows, cols, ld;
  const float* amax_held;
  float target;
  int layout;  // 0 ROW16, 1 COL16, 2 TILE16x16 (blocks along a row, down a column, square)
  int block;   // 16 or 32
  int scale_fmt;  // 0 UE5M3, 1 E4M3
  int pack;       // 0 row-major, 1 K64 (tiles of 64 along the contraction)
  int sr;      // 0 RNE, 1 SR
  uint64_t seed;
  uint32_t subseq;
  uint8_t* codes;
  uint8_t* scales;
  float* enc_scale_out;
  uint8_t* codes_t;
  uint8_t* scales_t;
  int32_t* diag;
};
hipError_t launch_quantize(const QuantArgs& a, hipStream_t s);

struct QOperand {
  const uint8_t* codes;
  const uint8_t* scales;
  const float* enc_scale;
  int64_t rows, cols;
  int tile;  // 0: ROW16 scales [rows][cols/block]; 1: TILE16x16 scales [rows/block][cols/block]
  int block;      // 16 or 32
  int scale_fmt;  // 0 UE5M3, 1 E4M3 (value = UE5M3 value * 256)
  int pack;       // 0 row-major, 1 K64 (tiles of 64 along the contraction)
};

hipError_t launch_dequant(const QOperand& q, void* out, int out_es, hipStream_t s);

// Y[M, N] = A[M, K] * B[N, K]^T over decoded operands, times 1 / (Sa Sb).
hipError_t launch_gemm(const QOperand& a, const QOperand& b, void* y, int y_es, hipStream_t s);

// The same contraction with the probe-matched accumulation (64-wide slices,
// round-toward-zero addition of the slice sums, optional snap to multiples of
// 2^-snap_log2 when snap_log2 > 0).
hipError_t launch_gemm_probe(const QOperand& a, const QOperand& b, void* y, int y_es, int snap_log2,
                             hipStream_t s);

}  // namespace fp4q
