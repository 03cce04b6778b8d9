// C ABI of libfp4q.so: argument validation (before anything is enqueued),
// status mapping, and dispatch to the HIP kernels. No C++ exception crosses
// this boundary and nothing here allocates.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>

#include "../../include/fp4q.h"
#include "kernels.h"

namespace {

constexpr int64_t kMaxGridX = 0x7FFFFFFF / 256;  // workgroups of 256 threads

int elem_size(int dt) { return dt == FP4Q_F32 ? 4 : (dt == FP4Q_BF16 ? 2 : 0); }

// Sizes beyond any device memory are rejected up front, so the launch
// arithmetic below (products of two sizes, grid counts) cannot overflow:
// each dimension at most 2^40, and at most 2^44 elements.
constexpr int64_t kMaxDim = int64_t(1) << 40;
constexpr int64_t kMaxElems = int64_t(1) << 44;
bool dims_ok(int64_t a, int64_t b) {
  if (a < 0 || b < 0 || a > kMaxDim || b > kMaxDim) return false;
  return a == 0 || b <= kMaxElems / a;
}

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

fp4q_status from_hip(hipError_t e) { return e == hipSuccess ? FP4Q_OK : FP4Q_E_HIP; }

fp4q_status check_operand(const fp4q_qtensor* q) {
  if (!q) return FP4Q_E_NULL;
  if (!dims_ok(q->rows, q->cols)) return FP4Q_E_SHAPE;
  if (q->layout != FP4Q_ROW16 && q->layout != FP4Q_TILE16x16) return FP4Q_E_ARG;
  if (q->block != 16 && q->block != 32) return FP4Q_E_ARG;
  if (q->scale_fmt != FP4Q_UE5M3 && q->scale_fmt != FP4Q_E4M3) return FP4Q_E_ARG;
  if (q->pack != FP4Q_PACK_ROWS && q->pack != FP4Q_PACK_K64) return FP4Q_E_ARG;
  if (q->cols % q->block) return FP4Q_E_SHAPE;
  if (q->pack == FP4Q_PACK_K64 && q->cols % 64) return FP4Q_E_SHAPE;
  if (q->layout == FP4Q_TILE16x16 && q->rows % q->block) return FP4Q_E_SHAPE;
  if (!q->enc_scale) return FP4Q_E_NULL;
  if (q->rows > 0 && q->cols > 0 && (!q->codes || !q->scales)) return FP4Q_E_NULL;
  if (!aligned(q->codes, 8) || !aligned(q->scales, 4)) return FP4Q_E_ALIGN;
  return FP4Q_OK;
}

fp4q::QOperand to_operand(const fp4q_qtensor* q) {
  fp4q::QOperand o;
  o.codes = q->codes;
  o.scales = q->scales;
  o.enc_scale = q->enc_scale;
  o.rows = q->rows;
  o.cols = q->cols;
  o.tile = q->layout == FP4Q_TILE16x16 ? 1 : 0;
  o.block = q->block;
  o.scale_fmt = q->scale_fmt;
  o.pack = q->pack;
  return o;
}

fp4q_status gemm(const fp4q_qtensor* a, const fp4q_qtensor* b, void* y, fp4q_dtype yt,
                 void* stream, bool probe = false, int snap_log2 = 0) {
  fp4q_status st = check_operand(a);
  if (st != FP4Q_OK) return st;
  st = check_operand(b);
  if (st != FP4Q_OK) return st;
  const int es = elem_size(yt);
  if (!es) return FP4Q_E_DTYPE;
  if (a->cols != b->cols) return FP4Q_E_SHAPE;
  if (a->pack != b->pack) return FP4Q_E_ARG;
  if (a->rows > 0 && b->rows > 0 && !y) return FP4Q_E_NULL;
  if (y && !aligned(y, es)) return FP4Q_E_ALIGN;  // element stores and fp32 atomic adds
  const int64_t tm = (a->rows + 127) / 128, tn = (b->rows + 127) / 128;
  if (tm > 0 && tn > (0x7FFFFFFF / 512) / tm) return FP4Q_E_SHAPE;
  if (probe)
    return from_hip(fp4q::launch_gemm_probe(to_operand(a), to_operand(b), y, es, snap_log2,
                                            static_cast<hipStream_t>(stream)));
  return from_hip(fp4q::launch_gemm(to_operand(a), to_operand(b), y, es,
                                    static_cast<hipStream_t>(stream)));
}

}  // namespace

extern "C" {

int fp4q_abi_version(void) { return FP4Q_ABI_VERSION; }

const char* fp4q_status_str(fp4q_status s) {
  switch (s) {
    case FP4Q_OK: return "ok";
    case FP4Q_E_NULL: return "a required pointer is NULL";
    case FP4Q_E_SHAPE: return "invalid shape";
    case FP4Q_E_ALIGN: return "misaligned pointer or row stride";
    case FP4Q_E_DTYPE: return "unknown dtype";
    case FP4Q_E_ARG: return "invalid argument";
    case FP4Q_E_HIP: return "HIP launch error";
  }
  return "unknown status";
}

fp4q_status fp4q_amax(const void* x, fp4q_dtype xt, int64_t rows, int64_t cols, int64_t ld,
                      float* amax_out, void* stream) {
  const int es = elem_size(xt);
  if (!es) return FP4Q_E_DTYPE;
  if (!amax_out) return FP4Q_E_NULL;
  if (!dims_ok(rows, cols) || !dims_ok(rows, ld) || ld < cols) return FP4Q_E_SHAPE;
  if (rows > 0 && cols > 0) {
    if (!x) return FP4Q_E_NULL;
    if (!aligned(x, 16) || (cols * es) % 16 || (ld * es) % 16) return FP4Q_E_ALIGN;
  }
  if (!aligned(amax_out, 4)) return FP4Q_E_ALIGN;
  return from_hip(fp4q::launch_amax(x, es, rows, cols, ld, amax_out,
                                    static_cast<hipStream_t>(stream)));
}

fp4q_status fp4q_quantize_fmt(const void* x, fp4q_dtype xt, int64_t rows, int64_t cols,
                              int64_t ld, const float* amax_held, float target, fp4q_layout layout,
                              int32_t block, fp4q_scale_fmt scale_fmt, int32_t pack,
                              fp4q_round rnd, uint64_t seed, uint32_t subseq, uint8_t* codes,
                              uint8_t* scales,
                              float* enc_scale_out, uint8_t* codes_t, uint8_t* scales_t,
                              int32_t* diag, void* stream) {
  const int es = elem_size(xt);
  if (!es) return FP4Q_E_DTYPE;
  if (layout != FP4Q_ROW16 && layout != FP4Q_COL16 && layout != FP4Q_TILE16x16) return FP4Q_E_ARG;
  if (block != 16 && block != 32) return FP4Q_E_ARG;
  if (scale_fmt != FP4Q_UE5M3 && scale_fmt != FP4Q_E4M3) return FP4Q_E_ARG;
  if (pack != FP4Q_PACK_ROWS && pack != FP4Q_PACK_K64) return FP4Q_E_ARG;
  if (rnd != FP4Q_RNE && rnd != FP4Q_SR) return FP4Q_E_ARG;
  if (!(target > 0.0f) || !std::isfinite(target)) return FP4Q_E_ARG;
  if ((codes_t == nullptr) != (scales_t == nullptr)) return FP4Q_E_ARG;
  if (codes_t && layout == FP4Q_COL16) return FP4Q_E_ARG;
  // ROW with the second orientation also needs whole column blocks
  if (codes_t && layout == FP4Q_ROW16 && rows % block) return FP4Q_E_SHAPE;
  if (!amax_held) return FP4Q_E_NULL;
  if (!aligned(amax_held, 4)) return FP4Q_E_ALIGN;
  if (!dims_ok(rows, cols) || !dims_ok(rows, ld) || ld < cols) return FP4Q_E_SHAPE;
  if (layout != FP4Q_COL16 && cols % block) return FP4Q_E_SHAPE;
  if (layout != FP4Q_ROW16 && rows % block) return FP4Q_E_SHAPE;
  if (layout == FP4Q_COL16 && cols % 8) return FP4Q_E_ALIGN;
  if (pack == FP4Q_PACK_K64) {
    // every output's contraction length: cols for ROW16 and TILE, rows for
    // COL16 and for the second (transposed) outputs
    if (layout != FP4Q_COL16 && cols % 64) return FP4Q_E_SHAPE;
    if ((layout == FP4Q_COL16 || codes_t) && rows % 64) return FP4Q_E_SHAPE;
  }
  const bool nonempty = rows > 0 && cols > 0;
  if (nonempty) {
    if (!x || !codes || !scales) return FP4Q_E_NULL;
    if (!aligned(x, 16) || (ld * es) % 16) return FP4Q_E_ALIGN;
    if (!aligned(codes, 8) || (codes_t && !aligned(codes_t, 8))) return FP4Q_E_ALIGN;
    // workgroup counts (upper bounds) and sizes of the kernels, as the
    // launchers set them up: a launch stays below 2^31 threads
    int64_t groups, threads;
    if (layout == FP4Q_ROW16 && !codes_t) {
      groups = rows * ((cols / block + 63) / 64);
      threads = 64;
    } else if (layout == FP4Q_TILE16x16) {
      groups = ((cols / 8 + 255) / 256) * (rows / 16);
      threads = 256;
    } else {
      const int64_t tc = 1024 / block, tr = 4 * block;
      groups = ((cols + tc - 1) / tc) * ((rows + tr - 1) / tr);
      threads = 4 * tc;
    }
    if (groups > 0x7FFFFFFF / threads) return FP4Q_E_SHAPE;
  }
  if ((enc_scale_out && !aligned(enc_scale_out, 4)) || (diag && !aligned(diag, 4)))
    return FP4Q_E_ALIGN;
  fp4q::QuantArgs a;
  a.x = x;
  a.es = es;
  a.rows = rows;
  a.cols = cols;
  a.ld = ld;
  a.amax_held = amax_held;
  a.target = target;
  a.layout = (int)layout;
  a.block = block;
  a.scale_fmt = (int)scale_fmt;
  a.pack = pack;
  a.sr = rnd == FP4Q_SR ? 1 : 0;
  a.seed = seed;
  a.subseq = subseq;
  a.codes = codes;
  a.scales = scales;
  a.enc_scale_out = enc_scale_out;
  a.codes_t = codes_t;
  a.scales_t = scales_t;
  a.diag = diag;
  return from_hip(fp4q::launch_quantize(a, static_cast<hipStream_t>(stream)));
}

fp4q_status fp4q_quantize(const void* x, fp4q_dtype xt, int64_t rows, int64_t cols, int64_t ld,
                          const float* amax_held, float target, fp4q_layout layout,
                          fp4q_round rnd, uint64_t seed, uint32_t subseq, uint8_t* codes,
                          uint8_t* scales, float* enc_scale_out, uint8_t* codes_t,
                          uint8_t* scales_t, int32_t* diag, void* stream) {
  return fp4q_quantize_fmt(x, xt, rows, cols, ld, amax_held, target, layout, 16, FP4Q_UE5M3,
                           FP4Q_PACK_ROWS, rnd, seed, subseq, codes, scales, enc_scale_out, codes_t,
                           scales_t, diag, stream);
}

fp4q_status fp4q_dequant(const fp4q_qtensor* q, void* out, fp4q_dtype ot, void* stream) {
  fp4q_status st = check_operand(q);
  if (st != FP4Q_OK) return st;
  const int es = elem_size(ot);
  if (!es) return FP4Q_E_DTYPE;
  if (q->rows > 0 && q->cols > 0) {
    if (!out) return FP4Q_E_NULL;
    if (!aligned(out, 16)) return FP4Q_E_ALIGN;
    if ((q->rows * (q->cols / 8) + 255) / 256 > kMaxGridX) return FP4Q_E_SHAPE;
  }
  return from_hip(fp4q::launch_dequant(to_operand(q), out, es, static_cast<hipStream_t>(stream)));
}

fp4q_status fp4q_linear_fwd(const fp4q_qtensor* xq, const fp4q_qtensor* wq, void* y,
                            fp4q_dtype yt, void* stream) {
  return gemm(xq, wq, y, yt, stream);
}

fp4q_status fp4q_linear_dgrad(const fp4q_qtensor* dyq, const fp4q_qtensor* wqt, void* dx,
                              fp4q_dtype dxt, void* stream) {
  return gemm(dyq, wqt, dx, dxt, stream);
}

fp4q_status fp4q_linear_wgrad(const fp4q_qtensor* dyqt, const fp4q_qtensor* xqt, void* dw,
                              fp4q_dtype dwt, void* stream) {
  return gemm(dyqt, xqt, dw, dwt, stream);
}

fp4q_status fp4q_linear_probe(const fp4q_qtensor* a, const fp4q_qtensor* b, void* y,
                              fp4q_dtype yt, int32_t snap_log2, void* stream) {
  if (snap_log2 < 0 || snap_log2 > 30) return FP4Q_E_ARG;
  return gemm(a, b, y, yt, stream, true, snap_log2);
}

}  // extern "C"
