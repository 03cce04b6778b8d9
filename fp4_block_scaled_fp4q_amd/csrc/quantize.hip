// Block-scaled FP4 quantization ("UE5M3 FP4 Block Scaling for Stable
// Language Model Pretraining", §3-§5): E2M1 payloads with one UE5M3 scale per
// block under the FP32 tensor scale derived from a held amax and target T;
// RNE payloads for activations and weights, stochastic rounding with Philox
// words for upstream gradients.
//
// Layouts (codes: two elements per byte, even element in the low nibble):
//   ROW16   blocks of 16 along a row           codes [R][C/2], scales [R][C/16]
//   COL16   blocks of 16 down a column,        codes [C][R/2], scales [C][R/16]
//           stored as ROW16 of the transpose (the wgrad operands, quantized
//           along the token axis)
//   TILE16  16 x 16 tiles (weights)            codes [R][C/2], scales [R/16][C/16]
//           plus an optional transposed copy   codes [C][R/2], scales [C/16][R/16]
// ROW16 may also emit the COL16 outputs of the same tensor in the same pass
// (one read of the input, one Philox word per element for both).
//
// Variants: blocks of 32 instead of 16 (the page's block-32 run, §7.3; the
// shapes above with 32 in place of 16, and 32 x 32 weight tiles) and E4M3
// block scales instead of UE5M3 (NVFP4's scale format, §3), selected per
// call.
//
// The RNE kernels are HBM-bound: every input byte is read once with 128-bit
// loads and the per-element work is a widening, one multiply and half a
// hardware FP4 conversion. SR adds a Philox4x32-10 evaluation per four
// elements and is ALU-bound.
#include "codec.h"
#include "kernels.h"

namespace fp4q {
namespace {

constexpr int kThreads = 256;

__device__ __forceinline__ uint32_t pkmax16(uint32_t a, uint32_t b) {
  typedef unsigned short us2 __attribute__((ext_vector_type(2)));
  return __builtin_bit_cast(uint32_t, __builtin_elementwise_max(__builtin_bit_cast(us2, a),
                                                                __builtin_bit_cast(us2, b)));
}

// Eight consecutive elements of one row: bf16 kept packed (4 words), fp32 as
// 8 words. get(j) widens element j exactly to fp32.
template <bool kBF16>
struct Oct;

template <>
struct Oct<true> {
  uint32_t d[4];
  __device__ __forceinline__ void load(const uint8_t* p) {
    const uint4 v = load16(p);
    d[0] = v.x; d[1] = v.y; d[2] = v.z; d[3] = v.w;
  }
  __device__ __forceinline__ void zero() { d[0] = d[1] = d[2] = d[3] = 0u; }
  __device__ __forceinline__ float get(int j) const { return (j & 1) ? bf16_hi(d[j >> 1]) : bf16_lo(d[j >> 1]); }
  // max |x| of the 8 elements as a sign-cleared fp32 bit pattern
  __device__ __forceinline__ uint32_t absmax() const {
    const uint32_t m = pkmax16(pkmax16(d[0] & 0x7FFF7FFFu, d[1] & 0x7FFF7FFFu),
                               pkmax16(d[2] & 0x7FFF7FFFu, d[3] & 0x7FFF7FFFu));
    return max(m & 0xFFFFu, m >> 16) << 16;
  }
};

template <>
struct Oct<false> {
  uint32_t d[8];
  __device__ __forceinline__ void load(const uint8_t* p) {
    const uint4 a = load16(p);
    const uint4 b = load16(p + 16);
    d[0] = a.x; d[1] = a.y; d[2] = a.z; d[3] = a.w;
    d[4] = b.x; d[5] = b.y; d[6] = b.z; d[7] = b.w;
  }
  __device__ __forceinline__ void zero() {
#pragma clang loop unroll(full)
    for (int j = 0; j < 8; ++j) d[j] = 0u;
  }
  __device__ __forceinline__ float get(int j) const { return u2f(d[j]); }
  __device__ __forceinline__ uint32_t absmax() const {
    uint32_t m = 0u;
#pragma clang loop unroll(full)
    for (int j = 0; j < 8; ++j) m = max(m, d[j] & 0x7FFFFFFFu);
    return m;
  }
};

// Stochastic-rounding operands of source elements idx0 .. idx0+7 (idx0 a
// multiple of 8): their Philox words w, as succ(RZ(w) 2^-33) (see sr8).
__device__ __forceinline__ void words8(uint64_t idx0, uint64_t seed, uint32_t subseq, float* wz) {
  const U4 r0 = sr_words(idx0 >> 2, subseq, seed);
  const U4 r1 = sr_words((idx0 >> 2) + 1, subseq, seed);
  const uint32_t w[8] = {r0.x, r0.y, r0.z, r0.w, r1.x, r1.y, r1.z, r1.w};
  sr_unit_words(w, wz);
}

// Codes of the 8 elements of an Oct under one block multiplier (RNE or SR).
template <bool kBF16, bool kSR>
__device__ __forceinline__ uint32_t encode_oct(const Oct<kBF16>& x, float mul, bool mul_inf,
                                               const float* w) {
  uint32_t out = 0u;
  if (__builtin_expect(mul_inf, 0)) {
#pragma clang loop unroll(full)
    for (int j = 0; j < 8; ++j) out |= inf_code(x.get(j)) << (4 * j);
    return out;
  }
  if (kSR) {
    float v[8];
#pragma clang loop unroll(full)
    for (int j = 0; j < 8; ++j) v[j] = x.get(j) * mul;
    out = sr8(v, w);
  } else {
    out = FP4Q_ENC2(out, x.get(0) * mul, x.get(1) * mul, 0);
    out = FP4Q_ENC2(out, x.get(2) * mul, x.get(3) * mul, 1);
    out = FP4Q_ENC2(out, x.get(4) * mul, x.get(5) * mul, 2);
    out = FP4Q_ENC2(out, x.get(6) * mul, x.get(7) * mul, 3);
  }
  return out;
}

__device__ __forceinline__ void add_diag(int32_t* diag, uint32_t nzero, uint32_t nsat) {
#pragma clang loop unroll(full)
  for (int off = 32; off >= 1; off >>= 1) {
    nzero += (uint32_t)__shfl_xor((int)nzero, off);
    nsat += (uint32_t)__shfl_xor((int)nsat, off);
  }
  if ((threadIdx.x & 63) == 0) {
    if (nzero) atomicAdd(diag, (int32_t)nzero);
    if (nsat) atomicAdd(diag + 1, (int32_t)nsat);
  }
}

__global__ void zero_diag(int32_t* d) {
  d[0] = 0;
  d[1] = 0;
}

// Writes the tensor scale when there is no block to carry it (empty tensor).
__global__ void write_scale_only(const float* amax_held, float target, float* enc_out) {
  *enc_out = tensor_scale(*amax_held, target);
}

// Work order for 2-D tile grids: workgroup L runs on XCD L % 8; each XCD
// gets a contiguous range of work items, so the row groups that share the
// same output lines of a transposed layout run back to back in one L2.
__device__ __forceinline__ int xcd_order(int L, int n) {
  const int per = (n + 7) / 8;
  const int xcd = L % 8;
  const int local = L / 8;
  const int full = n % 8 ? n % 8 : 8;
  return xcd < full ? xcd * per + local : full * per + (xcd - full) * (per - 1) + local;
}

// ------------------------------------------------------------------ ROW
// One block (kBlk = 16 or 32 elements, kBlk / 8 Octs) per lane. A workgroup
// (one wave) covers kRowThreads consecutive blocks of one row; small
// workgroups measured fastest for this stream.
constexpr int kRowThreads = 64;

// Stores the kBlk / 2 code bytes of one block (8-byte aligned destination).
template <int kBlk>
__device__ __forceinline__ void store_block_codes(uint8_t* dst, const uint32_t (&cw)[kBlk / 8]) {
#pragma clang loop unroll(full)
  for (int j = 0; j < kBlk / 16; ++j)
    reinterpret_cast<uint2*>(dst)[j] = make_uint2(cw[2 * j], cw[2 * j + 1]);
}

template <bool kBF16, bool kSR, int kBlk>
__global__ __launch_bounds__(kRowThreads) void quant_row_kernel(
    const uint8_t* __restrict__ x, int64_t rows, int64_t cols, int64_t ld_bytes, int segs_per_row,
    const float* __restrict__ amax_held, float target, int e4m3, int k64, uint64_t seed,
    uint32_t subseq, uint8_t* __restrict__ codes, uint8_t* __restrict__ scales,
    float* __restrict__ enc_out, int32_t* __restrict__ diag) {
  constexpr int es = kBF16 ? 2 : 4;
  constexpr int kOcts = kBlk / 8;
  const int64_t row = blockIdx.x / segs_per_row;
  const int seg = blockIdx.x - (int)(row * segs_per_row);
  const float S = tensor_scale(*amax_held, target);
  const double S_d = (double)S;
  if (enc_out && blockIdx.x == 0 && threadIdx.x == 0) *enc_out = S;
  const int64_t nblk = cols / kBlk;
  const int64_t blk = (int64_t)seg * kRowThreads + threadIdx.x;
  uint32_t nzero = 0u, nsat = 0u;
  if (blk < nblk) {
    const uint8_t* p = x + row * ld_bytes + blk * kBlk * es;
    Oct<kBF16> o[kOcts];
    uint32_t m = 0u;
#pragma clang loop unroll(full)
    for (int j = 0; j < kOcts; ++j) {
      o[j].load(p + 8 * j * es);
      m = max(m, o[j].absmax());
    }
    const BlockScale s = block_scale(m, S, S_d, e4m3 != 0);
    float w[kBlk];
    if (kSR) {
      const uint64_t idx0 = (uint64_t)row * (uint64_t)cols + (uint64_t)blk * kBlk;
#pragma clang loop unroll(full)
      for (int j = 0; j < kOcts; ++j) words8(idx0 + 8 * j, seed, subseq, w + 8 * j);
    }
    const bool mi = __builtin_isinf(s.mul);
    uint32_t cw[kOcts];
#pragma clang loop unroll(full)
    for (int j = 0; j < kOcts; ++j) cw[j] = encode_oct<kBF16, kSR>(o[j], s.mul, mi, w + 8 * j);
    store_block_codes<kBlk>(codes + code_offset(row, blk * (kBlk / 2), rows, cols, k64), cw);
    scales[scale_offset<64 / kBlk>(row, blk, rows, nblk, k64)] = (uint8_t)s.code;
    nzero = s.flags & 1u;
    nsat = s.flags >> 1;
  }
  if (diag) add_diag(diag, nzero, nsat);
}

// ------------------------------------------------------------------ ROW + COL
// A workgroup owns a tile of kDualRows(kBlk) = 4 kBlk rows by kDualCols(kBlk)
// = 1024 / kBlk columns (64 x 64 for blocks of 16, 128 x 32 for 32), with
// one block per thread in each phase. Phase 1: thread t takes one row block
// (row t / (cols per tile / kBlk)): coalesced loads, the ROW codes and scale
// when requested, and for SR the Philox words; it parks the raw inputs (and
// words) in LDS. Phase 2: thread t takes column t % cols-per-tile and the
// kBlk rows of block t / cols-per-tile (one COL block), reading LDS down the
// column, and writes the COL codes and scale. Each element's Philox word
// serves both orientations. Tiles are ordered so that one XCD runs the row
// tiles of a column tile back to back (they fill the same lines of the COL
// codes).
template <int kBlk>
constexpr int kDualCols() { return 1024 / kBlk; }
template <int kBlk>
constexpr int kDualRows() { return 4 * kBlk; }
template <int kBlk>
constexpr int kDualThreads() { return 4 * kDualCols<kBlk>(); }

// 8 RNE codes of v[0..7] * mu (the conversion takes a constant selector).
__device__ __forceinline__ uint32_t rne8(const float* v, float mu) {
  uint32_t w = 0u;
  w = FP4Q_ENC2(w, v[0] * mu, v[1] * mu, 0);
  w = FP4Q_ENC2(w, v[2] * mu, v[3] * mu, 1);
  w = FP4Q_ENC2(w, v[4] * mu, v[5] * mu, 2);
  w = FP4Q_ENC2(w, v[6] * mu, v[7] * mu, 3);
  return w;
}

template <bool kBF16, bool kSR, bool kRow, int kBlk>
__global__ __launch_bounds__(kDualThreads<kBlk>()) void quant_dual_kernel(
    const uint8_t* __restrict__ x, int64_t rows, int64_t cols, int64_t ld_bytes, int col_tiles,
    int row_tiles, const float* __restrict__ amax_held, float target, int e4m3, int k64,
    uint64_t seed, uint32_t subseq, uint8_t* __restrict__ codes_r, uint8_t* __restrict__ scales_r,
    uint8_t* __restrict__ codes_c, uint8_t* __restrict__ scales_c, float* __restrict__ enc_out,
    int32_t* __restrict__ diag) {
  constexpr int es = kBF16 ? 2 : 4;
  constexpr int kTC = kDualCols<kBlk>();
  constexpr int kTR = kDualRows<kBlk>();
  constexpr int kOcts = kBlk / 8;
  constexpr int kBPR = kTC / kBlk;          // row blocks per tile row
  constexpr int kXPitch = kTC * es + 16;    // bytes per LDS row of inputs (16 B pad)
  constexpr int kWPitch = kTC * 4 + 16;     // bytes per LDS row of Philox words
  __shared__ __attribute__((aligned(16))) uint8_t lx[kTR * kXPitch];
  __shared__ __attribute__((aligned(16))) uint8_t lw[kSR ? kTR * kWPitch : 16];

  const int item = xcd_order(blockIdx.x, col_tiles * row_tiles);
  const int ct = item / row_tiles;
  const int rt = item - ct * row_tiles;
  const int64_t r0 = (int64_t)rt * kTR;
  const int64_t c0 = (int64_t)ct * kTC;
  const float S = tensor_scale(*amax_held, target);
  const double S_d = (double)S;
  if (enc_out && blockIdx.x == 0 && threadIdx.x == 0) *enc_out = S;
  const int t = threadIdx.x;
  uint32_t nzero = 0u, nsat = 0u;

  // ---- phase 1: one row block per thread
  {
    const int r = t / kBPR;
    const int q = t % kBPR;
    const int64_t gr = r0 + r;
    const int64_t gc = c0 + kBlk * q;
    const bool vr = gr < rows;
    Oct<kBF16> o[kOcts];
#pragma clang loop unroll(full)
    for (int j = 0; j < kOcts; ++j) {
      if (vr && gc + 8 * j < cols) o[j].load(x + gr * ld_bytes + (gc + 8 * j) * es);
      else o[j].zero();
    }
    float w[kBlk];
    if (kSR) {
      const uint64_t idx0 = (uint64_t)gr * (uint64_t)cols + (uint64_t)gc;
#pragma clang loop unroll(full)
      for (int j = 0; j < kOcts; ++j) words8(idx0 + 8 * j, seed, subseq, w + 8 * j);
    }
    if (kRow && vr && gc < cols) {  // cols % kBlk == 0 here: the whole block is valid
      uint32_t m = 0u;
#pragma clang loop unroll(full)
      for (int j = 0; j < kOcts; ++j) m = max(m, o[j].absmax());
      const BlockScale s = block_scale(m, S, S_d, e4m3 != 0);
      const bool mi = __builtin_isinf(s.mul);
      uint32_t cw[kOcts];
#pragma clang loop unroll(full)
      for (int j = 0; j < kOcts; ++j) cw[j] = encode_oct<kBF16, kSR>(o[j], s.mul, mi, w + 8 * j);
      store_block_codes<kBlk>(codes_r + code_offset(gr, gc / 2, rows, cols, k64), cw);
      scales_r[scale_offset<64 / kBlk>(gr, gc / kBlk, rows, cols / kBlk, k64)] = (uint8_t)s.code;
      nzero += s.flags & 1u;
      nsat += s.flags >> 1;
    }
    uint4* dx = reinterpret_cast<uint4*>(lx + r * kXPitch + kBlk * q * es);
#pragma clang loop unroll(full)
    for (int j = 0; j < kOcts; ++j) {
      if (kBF16) {
        dx[j] = make_uint4(o[j].d[0], o[j].d[1], o[j].d[2], o[j].d[3]);
      } else {
        dx[2 * j] = make_uint4(o[j].d[0], o[j].d[1], o[j].d[2], o[j].d[3]);
        dx[2 * j + 1] = make_uint4(o[j].d[4], o[j].d[5], o[j].d[6], o[j].d[7]);
      }
    }
    if (kSR) {
      float4* dw = reinterpret_cast<float4*>(lw + r * kWPitch + 4 * kBlk * q);
#pragma clang loop unroll(full)
      for (int k = 0; k < kBlk / 4; ++k) dw[k] = make_float4(w[4 * k], w[4 * k + 1], w[4 * k + 2], w[4 * k + 3]);
    }
  }
  lds_barrier();  // phase 2 reads LDS only; the ROW code stores may still be in flight

  // ---- phase 2: one column block per thread
  {
    const int c = t % kTC;
    const int rb = t / kTC;
    const int64_t gc = c0 + c;
    const int64_t gr0 = r0 + kBlk * rb;
    if (gc < cols && gr0 < rows) {
      float v[kBlk];
      uint32_t m = 0u;
#pragma clang loop unroll(full)
      for (int r = 0; r < kBlk; ++r) {
        const uint8_t* src = lx + (kBlk * rb + r) * kXPitch + c * es;
        v[r] = kBF16 ? u2f((uint32_t)*reinterpret_cast<const uint16_t*>(src) << 16)
                     : *reinterpret_cast<const float*>(src);
        m = max(m, f2u(v[r]) & 0x7FFFFFFFu);
      }
      const BlockScale s = block_scale(m, S, S_d, e4m3 != 0);
      const bool mi = __builtin_isinf(s.mul);
      uint32_t cw[kOcts];
#pragma clang loop unroll(full)
      for (int j = 0; j < kOcts; ++j) cw[j] = 0u;
      if (__builtin_expect(mi, 0)) {
#pragma clang loop unroll(full)
        for (int r = 0; r < kBlk; ++r) cw[r >> 3] |= inf_code(v[r]) << (4 * (r & 7));
      } else if (kSR) {
#pragma clang loop unroll(full)
        for (int j = 0; j < kOcts; ++j) {
          float vs[8], wr[8];
#pragma clang loop unroll(full)
          for (int i = 0; i < 8; ++i) {
            vs[i] = v[8 * j + i] * s.mul;
            wr[i] = *reinterpret_cast<const float*>(lw + (kBlk * rb + 8 * j + i) * kWPitch + 4 * c);
          }
          cw[j] = sr8(vs, wr);
        }
      } else {
#pragma clang loop unroll(full)
        for (int j = 0; j < kOcts; ++j) cw[j] = rne8(v + 8 * j, s.mul);
      }
      store_block_codes<kBlk>(codes_c + code_offset(gc, gr0 / 2, cols, rows, k64), cw);
      scales_c[scale_offset<64 / kBlk>(gc, gr0 / kBlk, cols, rows / kBlk, k64)] = (uint8_t)s.code;
      nzero += s.flags & 1u;
      nsat += s.flags >> 1;
    }
  }
  if (diag) add_diag(diag, nzero, nsat);
}

// 16-row tile rows per lane: two (32 rows, 16 contiguous transposed bytes
// per column) measured faster than four for bf16 inputs, whose smaller grid
// left too few waves per SIMD to keep the loads in flight. Even, since
// store_col_codes writes 16-byte pieces.
constexpr int kTileSub = 2;

// Stores the 8 * kSub bytes of one column's codes (nsub sub-tiles valid),
// as 16-byte pieces when the column row is 16-byte aligned.
template <int kSub>
__device__ __forceinline__ void store_col_codes(uint8_t* dst, const uint32_t (&cw)[2 * kSub], int nsub,
                                                bool wide) {
  if (wide && nsub == kSub) {
#pragma clang loop unroll(full)
    for (int q = 0; q < kSub / 2; ++q)
      reinterpret_cast<uint4*>(dst)[q] = make_uint4(cw[4 * q], cw[4 * q + 1], cw[4 * q + 2], cw[4 * q + 3]);
  } else {
#pragma clang loop unroll(full)
    for (int st = 0; st < kSub; ++st)
      if (st < nsub) reinterpret_cast<uint2*>(dst)[st] = make_uint2(cw[2 * st], cw[2 * st + 1]);
  }
}

// ------------------------------------------------------------------ TILE16
// A lane holds 8 columns of kSub tile rows; a lane pair covers 16 x 16
// tiles. The transposed copy gets 8 * kSub contiguous bytes per column.
template <bool kBF16, bool kSR, bool kT>
__global__ __launch_bounds__(kThreads) void quant_tile_kernel(
    const uint8_t* __restrict__ x, int64_t rows, int64_t cols, int64_t ld_bytes, int col_groups,
    int row_groups, const float* __restrict__ amax_held, float target, int e4m3, int k64,
    uint64_t seed, uint32_t subseq, uint8_t* __restrict__ codes, uint8_t* __restrict__ scales,
    uint8_t* __restrict__ codes_t, uint8_t* __restrict__ scales_t, float* __restrict__ enc_out,
    int32_t* __restrict__ diag) {
  constexpr int es = kBF16 ? 2 : 4;
  constexpr int kSub = kTileSub;
  const int item = xcd_order(blockIdx.x, col_groups * row_groups);
  const int cg = item / row_groups;
  const int rg = item - cg * row_groups;
  const float S = tensor_scale(*amax_held, target);
  const double S_d = (double)S;
  if (enc_out && blockIdx.x == 0 && threadIdx.x == 0) *enc_out = S;
  const int64_t oct = (int64_t)cg * kThreads + threadIdx.x;
  const int64_t c0 = oct * 8;
  const bool valid = c0 < cols;  // equal within a lane pair (cols % 16 == 0)
  const int64_t r_begin = (int64_t)rg * 16 * kSub;
  const int nsub = (int)min((int64_t)kSub, (rows - r_begin) / 16);
  uint32_t nzero = 0u, nsat = 0u;
  uint32_t tcodes[8][2 * kSub];
#pragma clang loop unroll(full)
  for (int j = 0; j < 8; ++j)
#pragma clang loop unroll(full)
    for (int q = 0; q < 2 * kSub; ++q) tcodes[j][q] = 0u;

#pragma clang loop unroll(full)
  for (int st = 0; st < kSub; ++st) {
    if (st < nsub) {
    const int64_t r0 = r_begin + st * 16;
    Oct<kBF16> v[16];
    uint32_t m = 0u;
#pragma clang loop unroll(full)
    for (int r = 0; r < 16; ++r) {
      if (valid)
        v[r].load(x + (r0 + r) * ld_bytes + c0 * es);
      else
        v[r].zero();
      m = max(m, v[r].absmax());
    }
    m = max(m, (uint32_t)__shfl_xor((int)m, 1));
    const BlockScale b = block_scale(m, S, S_d, e4m3 != 0);
    const bool mi = __builtin_isinf(b.mul);
#pragma clang loop unroll(full)
    for (int r = 0; r < 16; ++r) {
      float w[8];
      if (kSR) words8((uint64_t)(r0 + r) * (uint64_t)cols + (uint64_t)c0, seed, subseq, w);
      const uint32_t word = encode_oct<kBF16, kSR>(v[r], b.mul, mi, w);
      if (valid) *reinterpret_cast<uint32_t*>(codes + code_offset(r0 + r, 4 * oct, rows, cols, k64)) = word;
      if (kT) {
#pragma clang loop unroll(full)
        for (int j = 0; j < 8; ++j)
          tcodes[j][2 * st + (r >> 3)] |= ((word >> (4 * j)) & 0xFu) << (4 * (r & 7));
      }
    }
    if (valid && (threadIdx.x & 1) == 0) {
      scales[scale_offset<4>(r0 / 16, oct >> 1, rows / 16, cols / 16, k64)] = (uint8_t)b.code;
      if (kT) scales_t[scale_offset<4>(oct >> 1, r0 / 16, cols / 16, rows / 16, k64)] = (uint8_t)b.code;
      nzero += b.flags & 1u;
      nsat += b.flags >> 1;
    }
    }  // st < nsub
  }
  if (kT && valid && nsub > 0) {
    // K64 runs are 16-byte aligned (each column's 8 * kSub bytes sit inside
    // one 32-byte tile row)
    const bool wide = k64 || (rows / 2) % 16 == 0;
#pragma clang loop unroll(full)
    for (int j = 0; j < 8; ++j)
      store_col_codes<kSub>(codes_t + code_offset(c0 + j, r_begin / 2, cols, rows, k64), tcodes[j], nsub,
                            wide);
  }
  if (diag) add_diag(diag, nzero, nsat);
}


// ------------------------------------------------------------------ TILE32
// 32 x 32 tiles (the block-32 weight layout). A lane holds 8 columns of one
// 32-row tile band; four adjacent lanes cover a tile. The band is read twice
// (once for the tile maxima, once to encode: the second read hits the
// cache), so a lane keeps one row at a time. The transposed copy gets 16
// contiguous bytes per column.
template <bool kBF16, bool kSR, bool kT>
__global__ __launch_bounds__(kThreads) void quant_tile32_kernel(
    const uint8_t* __restrict__ x, int64_t rows, int64_t cols, int64_t ld_bytes, int col_groups,
    int row_groups, const float* __restrict__ amax_held, float target, int e4m3, int k64,
    uint64_t seed, uint32_t subseq, uint8_t* __restrict__ codes, uint8_t* __restrict__ scales,
    uint8_t* __restrict__ codes_t, uint8_t* __restrict__ scales_t, float* __restrict__ enc_out,
    int32_t* __restrict__ diag) {
  constexpr int es = kBF16 ? 2 : 4;
  const int item = xcd_order(blockIdx.x, col_groups * row_groups);
  const int cg = item / row_groups;
  const int rg = item - cg * row_groups;
  const float S = tensor_scale(*amax_held, target);
  const double S_d = (double)S;
  if (enc_out && blockIdx.x == 0 && threadIdx.x == 0) *enc_out = S;
  const int64_t oct = (int64_t)cg * kThreads + threadIdx.x;
  const int64_t c0 = oct * 8;
  const bool valid = c0 < cols;  // equal within a lane quad (cols % 32 == 0)
  const int64_t r0 = (int64_t)rg * 32;
  uint32_t m = 0u;
#pragma clang loop unroll(full)
  for (int r = 0; r < 32; ++r) {
    Oct<kBF16> v;
    if (valid) v.load(x + (r0 + r) * ld_bytes + c0 * es);
    else v.zero();
    m = max(m, v.absmax());
  }
  m = max(m, (uint32_t)__shfl_xor((int)m, 1));
  m = max(m, (uint32_t)__shfl_xor((int)m, 2));
  const BlockScale b = block_scale(m, S, S_d, e4m3 != 0);
  const bool mi = __builtin_isinf(b.mul);
  uint32_t tcodes[8][4];
#pragma clang loop unroll(full)
  for (int j = 0; j < 8; ++j)
#pragma clang loop unroll(full)
    for (int q = 0; q < 4; ++q) tcodes[j][q] = 0u;
#pragma clang loop unroll(full)
  for (int r = 0; r < 32; ++r) {
    Oct<kBF16> v;
    if (valid) v.load(x + (r0 + r) * ld_bytes + c0 * es);
    else v.zero();
    float w[8];
    if (kSR) words8((uint64_t)(r0 + r) * (uint64_t)cols + (uint64_t)c0, seed, subseq, w);
    const uint32_t word = encode_oct<kBF16, kSR>(v, b.mul, mi, w);
    if (valid) *reinterpret_cast<uint32_t*>(codes + code_offset(r0 + r, 4 * oct, rows, cols, k64)) = word;
    if (kT) {
#pragma clang loop unroll(full)
      for (int j = 0; j < 8; ++j) tcodes[j][r >> 3] |= ((word >> (4 * j)) & 0xFu) << (4 * (r & 7));
    }
  }
  uint32_t nzero = 0u, nsat = 0u;
  if (valid && (threadIdx.x & 3) == 0) {
    scales[scale_offset<2>(r0 / 32, oct >> 2, rows / 32, cols / 32, k64)] = (uint8_t)b.code;
    if (kT) scales_t[scale_offset<2>(oct >> 2, r0 / 32, cols / 32, rows / 32, k64)] = (uint8_t)b.code;
    nzero = b.flags & 1u;
    nsat = b.flags >> 1;
  }
  if (kT && valid) {
#pragma clang loop unroll(full)
    for (int j = 0; j < 8; ++j)
      store_block_codes<32>(codes_t + code_offset(c0 + j, r0 / 2, cols, rows, k64), tcodes[j]);
  }
  if (diag) add_diag(diag, nzero, nsat);
}

template <bool kBF16, bool kSR, int kBlk>
hipError_t launch_typed(const QuantArgs& a, hipStream_t s) {
  const uint8_t* x = static_cast<const uint8_t*>(a.x);
  const int64_t ldb = a.ld * a.es;
  const int e4m3 = a.scale_fmt;
  const int k64 = a.pack;
  const bool both = a.layout == 0 && a.codes_t != nullptr;
  if (a.layout == 0 && !both) {
    const int64_t nblk = a.cols / kBlk;
    const int segs = (int)((nblk + kRowThreads - 1) / kRowThreads);
    hipLaunchKernelGGL((quant_row_kernel<kBF16, kSR, kBlk>), dim3((uint32_t)(a.rows * segs)),
                       dim3(kRowThreads), 0, s, x, a.rows, a.cols, ldb, segs, a.amax_held, a.target,
                       e4m3, k64, a.seed, a.subseq, a.codes, a.scales, a.enc_scale_out, a.diag);
    return hipGetLastError();
  }
  if (a.layout == 2) {
    const int col_groups = (int)((a.cols / 8 + kThreads - 1) / kThreads);
    if (kBlk == 32) {
      const dim3 grid((uint32_t)(col_groups * (a.rows / 32)));
      if (a.codes_t)
        hipLaunchKernelGGL((quant_tile32_kernel<kBF16, kSR, true>), grid, dim3(kThreads), 0, s, x,
                           a.rows, a.cols, ldb, col_groups, (int)(a.rows / 32), a.amax_held, a.target,
                           e4m3, k64, a.seed, a.subseq, a.codes, a.scales, a.codes_t, a.scales_t,
                           a.enc_scale_out, a.diag);
      else
        hipLaunchKernelGGL((quant_tile32_kernel<kBF16, kSR, false>), grid, dim3(kThreads), 0, s, x,
                           a.rows, a.cols, ldb, col_groups, (int)(a.rows / 32), a.amax_held, a.target,
                           e4m3, k64, a.seed, a.subseq, a.codes, a.scales, nullptr, nullptr,
                           a.enc_scale_out, a.diag);
      return hipGetLastError();
    }
    constexpr int ksub = kTileSub;
    const int row_groups = (int)((a.rows / 16 + ksub - 1) / ksub);
    const dim3 grid((uint32_t)(col_groups * row_groups));
    if (a.codes_t)
      hipLaunchKernelGGL((quant_tile_kernel<kBF16, kSR, true>), grid, dim3(kThreads), 0, s, x, a.rows,
                         a.cols, ldb, col_groups, row_groups, a.amax_held, a.target, e4m3, k64, a.seed,
                         a.subseq, a.codes, a.scales, a.codes_t, a.scales_t, a.enc_scale_out, a.diag);
    else
      hipLaunchKernelGGL((quant_tile_kernel<kBF16, kSR, false>), grid, dim3(kThreads), 0, s, x, a.rows,
                         a.cols, ldb, col_groups, row_groups, a.amax_held, a.target, e4m3, k64, a.seed,
                         a.subseq, a.codes, a.scales, nullptr, nullptr, a.enc_scale_out, a.diag);
    return hipGetLastError();
  }
  constexpr int kTC = kDualCols<kBlk>(), kTR = kDualRows<kBlk>();
  const int col_tiles = (int)((a.cols + kTC - 1) / kTC);
  const int row_tiles = (int)((a.rows + kTR - 1) / kTR);
  const dim3 grid((uint32_t)(col_tiles * row_tiles)), block(kDualThreads<kBlk>());
  if (both) {
    // ROW outputs in codes/scales, COL outputs in codes_t/scales_t
    hipLaunchKernelGGL((quant_dual_kernel<kBF16, kSR, true, kBlk>), grid, block, 0, s, x, a.rows,
                       a.cols, ldb, col_tiles, row_tiles, a.amax_held, a.target, e4m3, k64, a.seed,
                       a.subseq, a.codes, a.scales, a.codes_t, a.scales_t, a.enc_scale_out, a.diag);
  } else {
    hipLaunchKernelGGL((quant_dual_kernel<kBF16, kSR, false, kBlk>), grid, block, 0, s, x, a.rows,
                       a.cols, ldb, col_tiles, row_tiles, a.amax_held, a.target, e4m3, k64, a.seed,
                       a.subseq, nullptr, nullptr, a.codes, a.scales, a.enc_scale_out, a.diag);
  }
  return hipGetLastError();
}

template <bool kBF16, bool kSR>
hipError_t launch_block(const QuantArgs& a, hipStream_t s) {
  return a.block == 32 ? launch_typed<kBF16, kSR, 32>(a, s) : launch_typed<kBF16, kSR, 16>(a, s);
}

}  // namespace

hipError_t launch_quantize(const QuantArgs& a, hipStream_t s) {
  if (a.diag) hipLaunchKernelGGL(zero_diag, dim3(1), dim3(1), 0, s, a.diag);
  if (a.rows == 0 || a.cols == 0) {
    if (a.enc_scale_out)
      hipLaunchKernelGGL(write_scale_only, dim3(1), dim3(1), 0, s, a.amax_held, a.target,
                         a.enc_scale_out);
    return hipGetLastError();
  }
  if (a.es == 2) return a.sr ? launch_block<true, true>(a, s) : launch_block<true, false>(a, s);
  return a.sr ? launch_block<false, true>(a, s) : launch_block<false, false>(a, s);
}

}  // namespace fp4q
