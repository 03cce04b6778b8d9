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

// Philox words of source elements idx0 .. idx0+7 (idx0 a multiple of 8).
__device__ __forceinline__ void words8(uint64_t idx0, uint64_t seed, uint32_t subseq, uint32_t* w) {
  const U4 r0 = sr_words(idx0 >> 2, subseq, seed);
  const U4 r1 = sr_words((idx0 >> 2) + 1, subseq, seed);
  w[0] = r0.x; w[1] = r0.y; w[2] = r0.z; w[3] = r0.w;
  w[4] = r1.x; w[5] = r1.y; w[6] = r1.z; w[7] = r1.w;
}

// Codes of the 8 elements of an Oct under one block multiplier (RNE or SR).
template <bool kBF16, bool kSR>
__device__ __forceinline__ uint32_t encode_oct(const Oct<kBF16>& x, float mul, bool mul_inf,
                                               const uint32_t* w) {
  uint32_t out = 0u;
  if (__builtin_expect(mul_inf, 0)) {
#pragma clang loop unroll(full)
    for (int j = 0; j < 8; ++j) out |= inf_code(x.get(j)) << (4 * j);
    return out;
  }
  if (kSR) {
#pragma clang loop unroll(full)
    for (int j = 0; j < 8; ++j) out |= sr_code(x.get(j) * mul, w[j]) << (4 * j);
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

// ------------------------------------------------------------------ ROW16
// One 16-element block per lane (two Octs). A workgroup (one wave) covers
// kRowThreads consecutive blocks of one row; small workgroups measured
// fastest for this stream.
constexpr int kRowThreads = 64;

template <bool kBF16, bool kSR>
__global__ __launch_bounds__(kRowThreads) void quant_row16_kernel(
    const uint8_t* __restrict__ x, int64_t cols, int64_t ld_bytes, int segs_per_row,
    const float* __restrict__ amax_held, float target, uint64_t seed, uint32_t subseq,
    uint8_t* __restrict__ codes, uint8_t* __restrict__ scales, float* __restrict__ enc_out,
    int32_t* __restrict__ diag) {
  constexpr int es = kBF16 ? 2 : 4;
  const int64_t row = blockIdx.x / segs_per_row;
  const int seg = blockIdx.x - (int)(row * segs_per_row);
  const float S = tensor_scale(*amax_held, target);
  const double S_d = (double)S;
  if (enc_out && blockIdx.x == 0 && threadIdx.x == 0) *enc_out = S;
  const int64_t nblk = cols / 16;
  const int64_t blk = (int64_t)seg * kRowThreads + threadIdx.x;
  uint32_t nzero = 0u, nsat = 0u;
  if (blk < nblk) {
    const uint8_t* p = x + row * ld_bytes + blk * 16 * es;
    Oct<kBF16> a, b;
    a.load(p);
    b.load(p + 8 * es);
    const BlockScale s = block_scale(max(a.absmax(), b.absmax()), S, S_d);
    uint32_t w[16];
    if (kSR) {
      const uint64_t idx0 = (uint64_t)row * (uint64_t)cols + (uint64_t)blk * 16;
      words8(idx0, seed, subseq, w);
      words8(idx0 + 8, seed, subseq, w + 8);
    }
    const bool mi = __builtin_isinf(s.mul);
    const uint32_t lo = encode_oct<kBF16, kSR>(a, s.mul, mi, w);
    const uint32_t hi = encode_oct<kBF16, kSR>(b, s.mul, mi, w + 8);
    *reinterpret_cast<uint2*>(codes + row * (cols / 2) + blk * 8) = make_uint2(lo, hi);
    scales[row * nblk + blk] = (uint8_t)s.code;
    nzero = s.flags & 1u;
    nsat = s.flags >> 1;
  }
  if (diag) add_diag(diag, nzero, nsat);
}

// ------------------------------------------------------------------ ROW16 + COL16
// A workgroup owns a 64 x 64 tile. Phase 1: thread t takes row t / 4 and 16
// columns 16 (t % 4) .. +15 (one ROW16 block): coalesced loads, the ROW16
// codes and scale when requested, and for SR the 16 Philox words; it parks
// the raw inputs (and words) in LDS. Phase 2: thread t takes column t % 64
// and rows 16 (t / 64) .. +15 (one COL16 block), reading LDS down the column
// (a wave reads one LDS row, 64 consecutive elements: no bank conflicts),
// and writes the COL16 codes and scale. Each element's Philox word serves
// both orientations. Tiles are ordered so that one XCD runs the row tiles of
// a column tile back to back (they fill the same lines of the COL16 codes).
constexpr int kTT = 64;  // tile rows and columns

template <bool kBF16, bool kSR, bool kRow>
__global__ __launch_bounds__(kThreads) void quant_dual_kernel(
    const uint8_t* __restrict__ x, int64_t rows, int64_t cols, int64_t ld_bytes, int col_tiles,
    int row_tiles, const float* __restrict__ amax_held, float target, uint64_t seed,
    uint32_t subseq, uint8_t* __restrict__ codes_r, uint8_t* __restrict__ scales_r,
    uint8_t* __restrict__ codes_c, uint8_t* __restrict__ scales_c, float* __restrict__ enc_out,
    int32_t* __restrict__ diag) {
  constexpr int es = kBF16 ? 2 : 4;
  constexpr int kXPitch = kTT * es + 16;  // bytes per LDS row of inputs (16 B pad)
  constexpr int kWPitch = kTT * 4 + 16;   // bytes per LDS row of Philox words
  __shared__ __attribute__((aligned(16))) uint8_t lx[kTT * kXPitch];
  __shared__ __attribute__((aligned(16))) uint8_t lw[kSR ? kTT * kWPitch : 16];

  const int item = xcd_order(blockIdx.x, col_tiles * row_tiles);
  const int ct = item / row_tiles;
  const int rt = item - ct * row_tiles;
  const int64_t r0 = (int64_t)rt * kTT;
  const int64_t c0 = (int64_t)ct * kTT;
  const float S = tensor_scale(*amax_held, target);
  const double S_d = (double)S;
  if (enc_out && blockIdx.x == 0 && threadIdx.x == 0) *enc_out = S;
  const int t = threadIdx.x;
  uint32_t nzero = 0u, nsat = 0u;

  // ---- phase 1: one row block per thread
  {
    const int r = t >> 2;
    const int q = t & 3;
    const int64_t gr = r0 + r;
    const int64_t gc = c0 + 16 * q;
    const bool vr = gr < rows;
    const bool v0 = vr && gc < cols;
    const bool v1 = vr && gc + 8 < cols;
    Oct<kBF16> a, b;
    if (v0) a.load(x + gr * ld_bytes + gc * es); else a.zero();
    if (v1) b.load(x + gr * ld_bytes + (gc + 8) * es); else b.zero();
    uint32_t w[16];
    if (kSR) {
      const uint64_t idx0 = (uint64_t)gr * (uint64_t)cols + (uint64_t)gc;
      words8(idx0, seed, subseq, w);
      words8(idx0 + 8, seed, subseq, w + 8);
    }
    if (kRow && v0) {  // cols % 16 == 0 here, so v0 implies v1
      const BlockScale s = block_scale(max(a.absmax(), b.absmax()), S, S_d);
      const bool mi = __builtin_isinf(s.mul);
      const uint32_t lo = encode_oct<kBF16, kSR>(a, s.mul, mi, w);
      const uint32_t hi = encode_oct<kBF16, kSR>(b, s.mul, mi, w + 8);
      *reinterpret_cast<uint2*>(codes_r + gr * (cols / 2) + gc / 2) = make_uint2(lo, hi);
      scales_r[gr * (cols / 16) + gc / 16] = (uint8_t)s.code;
      nzero += s.flags & 1u;
      nsat += s.flags >> 1;
    }
    uint4* dx = reinterpret_cast<uint4*>(lx + r * kXPitch + 16 * q * es);
    if (kBF16) {
      dx[0] = make_uint4(a.d[0], a.d[1], a.d[2], a.d[3]);
      dx[1] = make_uint4(b.d[0], b.d[1], b.d[2], b.d[3]);
    } else {
      dx[0] = make_uint4(a.d[0], a.d[1], a.d[2], a.d[3]);
      dx[1] = make_uint4(a.d[4], a.d[5], a.d[6], a.d[7]);
      dx[2] = make_uint4(b.d[0], b.d[1], b.d[2], b.d[3]);
      dx[3] = make_uint4(b.d[4], b.d[5], b.d[6], b.d[7]);
    }
    if (kSR) {
      uint4* dw = reinterpret_cast<uint4*>(lw + r * kWPitch + 64 * q);
#pragma clang loop unroll(full)
      for (int k = 0; k < 4; ++k) dw[k] = make_uint4(w[4 * k], w[4 * k + 1], w[4 * k + 2], w[4 * k + 3]);
    }
  }
  __syncthreads();

  // ---- phase 2: one column block per thread
  {
    const int c = t & (kTT - 1);
    const int rb = t >> 6;
    const int64_t gc = c0 + c;
    const int64_t gr0 = r0 + 16 * rb;
    if (gc < cols && gr0 < rows) {
      float v[16];
      uint32_t m = 0u;
#pragma clang loop unroll(full)
      for (int r = 0; r < 16; ++r) {
        const uint8_t* src = lx + (16 * rb + r) * kXPitch + c * es;
        v[r] = kBF16 ? u2f((uint32_t)*reinterpret_cast<const uint16_t*>(src) << 16)
                     : *reinterpret_cast<const float*>(src);
        m = max(m, f2u(v[r]) & 0x7FFFFFFFu);
      }
      const BlockScale s = block_scale(m, S, S_d);
      const bool mi = __builtin_isinf(s.mul);
      uint32_t cw[2] = {0u, 0u};
      if (__builtin_expect(mi, 0)) {
#pragma clang loop unroll(full)
        for (int r = 0; r < 16; ++r) cw[r >> 3] |= inf_code(v[r]) << (4 * (r & 7));
      } else if (kSR) {
#pragma clang loop unroll(full)
        for (int r = 0; r < 16; ++r) {
          const uint32_t wr = *reinterpret_cast<const uint32_t*>(lw + (16 * rb + r) * kWPitch + 4 * c);
          cw[r >> 3] |= sr_code(v[r] * s.mul, wr) << (4 * (r & 7));
        }
      } else {
        const float mu = s.mul;
        cw[0] = FP4Q_ENC2(cw[0], v[0] * mu, v[1] * mu, 0);
        cw[0] = FP4Q_ENC2(cw[0], v[2] * mu, v[3] * mu, 1);
        cw[0] = FP4Q_ENC2(cw[0], v[4] * mu, v[5] * mu, 2);
        cw[0] = FP4Q_ENC2(cw[0], v[6] * mu, v[7] * mu, 3);
        cw[1] = FP4Q_ENC2(cw[1], v[8] * mu, v[9] * mu, 0);
        cw[1] = FP4Q_ENC2(cw[1], v[10] * mu, v[11] * mu, 1);
        cw[1] = FP4Q_ENC2(cw[1], v[12] * mu, v[13] * mu, 2);
        cw[1] = FP4Q_ENC2(cw[1], v[14] * mu, v[15] * mu, 3);
      }
      *reinterpret_cast<uint2*>(codes_c + gc * (rows / 2) + gr0 / 2) = make_uint2(cw[0], cw[1]);
      scales_c[gc * (rows / 16) + gr0 / 16] = (uint8_t)s.code;
      nzero += s.flags & 1u;
      nsat += s.flags >> 1;
    }
  }
  if (diag) add_diag(diag, nzero, nsat);
}

template <bool kBF16>
constexpr int sub_tiles() { return kBF16 ? 4 : 2; }

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
    int row_groups, const float* __restrict__ amax_held, float target, uint64_t seed,
    uint32_t subseq, uint8_t* __restrict__ codes, uint8_t* __restrict__ scales,
    uint8_t* __restrict__ codes_t, uint8_t* __restrict__ scales_t, float* __restrict__ enc_out,
    int32_t* __restrict__ diag) {
  constexpr int es = kBF16 ? 2 : 4;
  constexpr int kSub = sub_tiles<kBF16>();
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
    const BlockScale b = block_scale(m, S, S_d);
    const bool mi = __builtin_isinf(b.mul);
#pragma clang loop unroll(full)
    for (int r = 0; r < 16; ++r) {
      uint32_t w[8];
      if (kSR) words8((uint64_t)(r0 + r) * (uint64_t)cols + (uint64_t)c0, seed, subseq, w);
      const uint32_t word = encode_oct<kBF16, kSR>(v[r], b.mul, mi, w);
      if (valid) reinterpret_cast<uint32_t*>(codes + (r0 + r) * (cols / 2))[oct] = word;
      if (kT) {
#pragma clang loop unroll(full)
        for (int j = 0; j < 8; ++j)
          tcodes[j][2 * st + (r >> 3)] |= ((word >> (4 * j)) & 0xFu) << (4 * (r & 7));
      }
    }
    if (valid && (threadIdx.x & 1) == 0) {
      scales[(r0 / 16) * (cols / 16) + (oct >> 1)] = (uint8_t)b.code;
      if (kT) scales_t[(oct >> 1) * (rows / 16) + r0 / 16] = (uint8_t)b.code;
      nzero += b.flags & 1u;
      nsat += b.flags >> 1;
    }
    }  // st < nsub
  }
  if (kT && valid && nsub > 0) {
    const bool wide = (rows / 2) % 16 == 0;
#pragma clang loop unroll(full)
    for (int j = 0; j < 8; ++j)
      store_col_codes<kSub>(codes_t + (c0 + j) * (rows / 2) + r_begin / 2, tcodes[j], nsub, wide);
  }
  if (diag) add_diag(diag, nzero, nsat);
}

template <bool kBF16, bool kSR>
hipError_t launch_typed(const QuantArgs& a, hipStream_t s) {
  const uint8_t* x = static_cast<const uint8_t*>(a.x);
  const int64_t ldb = a.ld * a.es;
  const bool both = a.layout == 0 && a.codes_t != nullptr;
  if (a.layout == 0 && !both) {
    const int64_t nblk = a.cols / 16;
    const int segs = (int)((nblk + kRowThreads - 1) / kRowThreads);
    hipLaunchKernelGGL((quant_row16_kernel<kBF16, kSR>), dim3((uint32_t)(a.rows * segs)), dim3(kRowThreads),
                       0, s, x, a.cols, ldb, segs, a.amax_held, a.target, a.seed, a.subseq, a.codes,
                       a.scales, a.enc_scale_out, a.diag);
    return hipGetLastError();
  }
  if (a.layout == 2) {
    const int col_groups = (int)((a.cols / 8 + kThreads - 1) / kThreads);
    constexpr int ksub = sub_tiles<kBF16>();
    const int row_groups = (int)((a.rows / 16 + ksub - 1) / ksub);
    const dim3 grid((uint32_t)(col_groups * row_groups));
    if (a.codes_t)
      hipLaunchKernelGGL((quant_tile_kernel<kBF16, kSR, true>), grid, dim3(kThreads), 0, s, x, a.rows,
                         a.cols, ldb, col_groups, row_groups, a.amax_held, a.target, a.seed, a.subseq,
                         a.codes, a.scales, a.codes_t, a.scales_t, a.enc_scale_out, a.diag);
    else
      hipLaunchKernelGGL((quant_tile_kernel<kBF16, kSR, false>), grid, dim3(kThreads), 0, s, x, a.rows,
                         a.cols, ldb, col_groups, row_groups, a.amax_held, a.target, a.seed, a.subseq,
                         a.codes, a.scales, nullptr, nullptr, a.enc_scale_out, a.diag);
    return hipGetLastError();
  }
  const int col_tiles = (int)((a.cols + kTT - 1) / kTT);
  const int row_tiles = (int)((a.rows + kTT - 1) / kTT);
  const dim3 grid((uint32_t)(col_tiles * row_tiles));
  if (both) {
    // ROW16 outputs in codes/scales, COL16 outputs in codes_t/scales_t
    hipLaunchKernelGGL((quant_dual_kernel<kBF16, kSR, true>), grid, dim3(kThreads), 0, s, x, a.rows,
                       a.cols, ldb, col_tiles, row_tiles, a.amax_held, a.target, a.seed, a.subseq,
                       a.codes, a.scales, a.codes_t, a.scales_t, a.enc_scale_out, a.diag);
  } else {
    hipLaunchKernelGGL((quant_dual_kernel<kBF16, kSR, false>), grid, dim3(kThreads), 0, s, x, a.rows,
                       a.cols, ldb, col_tiles, row_tiles, a.amax_held, a.target, a.seed, a.subseq,
                       nullptr, nullptr, a.codes, a.scales, a.enc_scale_out, a.diag);
  }
  return hipGetLastError();
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
  if (a.es == 2) return a.sr ? launch_typed<true, true>(a, s) : launch_typed<true, false>(a, s);
  return a.sr ? launch_typed<false, true>(a, s) : launch_typed<false, false>(a, s);
}

}  // namespace fp4q
