// Block-scaled FP4 quantization ("UE5M3 FP4 Block Scaling for Stable
// Language Model Pretraining", §3-§5): E2M1 payloads with one UE5M3 scale per
// block under the FP32 tensor scale derived from a held amax and target T;
// RNE payloads for activations and weights, stochastic rounding with Philox
// words for upstream gradients.
//
// Layouts (codes: two elements per byte, even element in the low nibble):
//   ROW16   blocks of 16 along a row           codes [R][C/2], scales [R][C/16]
//   COL16   blocks of 16 down a column,        codes [C][R/2], scales [C][R/16]
//           stored as ROW16 of the transpose (wgrad operands, quantized
//           along the token axis)
//   TILE16  16 x 16 tiles (weights)            codes [R][C/2], scales [R/16][C/16]
//           plus an optional transposed copy   codes [C][R/2], scales [C/16][R/16]
//
// The kernels are HBM-bound (SR ones ALU-bound): every input byte is read
// once with 128-bit loads, one lane holds 8 consecutive elements of a row, and
// a block's maximum is combined across the lanes that hold it with
// cross-lane swizzles.
#include "codec.h"
#include "kernels.h"

namespace fp4q {
namespace {

constexpr int kThreads = 256;

// Eight consecutive elements held by one lane, widened to fp32.
struct Vec8 {
  float v[8];
};

template <bool kBF16>
__device__ __forceinline__ Vec8 load8(const uint8_t* p) {
  Vec8 r;
  if (kBF16) {
    const uint4 d = load_nt16(p);
    const uint32_t w[4] = {d.x, d.y, d.z, d.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      r.v[2 * i] = bf16_lo(w[i]);
      r.v[2 * i + 1] = bf16_hi(w[i]);
    }
  } else {
    const uint4 a = load_nt16(p);
    const uint4 b = load_nt16(p + 16);
    r.v[0] = u2f(a.x); r.v[1] = u2f(a.y); r.v[2] = u2f(a.z); r.v[3] = u2f(a.w);
    r.v[4] = u2f(b.x); r.v[5] = u2f(b.y); r.v[6] = u2f(b.z); r.v[7] = u2f(b.w);
  }
  return r;
}

// max |v| of 8 values as a sign-cleared bit pattern (exact for finite input)
__device__ __forceinline__ uint32_t absmax_bits8(const Vec8& x) {
  uint32_t m = 0u;
#pragma unroll
  for (int i = 0; i < 8; ++i) m = max(m, f2u(x.v[i]) & 0x7FFFFFFFu);
  return m;
}

// Eight payload codes packed into one 32-bit word (element e in bits 4e+3:4e).
// For SR, idx0 is the source linear index of element 0 (a multiple of 8).
template <bool kSR>
__device__ __forceinline__ uint32_t pack8(const Vec8& x, const BlockScale& b, uint64_t idx0,
                                          uint64_t seed, uint32_t subseq) {
  uint32_t w[8] = {0, 0, 0, 0, 0, 0, 0, 0};
  if (kSR && !b.zero && !b.mul_inf) {
    const U4 r0 = sr_words(idx0 >> 2, subseq, seed);
    const U4 r1 = sr_words((idx0 >> 2) + 1, subseq, seed);
    w[0] = r0.x; w[1] = r0.y; w[2] = r0.z; w[3] = r0.w;
    w[4] = r1.x; w[5] = r1.y; w[6] = r1.z; w[7] = r1.w;
  }
  uint32_t out = 0u;
#pragma unroll
  for (int e = 0; e < 8; ++e) out |= payload_code<kSR>(x.v[e], b, w[e]) << (4 * e);
  return out;
}

__device__ __forceinline__ void add_diag(int32_t* diag, uint32_t nzero, uint32_t nsat) {
#pragma unroll
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

// ------------------------------------------------------------------ ROW16
// Lane pairs (2t, 2t+1) hold one block; a workgroup covers kThreads * kCPT
// lane-chunks of one row segment.
template <bool kBF16, bool kSR, int kCPT>
__global__ __launch_bounds__(kThreads) void quant_row16_kernel(
    const uint8_t* __restrict__ x, int64_t rows, int64_t cols, int64_t ld_bytes, int segs_per_row,
    const float* __restrict__ amax_held, float target, uint64_t seed, uint32_t subseq,
    uint8_t* __restrict__ codes, uint8_t* __restrict__ scales, float* __restrict__ enc_out,
    int32_t* __restrict__ diag) {
  constexpr int es = kBF16 ? 2 : 4;
  const int64_t row = blockIdx.x / segs_per_row;
  const int seg = blockIdx.x - (int)(row * segs_per_row);
  const float S = tensor_scale(*amax_held, target);
  if (enc_out && blockIdx.x == 0 && threadIdx.x == 0) *enc_out = S;
  const int64_t chunks = cols / 8;
  uint32_t nzero = 0, nsat = 0;
  const uint8_t* xrow = x + row * ld_bytes;
#pragma unroll
  for (int i = 0; i < kCPT; ++i) {
    const int64_t ch = ((int64_t)seg * kCPT + i) * kThreads + threadIdx.x;
    const bool valid = ch < chunks;  // equal for both lanes of a pair (chunks is even)
    Vec8 v;
    if (valid) {
      v = load8<kBF16>(xrow + ch * 8 * es);
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e) v.v[e] = 0.0f;
    }
    uint32_t m = absmax_bits8(v);
    m = max(m, (uint32_t)__shfl_xor((int)m, 1));
    const BlockScale b = block_scale(u2f(m), S);
    const uint32_t word = pack8<kSR>(v, b, (uint64_t)row * cols + ch * 8, seed, subseq);
    if (valid) {
      reinterpret_cast<uint32_t*>(codes + row * (cols / 2))[ch] = word;
      if ((threadIdx.x & 1) == 0) {
        scales[row * (cols / 16) + (ch >> 1)] = (uint8_t)b.code;
        nzero += b.flags & 1u;
        nsat += b.flags >> 1;
      }
    }
  }
  if (diag) add_diag(diag, nzero, nsat);
}

// ------------------------------------------------------------------ COL16
// A lane holds 16 rows x 8 consecutive columns: eight complete column blocks.
// Grid: x over groups of kThreads column-octets, y over 16-row block rows.
template <bool kBF16, bool kSR>
__global__ __launch_bounds__(kThreads) void quant_col16_kernel(
    const uint8_t* __restrict__ x, int64_t rows, int64_t cols, int64_t ld_bytes,
    const float* __restrict__ amax_held, float target, uint64_t seed, uint32_t subseq,
    uint8_t* __restrict__ codes, uint8_t* __restrict__ scales, float* __restrict__ enc_out,
    int32_t* __restrict__ diag) {
  constexpr int es = kBF16 ? 2 : 4;
  const int64_t oct = (int64_t)blockIdx.x * kThreads + threadIdx.x;  // column octet
  const int64_t rb = blockIdx.y;                                       // 16-row block
  const float S = tensor_scale(*amax_held, target);
  if (enc_out && blockIdx.x == 0 && blockIdx.y == 0 && threadIdx.x == 0) *enc_out = S;
  uint32_t nzero = 0, nsat = 0;
  if (oct * 8 < cols) {
    const int64_t c0 = oct * 8;
    Vec8 v[16];
#pragma unroll
    for (int r = 0; r < 16; ++r) v[r] = load8<kBF16>(x + (rb * 16 + r) * ld_bytes + c0 * es);
    uint32_t lo[8], hi[8];
    BlockScale bs[8];
#pragma unroll
    for (int c = 0; c < 8; ++c) {
      uint32_t m = 0u;
#pragma unroll
      for (int r = 0; r < 16; ++r) m = max(m, f2u(v[r].v[c]) & 0x7FFFFFFFu);
      bs[c] = block_scale(u2f(m), S);
      nzero += bs[c].flags & 1u;
      nsat += bs[c].flags >> 1;
      lo[c] = 0u;
      hi[c] = 0u;
    }
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      uint32_t w[8] = {0, 0, 0, 0, 0, 0, 0, 0};
      if (kSR) {
        const uint64_t idx0 = (uint64_t)(rb * 16 + r) * cols + c0;
        const U4 r0 = sr_words(idx0 >> 2, subseq, seed);
        const U4 r1 = sr_words((idx0 >> 2) + 1, subseq, seed);
        w[0] = r0.x; w[1] = r0.y; w[2] = r0.z; w[3] = r0.w;
        w[4] = r1.x; w[5] = r1.y; w[6] = r1.z; w[7] = r1.w;
      }
#pragma unroll
      for (int c = 0; c < 8; ++c) {
        const uint32_t q = payload_code<kSR>(v[r].v[c], bs[c], w[c]);
        if (r < 8)
          lo[c] |= q << (4 * r);
        else
          hi[c] |= q << (4 * (r - 8));
      }
    }
#pragma unroll
    for (int c = 0; c < 8; ++c) {
      uint8_t* dst = codes + (c0 + c) * (rows / 2) + rb * 8;
      *reinterpret_cast<uint2*>(dst) = make_uint2(lo[c], hi[c]);
      scales[(c0 + c) * (rows / 16) + rb] = (uint8_t)bs[c].code;
    }
  }
  if (diag) add_diag(diag, nzero, nsat);
}

// ------------------------------------------------------------------ TILE16
// A lane holds 16 rows x 8 columns, a lane pair one 16 x 16 tile.
template <bool kBF16, bool kSR>
__global__ __launch_bounds__(kThreads) void quant_tile_kernel(
    const uint8_t* __restrict__ x, int64_t rows, int64_t cols, int64_t ld_bytes,
    const float* __restrict__ amax_held, float target, uint64_t seed, uint32_t subseq,
    uint8_t* __restrict__ codes, uint8_t* __restrict__ scales, uint8_t* __restrict__ codes_t,
    uint8_t* __restrict__ scales_t, float* __restrict__ enc_out, int32_t* __restrict__ diag) {
  constexpr int es = kBF16 ? 2 : 4;
  const int64_t oct = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  const int64_t rb = blockIdx.y;
  const float S = tensor_scale(*amax_held, target);
  if (enc_out && blockIdx.x == 0 && blockIdx.y == 0 && threadIdx.x == 0) *enc_out = S;
  uint32_t nzero = 0, nsat = 0;
  const bool valid = oct * 8 < cols;  // equal for both lanes of a pair (cols % 16 == 0)
  const int64_t c0 = oct * 8;
  Vec8 v[16];
  uint32_t m = 0u;
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    if (valid) {
      v[r] = load8<kBF16>(x + (rb * 16 + r) * ld_bytes + c0 * es);
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e) v[r].v[e] = 0.0f;
    }
    m = max(m, absmax_bits8(v[r]));
  }
  m = max(m, (uint32_t)__shfl_xor((int)m, 1));
  const BlockScale b = block_scale(u2f(m), S);
  uint32_t tlo[8] = {0, 0, 0, 0, 0, 0, 0, 0}, thi[8] = {0, 0, 0, 0, 0, 0, 0, 0};
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    uint32_t w[8] = {0, 0, 0, 0, 0, 0, 0, 0};
    if (kSR) {
      const uint64_t idx0 = (uint64_t)(rb * 16 + r) * cols + c0;
      const U4 r0 = sr_words(idx0 >> 2, subseq, seed);
      const U4 r1 = sr_words((idx0 >> 2) + 1, subseq, seed);
      w[0] = r0.x; w[1] = r0.y; w[2] = r0.z; w[3] = r0.w;
      w[4] = r1.x; w[5] = r1.y; w[6] = r1.z; w[7] = r1.w;
    }
    uint32_t word = 0u;
#pragma unroll
    for (int c = 0; c < 8; ++c) {
      const uint32_t q = payload_code<kSR>(v[r].v[c], b, w[c]);
      word |= q << (4 * c);
      if (r < 8)
        tlo[c] |= q << (4 * r);
      else
        thi[c] |= q << (4 * (r - 8));
    }
    if (valid) reinterpret_cast<uint32_t*>(codes + (rb * 16 + r) * (cols / 2))[oct] = word;
  }
  if (valid) {
    if ((threadIdx.x & 1) == 0) {
      scales[rb * (cols / 16) + (oct >> 1)] = (uint8_t)b.code;
      if (scales_t) scales_t[(oct >> 1) * (rows / 16) + rb] = (uint8_t)b.code;
      nzero += b.flags & 1u;
      nsat += b.flags >> 1;
    }
    if (codes_t) {
#pragma unroll
      for (int c = 0; c < 8; ++c)
        *reinterpret_cast<uint2*>(codes_t + (c0 + c) * (rows / 2) + rb * 8) = make_uint2(tlo[c], thi[c]);
    }
  }
  if (diag) add_diag(diag, nzero, nsat);
}

template <bool kBF16, bool kSR>
hipError_t launch_typed(const QuantArgs& a, hipStream_t s) {
  const uint8_t* x = static_cast<const uint8_t*>(a.x);
  const int64_t ldb = a.ld * a.es;
  if (a.layout == 0) {
    const int64_t chunks = a.cols / 8;
    // chunks-per-thread: the largest of 4, 2, 1 that tiles a row exactly
    int cpt = 1;
    if (chunks % (4 * kThreads) == 0) cpt = 4;
    else if (chunks % (2 * kThreads) == 0) cpt = 2;
    const int64_t seg = (int64_t)cpt * kThreads;
    const int segs = (int)((chunks + seg - 1) / seg);
    const dim3 grid((uint32_t)(a.rows * segs));
#define FP4Q_ROW(CPT)                                                                              \
  hipLaunchKernelGGL((quant_row16_kernel<kBF16, kSR, CPT>), grid, dim3(kThreads), 0, s, x, a.rows, \
                     a.cols, ldb, segs, a.amax_held, a.target, a.seed, a.subseq, a.codes,          \
                     a.scales, a.enc_scale_out, a.diag)
    if (cpt == 4) FP4Q_ROW(4);
    else if (cpt == 2) FP4Q_ROW(2);
    else FP4Q_ROW(1);
#undef FP4Q_ROW
  } else {
    const int64_t octs = a.cols / 8;
    const dim3 grid((uint32_t)((octs + kThreads - 1) / kThreads), (uint32_t)(a.rows / 16));
    if (a.layout == 1)
      hipLaunchKernelGGL((quant_col16_kernel<kBF16, kSR>), grid, dim3(kThreads), 0, s, x, a.rows,
                         a.cols, ldb, a.amax_held, a.target, a.seed, a.subseq, a.codes, a.scales,
                         a.enc_scale_out, a.diag);
    else
      hipLaunchKernelGGL((quant_tile_kernel<kBF16, kSR>), grid, dim3(kThreads), 0, s, x, a.rows,
                         a.cols, ldb, a.amax_held, a.target, a.seed, a.subseq, a.codes, a.scales,
                         a.codes_t, a.scales_t, a.enc_scale_out, a.diag);
  }
  return hipGetLastError();
}

// Writes the tensor scale when there is no block to carry it (empty tensor).
__global__ void write_scale_only(const float* amax_held, float target, float* enc_out) {
  *enc_out = tensor_scale(*amax_held, target);
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
