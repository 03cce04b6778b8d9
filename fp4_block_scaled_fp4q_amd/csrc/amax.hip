// Tensor amax ("UE5M3 FP4 Block Scaling for Stable Language Model
// Pretraining", §5.1: each operand's tensor maximum is sampled and held).
//
// HBM-bound: every byte is read once with 128-bit loads. The maximum is taken
// over sign-cleared bit patterns, which order like the magnitudes of finite
// values, so the result is exact and independent of the reduction order.
// bf16 pairs are reduced with packed 16-bit integer max; each workgroup
// reduces across its lanes and issues at most one 32-bit atomic max on the
// output word (non-negative floats order like their bit patterns).
#include "codec.h"
#include "kernels.h"

namespace fp4q {
namespace {

typedef unsigned short us2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ uint32_t pkmax16(uint32_t a, uint32_t b) {
  us2 va = __builtin_bit_cast(us2, a);
  us2 vb = __builtin_bit_cast(us2, b);
  return __builtin_bit_cast(uint32_t, __builtin_elementwise_max(va, vb));
}

__global__ void zero_word(uint32_t* p) { *p = 0u; }

template <bool kBF16>
__device__ __forceinline__ uint32_t fold(uint32_t acc, const uint4 v) {
  const uint32_t mask = kBF16 ? 0x7FFF7FFFu : 0x7FFFFFFFu;
  const uint32_t w0 = v.x & mask, w1 = v.y & mask, w2 = v.z & mask, w3 = v.w & mask;
  if (kBF16) return pkmax16(acc, pkmax16(pkmax16(w0, w1), pkmax16(w2, w3)));
  return max(acc, max(max(w0, w1), max(w2, w3)));
}

// Maximum over the 64 lanes of a wave, valid in lane 0: DPP steps inside
// each row of 16 lanes (swap neighbours, swap pairs, mirror each half row,
// mirror the row), a ds_swizzle exchange between the two rows of each
// 32-lane half (xor 16), then the two halves' lanes 0 and 32.
template <int kCtrl>
__device__ __forceinline__ uint32_t dpp(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, kCtrl, 0xF, 0xF, false);
}

__device__ __forceinline__ uint32_t wave_max_lane0(uint32_t m) {
  m = max(m, dpp<0xB1>(m));   // quad_perm [1, 0, 3, 2]
  m = max(m, dpp<0x4E>(m));   // quad_perm [2, 3, 0, 1]
  m = max(m, dpp<0x141>(m));  // row_half_mirror
  m = max(m, dpp<0x140>(m));  // row_mirror
  m = max(m, (uint32_t)__builtin_amdgcn_ds_swizzle((int)m, 0x401F));  // and 0x1F, xor 0x10
  return max((uint32_t)__builtin_amdgcn_readlane((int)m, 0), (uint32_t)__builtin_amdgcn_readlane((int)m, 32));
}

// Workgroup-wide maximum, then at most one atomic per workgroup, skipped
// when the output already holds a value at least as large (atomics on one
// address serialize, so their number is kept to a few hundred).
template <bool kBF16>
__device__ __forceinline__ void finish(uint32_t acc, uint32_t* out) {
  __shared__ uint32_t wmax[4];
  uint32_t m = kBF16 ? (max(acc & 0xFFFFu, acc >> 16) << 16) : acc;
  m = wave_max_lane0(m);
  if ((threadIdx.x & 63) == 0) wmax[threadIdx.x >> 6] = m;
  __syncthreads();
  if (threadIdx.x == 0) {
    m = max(max(wmax[0], wmax[1]), max(wmax[2], wmax[3]));
    if (m > __hip_atomic_load(out, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)) atomicMax(out, m);
  }
}

// Contiguous tensor (ld == cols): a flat grid-stride walk over 16-byte
// chunks, four chunks in flight per lane.
template <bool kBF16>
__global__ __launch_bounds__(256) void amax_flat_kernel(const uint4* __restrict__ x, int64_t nchunks,
                                                        uint32_t* __restrict__ out) {
  uint32_t acc = 0u;
  const int64_t stride = (int64_t)gridDim.x * 256;
  int64_t c = (int64_t)blockIdx.x * 256 + threadIdx.x;
  for (; c + 3 * stride < nchunks; c += 4 * stride) {
    uint4 v[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) v[u] = load_nt16(x + c + u * stride);
#pragma unroll
    for (int u = 0; u < 4; ++u) acc = fold<kBF16>(acc, v[u]);
  }
  for (; c < nchunks; c += stride) acc = fold<kBF16>(acc, load_nt16(x + c));
  finish<kBF16>(acc, out);
}

// Strided rows: one workgroup per row range, lanes stride over the chunks
// of each row.
template <bool kBF16>
__global__ __launch_bounds__(256) void amax_rows_kernel(const uint8_t* __restrict__ x, int64_t rows,
                                                        int64_t chunks_per_row, int64_t ld_bytes,
                                                        int64_t rows_per_wg, uint32_t* __restrict__ out) {
  const int64_t r0 = (int64_t)blockIdx.x * rows_per_wg;
  const int64_t r1 = r0 + rows_per_wg < rows ? r0 + rows_per_wg : rows;
  uint32_t acc = 0u;
  for (int64_t r = r0; r < r1; ++r) {
    const uint4* row = reinterpret_cast<const uint4*>(x + r * ld_bytes);
    for (int64_t c = threadIdx.x; c < chunks_per_row; c += 256)
      acc = fold<kBF16>(acc, load_nt16(row + c));
  }
  finish<kBF16>(acc, out);
}

}  // namespace

hipError_t launch_amax(const void* x, int es, int64_t rows, int64_t cols, int64_t ld, float* out,
                       hipStream_t s) {
  uint32_t* o = reinterpret_cast<uint32_t*>(out);
  hipLaunchKernelGGL(zero_word, dim3(1), dim3(1), 0, s, o);
  if (rows == 0 || cols == 0) return hipGetLastError();
  const int64_t chunks_per_row = cols * es / 16;
  if (ld == cols) {
    const int64_t nchunks = rows * chunks_per_row;
    int64_t wgs = (nchunks + 4 * 256 - 1) / (4 * 256);
    if (wgs > 1024) wgs = 1024;
    if (es == 2)
      hipLaunchKernelGGL(amax_flat_kernel<true>, dim3((uint32_t)wgs), dim3(256), 0, s,
                         (const uint4*)x, nchunks, o);
    else
      hipLaunchKernelGGL(amax_flat_kernel<false>, dim3((uint32_t)wgs), dim3(256), 0, s,
                         (const uint4*)x, nchunks, o);
    return hipGetLastError();
  }
  const int64_t target_wgs = 1024;
  int64_t rows_per_wg = (rows + target_wgs - 1) / target_wgs;
  const int64_t wgs = (rows + rows_per_wg - 1) / rows_per_wg;
  if (es == 2)
    hipLaunchKernelGGL(amax_rows_kernel<true>, dim3((uint32_t)wgs), dim3(256), 0, s,
                       (const uint8_t*)x, rows, chunks_per_row, ld * es, rows_per_wg, o);
  else
    hipLaunchKernelGGL(amax_rows_kernel<false>, dim3((uint32_t)wgs), dim3(256), 0, s,
                       (const uint8_t*)x, rows, chunks_per_row, ld * es, rows_per_wg, o);
  return hipGetLastError();
}

}  // namespace fp4q
