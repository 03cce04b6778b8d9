// Emulated FP4 GEMM: Y[M, N] = (A[M, K] . B[N, K]^T) / (Sa Sb) over the
// decoded operands ("UE5M3 FP4 Block Scaling for Stable Language Model
// Pretraining", §6: the contraction of decoded operands, with the encoded
// tensor-scale product applied after accumulation).
//
// Each decoded element e2m1 * dec has at most 6 significant bits and lies in
// [2^-18, 368640], so it is exact in bf16; the contraction runs on bf16 MFMA
// (v_mfma_f32_32x32x16_bf16) with fp32 accumulation. FP4 codes and scales
// are read from HBM (4.5 bits per element), decoded once per workgroup into
// LDS as bf16, and consumed from LDS by the MFMA fragments.
//
// One kernel serves fwd (A = X, ROW16; B = W, TILE), dgrad (A = dY, ROW16;
// B = W^T, TILE) and wgrad (A = dY^T, B = X^T, both quantized along tokens):
// both operands are stored contiguous along the contraction.
#include "codec.h"
#include "kernels.h"

namespace fp4q {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int BM = 128;
constexpr int BN = 128;
constexpr int BK = 64;
constexpr int kThreads = 256;

// Decode 8 packed codes of one block into 8 bf16 (exact), element order kept.
// A half with bit pattern m << 9 equals e2m1(m) * 2^-14 for every magnitude
// m (E2M1's subnormal 0.5 lines up with the half subnormals), so
// e2m1 * dec = half(m << 9) * (dec * 2^14), one exact fp32 product.
__device__ __forceinline__ uint4 decode8(uint32_t d, float dec14) {
  uint32_t h[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const uint32_t q = (d >> (4 * e)) & 0xFu;
    const float f = half_bits_to_float((q & 7u) << 9) * dec14;
    h[e] = (f2u(f) >> 16) | ((q & 8u) << 12);
  }
  return make_uint4(h[0] | (h[1] << 16), h[2] | (h[3] << 16), h[4] | (h[5] << 16), h[6] | (h[7] << 16));
}

struct Stage {
  uint2 c[2];      // codes of two 16-element blocks (8 bytes each)
  uint32_t s[2];   // their scale codes
};

// Loader: thread t owns row (t >> 1) of the 128-row tile and k range
// 32 * (t & 1) .. +31 of the 64-wide k tile: two blocks of 16.
__device__ __forceinline__ Stage load_stage(const uint8_t* __restrict__ codes,
                                            const uint8_t* __restrict__ scales, int64_t rows,
                                            int64_t K, int tile_shift, int64_t r, int64_t k) {
  Stage st;
#pragma unroll
  for (int b = 0; b < 2; ++b) {
    const int64_t kb = k + 16 * b;
    if (r < rows && kb < K) {
      st.c[b] = *reinterpret_cast<const uint2*>(codes + r * (K / 2) + kb / 2);
      st.s[b] = scales[(r >> tile_shift) * (K / 16) + kb / 16];
    } else {
      st.c[b] = make_uint2(0u, 0u);
      st.s[b] = 0u;
    }
  }
  return st;
}

__device__ __forceinline__ void store_stage(uint4* lds, const Stage& st, int row, int half) {
#pragma unroll
  for (int b = 0; b < 2; ++b) {
    const float dec14 = ue5m3_value(st.s[b]) * 16384.0f;
    const uint4 lo = decode8(st.c[b].x, dec14);
    const uint4 hi = decode8(st.c[b].y, dec14);
    const int c0 = half * 4 + 2 * b;  // 16-byte chunk index (8 k each) in the row
    lds[row * 8 + ((c0) ^ (row & 7))] = lo;
    lds[row * 8 + ((c0 + 1) ^ (row & 7))] = hi;
  }
}

__global__ __launch_bounds__(kThreads) void gemm_kernel(
    const uint8_t* __restrict__ a_codes, const uint8_t* __restrict__ a_scales, int a_shift,
    const float* __restrict__ a_S, const uint8_t* __restrict__ b_codes,
    const uint8_t* __restrict__ b_scales, int b_shift, const float* __restrict__ b_S, int64_t M,
    int64_t N, int64_t K, void* __restrict__ y, int y_es) {
  __shared__ uint4 As[BM * BK / 8];
  __shared__ uint4 Bs[BN * BK / 8];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wm = wave >> 1;
  const int wn = wave & 1;
  const int64_t m0 = (int64_t)blockIdx.y * BM;
  const int64_t n0 = (int64_t)blockIdx.x * BN;
  const int lrow = tid >> 1;
  const int lhalf = tid & 1;

  f32x16 acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.0f;

  Stage sa = load_stage(a_codes, a_scales, M, K, a_shift, m0 + lrow, 32 * lhalf);
  Stage sb = load_stage(b_codes, b_scales, N, K, b_shift, n0 + lrow, 32 * lhalf);
  for (int64_t k0 = 0; k0 < K; k0 += BK) {
    store_stage(As, sa, lrow, lhalf);
    store_stage(Bs, sb, lrow, lhalf);
    __syncthreads();
    if (k0 + BK < K) {
      sa = load_stage(a_codes, a_scales, M, K, a_shift, m0 + lrow, k0 + BK + 32 * lhalf);
      sb = load_stage(b_codes, b_scales, N, K, b_shift, n0 + lrow, k0 + BK + 32 * lhalf);
    }
#pragma unroll
    for (int s = 0; s < BK / 16; ++s) {
      bf16x8 af[2], bfr[2];
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        const int ar = wm * 64 + t * 32 + (lane & 31);
        const int br = wn * 64 + t * 32 + (lane & 31);
        const int ch = 2 * s + (lane >> 5);
        af[t] = __builtin_bit_cast(bf16x8, As[ar * 8 + (ch ^ (ar & 7))]);
        bfr[t] = __builtin_bit_cast(bf16x8, Bs[br * 8 + (ch ^ (br & 7))]);
      }
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[i], bfr[j], acc[i][j], 0, 0, 0);
    }
    __syncthreads();
  }

  const double alpha = 1.0 / ((double)*a_S * (double)*b_S);
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int64_t r = m0 + wm * 64 + i * 32 + 8 * (e >> 2) + 4 * (lane >> 5) + (e & 3);
        const int64_t c = n0 + wn * 64 + j * 32 + (lane & 31);
        if (r < M && c < N) {
          const float v = (float)((double)acc[i][j][e] * alpha);
          if (y_es == 4) {
            static_cast<float*>(y)[r * N + c] = v;
          } else {
            const uint32_t u = f2u(v);
            static_cast<uint16_t*>(y)[r * N + c] = (uint16_t)((u + 0x7FFFu + ((u >> 16) & 1u)) >> 16);
          }
        }
      }
}

}  // namespace

hipError_t launch_gemm(const QOperand& a, const QOperand& b, void* y, int y_es, hipStream_t s) {
  const int64_t M = a.rows, N = b.rows, K = a.cols;
  if (M == 0 || N == 0) return hipSuccess;
  const dim3 grid((uint32_t)((N + BN - 1) / BN), (uint32_t)((M + BM - 1) / BM));
  hipLaunchKernelGGL(gemm_kernel, grid, dim3(kThreads), 0, s, a.codes, a.scales, a.tile ? 4 : 0,
                     a.enc_scale, b.codes, b.scales, b.tile ? 4 : 0, b.enc_scale, M, N, K, y, y_es);
  return hipGetLastError();
}

}  // namespace fp4q
