// Dequantization of a stored quantized operand: x_hat = RN((e2m1 * dec) / S)
// ("UE5M3 FP4 Block Scaling for Stable Language Model Pretraining", §6: the
// emulated GEMM works on decoded operands and the tensor scale is removed
// after the product). The product e2m1 * dec is exact in fp32; one division
// rounds it; a bf16 output rounds that fp32 value once more (RNE).
#include "codec.h"
#include "kernels.h"

namespace fp4q {
namespace {

__device__ __forceinline__ float e2m1_value(uint32_t q) {
  // half with bit pattern (q & 7) << 9 equals e2m1(q) * 2^-14 for all eight
  // magnitudes (the E2M1 subnormal lines up with the half subnormals)
  const float m = half_bits_to_float((q & 7u) << 9) * 16384.0f;
  return (q & 8u) ? -m : m;
}

__device__ __forceinline__ uint32_t f32_to_bf16_rne(float f) {
  const uint32_t u = f2u(f);
  return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;  // inputs are finite
}

// One lane per 8 elements (one 32-bit word of codes).
__global__ __launch_bounds__(256) void dequant_kernel(const uint8_t* __restrict__ codes,
                                                      const uint8_t* __restrict__ scales,
                                                      const float* __restrict__ enc_scale,
                                                      int64_t rows, int64_t cols, int tile,
                                                      int block, int e4m3, int k64,
                                                      void* __restrict__ out, int out_es) {
  const int64_t words_per_row = cols / 8;
  const int64_t g = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (g >= rows * words_per_row) return;
  const int64_t r = g / words_per_row;
  const int64_t w = g - r * words_per_row;
  const uint32_t d = *reinterpret_cast<const uint32_t*>(codes + code_offset(r, 4 * w, rows, cols, k64));
  const int64_t srow = tile ? r / block : r;
  const int64_t nsrow = tile ? rows / block : rows;
  const int64_t j = (w * 8) / block;
  const int64_t si = block == 32 ? scale_offset<2>(srow, j, nsrow, cols / block, k64)
                                 : scale_offset<4>(srow, j, nsrow, cols / block, k64);
  const float dec = scale_value(scales[si], e4m3 != 0);
  const float S = *enc_scale;
  float v[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) v[e] = (e2m1_value((d >> (4 * e)) & 0xFu) * dec) / S;
  if (out_es == 4) {
    float4* o = reinterpret_cast<float4*>(static_cast<float*>(out) + r * cols + w * 8);
    o[0] = make_float4(v[0], v[1], v[2], v[3]);
    o[1] = make_float4(v[4], v[5], v[6], v[7]);
  } else {
    uint32_t p[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) p[i] = f32_to_bf16_rne(v[2 * i]) | (f32_to_bf16_rne(v[2 * i + 1]) << 16);
    *reinterpret_cast<uint4*>(static_cast<uint16_t*>(out) + r * cols + w * 8) = make_uint4(p[0], p[1], p[2], p[3]);
  }
}

}  // namespace

hipError_t launch_dequant(const QOperand& q, void* out, int out_es, hipStream_t s) {
  const int64_t n = q.rows * (q.cols / 8);
  if (n == 0) return hipSuccess;
  hipLaunchKernelGGL(dequant_kernel, dim3((uint32_t)((n + 255) / 256)), dim3(256), 0, s, q.codes,
                     q.scales, q.enc_scale, q.rows, q.cols, q.tile, q.block, q.scale_fmt, q.pack, out,
                     out_es);
  return hipGetLastError();
}

}  // namespace fp4q
