// Device-side codec for the block-scaled FP4 format of "UE5M3 FP4 Block
// Scaling for Stable Language Model Pretraining": E2M1 payloads (§3), UE5M3
// block scales (§4.1), an FP32 tensor scale with tunable target T (§5.2),
// repair of zero-rounded and saturated scale codes (§5.3), RNE (§2) and
// stochastic rounding (§5.2) of payloads, Philox4x32-10 words (named in
// "Gaussian Weight Sampling ...", §3.4).
//
// Every rounding here is done with integer arithmetic on IEEE bit patterns or
// with single correctly rounded binary32 operations, so results are
// bit-identical to any other correct implementation of the same rules. All
// HIP sources are compiled with -ffp-contract=off, correctly rounded fp32
// division and fp32 denormals kept.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fp4q {

constexpr float kFltMax = 3.40282346638528859812e+38f;

__device__ __forceinline__ uint32_t f2u(float f) { return __float_as_uint(f); }
__device__ __forceinline__ float u2f(uint32_t u) { return __uint_as_float(u); }

// FP32 tensor (encode) scale S = RN(RN(6 T) / A) from the held amax A; 1 when
// A is zero or not finite; the largest finite binary32 when the quotient
// overflows.
__device__ __forceinline__ float tensor_scale(float amax, float target) {
  if (!(amax > 0.0f) || __builtin_isinf(amax)) return 1.0f;
  float six_t = 6.0f * target;
  float s = six_t / amax;
  if (__builtin_isinf(s)) s = kFltMax;
  return s;
}

// UE5M3: 5 exponent bits (bias 15) and 3 fraction bits; exponent field 31 is
// not finite, so the largest finite code is 0xF7 (61,440). The code c has the
// same value as the IEEE half whose bit pattern is c << 7.
__device__ __forceinline__ float half_bits_to_float(uint32_t bits16) {
  return (float)__builtin_bit_cast(_Float16, (unsigned short)bits16);
}

__device__ __forceinline__ float ue5m3_value(uint32_t code) { return half_bits_to_float(code << 7); }

// 16-byte streaming load (read once, do not keep in cache).
typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));
__device__ __forceinline__ uint4 load_nt16(const void* p) {
  const u32x4_t v = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(p));
  return make_uint4(v.x, v.y, v.z, v.w);
}

// Nearest UE5M3 code of raw >= 0 with ties to the even code, then repair:
// a code that rounds to 0 becomes 0x01, one that rounds beyond 61,440
// (raw >= 63,488, the midpoint to 2^16, tie to the even side) becomes 0xF7.
// flags: bit 0 zero-rounded, bit 1 saturated (both before repair).
__device__ __forceinline__ uint32_t ue5m3_encode(float raw, uint32_t* flags) {
  const uint32_t u = f2u(raw);
  if (u >= 0x47780000u) {  // raw >= 63488.0f, or +Inf
    *flags = 2u;
    return 0xF7u;
  }
  const uint32_t e32 = u >> 23;
  uint32_t code;
  if (e32 >= 113u) {
    // normal range of UE5M3 (>= 2^-14): keep 3 fraction bits, RNE on 20
    const uint32_t m = u & 0x7FFFFFu;
    const uint32_t base = ((e32 - 112u) << 3) | (m >> 20);
    const uint32_t rem = m & 0xFFFFFu;
    const uint32_t up = (rem > 0x80000u) | ((rem == 0x80000u) & (base & 1u));
    code = base + up;  // a carry moves into the exponent field
  } else if (e32 == 0u) {
    code = 0u;  // +0 or an fp32 denormal (< 2^-126)
  } else {
    // subnormal range: code = RN(raw * 2^17), value = code * 2^-17
    const uint32_t sig = (u & 0x7FFFFFu) | 0x800000u;
    const uint32_t sh = 133u - e32;  // >= 21
    if (sh >= 25u) {
      code = 0u;  // raw < 2^-18, strictly below the half-way point
    } else {
      const uint32_t base = sig >> sh;
      const uint32_t rem = sig & ((1u << sh) - 1u);
      const uint32_t half = 1u << (sh - 1u);
      const uint32_t up = (rem > half) | ((rem == half) & (base & 1u));
      code = base + up;
    }
  }
  if (code == 0u) {
    *flags = 1u;
    return 1u;
  }
  *flags = 0u;
  return code;
}

// Per-block quantities shared by every element of a block.
struct BlockScale {
  uint32_t code;   // UE5M3 code written to the scale array
  float mul;       // r = RN(S / dec); multiplies each element
  uint32_t flags;  // repair flags
  bool zero;       // bamax == 0: scale 0, sign-only payloads
  bool mul_inf;    // r overflowed: payload is 6 for x != 0, 0 for x == 0
};

__device__ __forceinline__ BlockScale block_scale(float bamax, float S) {
  BlockScale b;
  if (!(bamax > 0.0f)) {
    b.code = 0u;
    b.mul = 0.0f;
    b.flags = 0u;
    b.zero = true;
    b.mul_inf = false;
    return b;
  }
  const float d6 = bamax / 6.0f;
  const float raw = d6 * S;
  b.code = ue5m3_encode(raw, &b.flags);
  const float dec = ue5m3_value(b.code);
  b.mul = S / dec;
  b.zero = false;
  b.mul_inf = __builtin_isinf(b.mul);
  return b;
}

// E2M1 magnitude code (0..7) of |v| by round to nearest, ties to the even
// code, saturating at 6 (code 7). The magic-constant addition rounds |v| to
// the E2M1 spacing of its binade (0.5 below 2, 1 in [2, 4), 2 from 4) with
// the hardware's own RNE; the low bits of the sum are then the code offset
// inside that binade. |v| is clamped to 8 first so that huge values and Inf
// stay in range (8 rounds to code 8, clamped to 7). NaN cannot reach here.
__device__ __forceinline__ uint32_t e2m1_rne_mag(float v) {
  const float a = __builtin_fminf(__builtin_fabsf(v), 8.0f);
  const bool ge2 = a >= 2.0f;
  const bool ge4 = a >= 4.0f;
  const float magic = ge4 ? 16777216.0f : (ge2 ? 8388608.0f : 4194304.0f);
  const uint32_t off = ge4 ? 4u : (ge2 ? 2u : 0u);
  const float t = a + magic;
  const uint32_t q = (f2u(t) & 0xFu) + off;
  return q < 7u ? q : 7u;
}

// Stochastic rounding between the adjacent E2M1 magnitudes lo <= |v| < hi:
// rounds up iff w < ceil(p * 2^32) with p = (|v| - lo) / (hi - lo), computed
// in binary32 (exact: Sterbenz for the difference, a power-of-two gap).
// |v| >= 6 gives 6. NaN cannot reach here.
__device__ __forceinline__ uint32_t e2m1_sr_mag(float v, uint32_t w) {
  const float a = __builtin_fabsf(v);
  if (a >= 6.0f) return 7u;
  // lower neighbour index q and its value / gap
  uint32_t q;
  float lo, inv_gap;
  if (a < 2.0f) {
    q = (uint32_t)(a * 2.0f);  // floor: exact for a < 2
    lo = (float)q * 0.5f;
    inv_gap = 2.0f;
  } else if (a < 4.0f) {
    const uint32_t k = (uint32_t)a;  // 2 or 3
    q = k + 2u;
    lo = (float)k;
    inv_gap = 1.0f;
  } else {
    q = 6u;
    lo = 4.0f;
    inv_gap = 0.5f;
  }
  const float p = (a - lo) * inv_gap;  // exact
  const float thr = __builtin_ceilf(p * 4294967296.0f);
  // thr <= 2^32 - 256 fits in uint32 after the cast for p < 1
  const uint32_t t = (uint32_t)thr;
  return q + (w < t ? 1u : 0u);
}

// ---------------------------------------------------------------- Philox
// Philox4x32-10 (Salmon et al., SC'11): ten rounds of two 32x32->64 products
// mixed into the other words and the key; the key advances by two Weyl
// constants per round.
struct U4 {
  uint32_t x, y, z, w;
};

__device__ __forceinline__ U4 philox4x32_10(U4 c, uint32_t k0, uint32_t k1) {
#pragma unroll
  for (int i = 0; i < 10; ++i) {
    const uint64_t p0 = (uint64_t)0xD2511F53u * c.x;
    const uint64_t p1 = (uint64_t)0xCD9E8D57u * c.z;
    const uint32_t hi0 = (uint32_t)(p0 >> 32), lo0 = (uint32_t)p0;
    const uint32_t hi1 = (uint32_t)(p1 >> 32), lo1 = (uint32_t)p1;
    U4 n;
    n.x = hi1 ^ c.y ^ k0;
    n.y = lo1;
    n.z = hi0 ^ c.w ^ k1;
    n.w = lo0;
    c = n;
    k0 += 0x9E3779B9u;
    k1 += 0xBB67AE85u;
  }
  return c;
}

// The four words for source elements 4j .. 4j+3 (row-major linear index of
// the logical tensor): counter (j lo, j hi, subseq, 0), key = the 64-bit seed.
__device__ __forceinline__ U4 sr_words(uint64_t j, uint32_t subseq, uint64_t seed) {
  U4 c;
  c.x = (uint32_t)j;
  c.y = (uint32_t)(j >> 32);
  c.z = subseq;
  c.w = 0u;
  return philox4x32_10(c, (uint32_t)seed, (uint32_t)(seed >> 32));
}

// Payload code (sign | magnitude) for one element, RNE or SR.
template <bool kSR>
__device__ __forceinline__ uint32_t payload_code(float x, const BlockScale& b, uint32_t w) {
  const uint32_t sign = (f2u(x) >> 28) & 8u;
  if (b.zero) return sign;
  if (b.mul_inf) return sign | (x != 0.0f ? 7u : 0u);
  const float v = x * b.mul;
  const uint32_t mag = kSR ? e2m1_sr_mag(v, w) : e2m1_rne_mag(v);
  return sign | mag;
}

// bf16 -> fp32 widening of a packed pair.
__device__ __forceinline__ float bf16_lo(uint32_t d) { return u2f(d << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t d) { return u2f(d & 0xFFFF0000u); }

}  // namespace fp4q
