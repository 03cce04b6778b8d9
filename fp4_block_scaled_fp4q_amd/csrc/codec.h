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

// 16-byte loads. The quantize kernels use plain loads; the amax reduction
// (a pure read stream) measured faster with the nontemporal form.
__device__ __forceinline__ uint4 load16(const void* p) { return *reinterpret_cast<const uint4*>(p); }
typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));
__device__ __forceinline__ uint4 load_nt16(const void* p) {
  const u32x4_t v = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(p));
  return make_uint4(v.x, v.y, v.z, v.w);
}

// Workgroup barrier for data exchanged through LDS: waits for this wave's
// LDS (and scalar memory) operations only, then s_barrier. __syncthreads()
// also waits for every global load and store still in flight (prefetches
// for later work, output stores), which these kernels never need to order
// against another wave. The memory clobber keeps the compiler from moving
// memory operations across it.
__device__ __forceinline__ void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

// Nearest UE5M3 code of raw >= 0 with ties to the even code, then repair:
// a code that rounds to 0 becomes 0x01, one that rounds beyond 61,440
// (raw >= 63,488, the midpoint to 2^16, tie to the even side) becomes 0xF7.
// flags: bit 0 zero-rounded, bit 1 saturated (both before repair).
//  * raw >= 2^-14 (normal UE5M3): the code is the binary32 pattern rounded
//    to 3 fraction bits (RNE by adding 0x7FFFF plus the kept lsb, a carry
//    moving into the exponent), shifted down and rebased from bias 127 to 15.
//  * raw < 2^-14 (subnormal UE5M3, code = RN(raw * 2^17) in 0..8): the
//    exact product raw * 2^17 < 8 is rounded to an integer by adding 2^23.
__device__ __forceinline__ uint32_t ue5m3_encode(float raw, uint32_t* flags) {
  const uint32_t u = f2u(raw);
  const uint32_t normal = ((u + 0x7FFFFu + ((u >> 20) & 1u)) >> 20) - (112u << 3);
  const uint32_t sub = f2u(raw * 131072.0f + 8388608.0f) - 0x4B000000u;
  uint32_t code = u >= 0x38800000u ? normal : sub;  // 2^-14
  const bool sat = u >= 0x47780000u;                 // raw >= 63488 (or +Inf)
  const bool zero = code == 0u;
  *flags = (zero ? 1u : 0u) | (sat ? 2u : 0u);
  code = zero ? 1u : code;
  return sat ? 0xF7u : code;
}

// RN(a / 6) for finite a >= 0, computed as RN32(RN64(a * RN64(1/6))). This
// equals the correctly rounded binary32 quotient: the exact quotient of a
// 24-bit significand by 3 stays at least 2^-26 (relative) away from every
// binary32 rounding midpoint, far more than the < 2^-52 error of the double
// product.
__device__ __forceinline__ float div6_rn(float a) { return (float)((double)a * (1.0 / 6.0)); }

// RN(s / d) for s > 0 and d a positive UE5M3 or E4M3 value, as RN32(s * 1/d) in
// double with a Newton-refined reciprocal. d = (8 + m) 2^k with an odd part
// of 8 + m in {1, 3, 5, ..., 15}: the quotient is either exact or at least
// 2^-29 (relative) away from every binary32 midpoint, again far more than
// the double error.
__device__ __forceinline__ float div_rn(double s, float d) {
  const double dd = (double)d;
  double y = __builtin_amdgcn_rcp(dd);
  y = __builtin_fma(y, __builtin_fma(-dd, y, 1.0), y);
  return (float)(s * y);
}

// E4M3 block scale (NVFP4's format; codes 0x00..0x7E, 448 the largest, 2^-9
// the smallest subnormal): its codebook is the UE5M3 codebook times 2^8, cut
// at 448. So the nearest E4M3 code of raw is the nearest UE5M3 code of
// raw * 2^-8 (an exact scaling wherever the result can be non-zero), with
// saturation once raw > 464 (the midpoint to the next point, 480; 464 itself
// ties to the even code 0x7E); zero-rounding repairs to 0x01 as for UE5M3.
__device__ __forceinline__ uint32_t e4m3_encode(float raw, uint32_t* flags) {
  const float q = raw * 0.00390625f;
  uint32_t f;
  const uint32_t code = ue5m3_encode(q, &f);
  const bool sat = f2u(q) > 0x3FE80000u;  // q > 1.8125, i.e. raw > 464
  *flags = (f & 1u) | (sat ? 2u : 0u);
  return sat ? 0x7Eu : code;
}

// Value of a scale code: UE5M3, or E4M3 (UE5M3 value times 256).
__device__ __forceinline__ float scale_value(uint32_t code, bool e4m3) {
  return ue5m3_value(code) * (e4m3 ? 256.0f : 1.0f);
}

// Per-block quantities shared by every element of a block.
struct BlockScale {
  uint32_t code;  // scale code written to the scale array (0 for an all-zero block)
  float mul;      // r = RN(S / dec); 0 for an all-zero block, so x * r keeps only the sign
  uint32_t flags; // repair flags
};

// bamax is the block's max |x| as a sign-cleared bit pattern; e4m3 selects
// the scale format (uniform across a launch).
__device__ __forceinline__ BlockScale block_scale(uint32_t bamax, float S, double S_d, bool e4m3) {
  const float d6 = div6_rn(u2f(bamax));
  const float raw = d6 * S;
  uint32_t flags;
  const uint32_t code = e4m3 ? e4m3_encode(raw, &flags) : ue5m3_encode(raw, &flags);
  const float mul = div_rn(S_d, scale_value(code, e4m3));
  BlockScale b;
  const bool nz = bamax != 0u;
  b.code = nz ? code : 0u;
  b.flags = nz ? flags : 0u;
  b.mul = nz ? mul : 0.0f;
  return b;
}

// RNE payload codes of two values packed in byte `sel` of `word`: the gfx950
// conversion v_cvt_scalef32_pk_fp4_f32 with scale 1.0 rounds to nearest,
// ties to the even code, saturates at 6 and keeps the sign of zero; this was
// checked against the reference rule for every bf16 input and is covered by
// the parity tests for fp32 inputs.
#define FP4Q_ENC2(word, a, b, sel) __builtin_amdgcn_cvt_scalef32_pk_fp4_f32((word), (a), (b), 1.0f, (sel))

// Stochastic rounding to E2M1 (sign | magnitude): |v| rounds up to the
// next magnitude iff the element's 32-bit word w is below ceil(p 2^32), p
// the position of |v| between its neighbours lo <= |v| < hi (spacing
// s = hi - lo, 1/2 below 2, 1 below 4, 2 above). The decision is made
// exactly in binary32 and the code is produced by a hardware conversion:
//  1. w < ceil(P) iff w < P for integer w and real P = p 2^32; P is a
//     binary32 value (p = (|v| - lo) / s is), so w < P iff RZ(w) < P, i.e.
//     q < p / 2 with q = RZ(w) 2^-33 (exact scaling; p / 2 is exact too).
//  2. q < p / 2 iff q' <= p / 2, where q' is the binary32 successor of q
//     (bit pattern plus one; no binary32 value lies strictly between), i.e.
//     iff A = |v| - q' s2 >= lo, with s2 = 2 s (the binade base of |v|,
//     at least 1) and q' <= 1/2, so q' s2 <= s.
//  3. z = RZ(RZ(A) + s) lies in [hi, hi + s) when A >= lo and in [lo, hi)
//     otherwise (lo, hi and lo - s are binary32 values, the rounding is
//     toward zero, and the spacing above hi is at least s), so rounding z
//     toward zero onto the E2M1 grid gives hi or lo as required. |v| >= 6
//     (lo = 6) gives z >= 6, which the conversion saturates to 6; s2 is
//     clamped to [1, 4] (its value for |v| in [4, 8)), so that |v| = Inf (a
//     finite x times a finite multiplier can overflow) gives z = Inf, not
//     Inf - Inf.
//  4. Toward zero onto the grid is the gfx950 stochastic conversion
//     v_cvt_scalef32_sr_pk_fp4_f32 with random operand 0 (it adds the
//     random bits below the kept ones before truncating), checked against
//     floor-to-grid on every binade down to the subnormals; it keeps the
//     sign, which z gets from v (rounding toward zero is symmetric).
// Per element: one median and one mask for s2, two fused multiply-adds under
// the MODE register's toward-zero rounding, one bit insert for the sign
// and half a conversion.

// q' of step 2 for eight Philox words: f[j] = succ(RZ(w[j]) 2^-33). The
// conversions run with the MODE register's single-precision rounding field
// set to toward zero, inside one asm block (nothing else can be scheduled
// into it; the field is restored to nearest even before the block ends,
// and each MODE write is followed by two wait states before an instruction
// that depends on it). The scaling by 2^-33 is exact in any rounding mode;
// for w = 0 the successor is the smallest subnormal.
__device__ __forceinline__ void sr_unit_words(const uint32_t* w, float* f) {
  float t0, t1, t2, t3, t4, t5, t6, t7;
  asm volatile(
      "s_setreg_imm32_b32 hwreg(HW_REG_MODE, 0, 2), 3\n\t"
      "s_nop 1\n\t"
      "v_cvt_f32_u32 %0, %8\n\t"
      "v_cvt_f32_u32 %1, %9\n\t"
      "v_cvt_f32_u32 %2, %10\n\t"
      "v_cvt_f32_u32 %3, %11\n\t"
      "v_cvt_f32_u32 %4, %12\n\t"
      "v_cvt_f32_u32 %5, %13\n\t"
      "v_cvt_f32_u32 %6, %14\n\t"
      "v_cvt_f32_u32 %7, %15\n\t"
      "s_setreg_imm32_b32 hwreg(HW_REG_MODE, 0, 2), 0\n\t"
      "s_nop 1"
      : "=&v"(t0), "=&v"(t1), "=&v"(t2), "=&v"(t3), "=&v"(t4), "=&v"(t5), "=&v"(t6), "=&v"(t7)
      : "v"(w[0]), "v"(w[1]), "v"(w[2]), "v"(w[3]), "v"(w[4]), "v"(w[5]), "v"(w[6]), "v"(w[7]));
  constexpr float k = 0x1p-33f;
  f[0] = u2f(f2u(t0 * k) + 1u); f[1] = u2f(f2u(t1 * k) + 1u);
  f[2] = u2f(f2u(t2 * k) + 1u); f[3] = u2f(f2u(t3 * k) + 1u);
  f[4] = u2f(f2u(t4 * k) + 1u); f[5] = u2f(f2u(t5 * k) + 1u);
  f[6] = u2f(f2u(t6 * k) + 1u); f[7] = u2f(f2u(t7 * k) + 1u);
}

// z of step 3 for four elements: z = RZ(RZ(|v| - q s2) + s2 / 2), both
// fused multiply-adds under toward-zero rounding in one asm block (MODE
// handling as in sr_unit_words).
__device__ __forceinline__ void sr_z4(const float* v, const float* q, const float* s2, float* z) {
  float z0, z1, z2, z3;
  asm volatile(
      "s_setreg_imm32_b32 hwreg(HW_REG_MODE, 0, 2), 3\n\t"
      "s_nop 1\n\t"
      "v_fma_f32 %0, -%4, %8, |%12|\n\t"
      "v_fma_f32 %1, -%5, %9, |%13|\n\t"
      "v_fma_f32 %2, -%6, %10, |%14|\n\t"
      "v_fma_f32 %3, -%7, %11, |%15|\n\t"
      "v_fma_f32 %0, %8, 0.5, %0\n\t"
      "v_fma_f32 %1, %9, 0.5, %1\n\t"
      "v_fma_f32 %2, %10, 0.5, %2\n\t"
      "v_fma_f32 %3, %11, 0.5, %3\n\t"
      "s_setreg_imm32_b32 hwreg(HW_REG_MODE, 0, 2), 0\n\t"
      "s_nop 1"
      : "=&v"(z0), "=&v"(z1), "=&v"(z2), "=&v"(z3)
      : "v"(q[0]), "v"(q[1]), "v"(q[2]), "v"(q[3]), "v"(s2[0]), "v"(s2[1]), "v"(s2[2]), "v"(s2[3]),
        "v"(v[0]), "v"(v[1]), "v"(v[2]), "v"(v[3]));
  z[0] = z0; z[1] = z1; z[2] = z2; z[3] = z3;
}

// Stochastic-rounding codes of v[0..7] (packed, even element in the low
// nibble), q[j] from sr_unit_words. The conversion writes one byte of its
// destination and keeps the other three; it is written as asm with the
// destination read and written, since the compiler's builtin for it does
// not carry the kept bytes through. A scaled conversion that writes a
// byte other than the lowest is followed by one wait state before an
// instruction that reads its result, as the compiler schedules the
// round-to-nearest form of the same chain.
__device__ __forceinline__ uint32_t sr8(const float* v, const float* q) {
  float s2[8], z[8];
#pragma clang loop unroll(full)
  for (int j = 0; j < 8; ++j) s2[j] = u2f(min(max(f2u(v[j]) & 0x7F800000u, 0x3F800000u), 0x40800000u));
  sr_z4(v, q, s2, z);
  sr_z4(v + 4, q + 4, s2 + 4, z + 4);
  typedef float f32x2_t __attribute__((ext_vector_type(2)));
  double zp[4];
#pragma clang loop unroll(full)
  for (int k = 0; k < 4; ++k)
    zp[k] = __builtin_bit_cast(double, f32x2_t{u2f((f2u(v[2 * k]) & 0x80000000u) | f2u(z[2 * k])),
                                               u2f((f2u(v[2 * k + 1]) & 0x80000000u) | f2u(z[2 * k + 1]))});
  uint32_t out = 0u;
  asm("v_cvt_scalef32_sr_pk_fp4_f32 %0, %1, 0, 1.0\n\t"
      "v_cvt_scalef32_sr_pk_fp4_f32 %0, %2, 0, 1.0 op_sel:[0,0,1,0]\n\t"
      "s_nop 0\n\t"
      "v_cvt_scalef32_sr_pk_fp4_f32 %0, %3, 0, 1.0 op_sel:[0,0,0,1]\n\t"
      "s_nop 0\n\t"
      "v_cvt_scalef32_sr_pk_fp4_f32 %0, %4, 0, 1.0 op_sel:[0,0,1,1]\n\t"
      "s_nop 0"
      : "+v"(out)
      : "v"(zp[0]), "v"(zp[1]), "v"(zp[2]), "v"(zp[3]));
  return out;
}

// Payload code when r overflowed (possible only for a tiny held amax):
// x * r is +-Inf (code 6) for x != 0 and 0 * Inf for x == 0, encoded as a
// signed zero.
__device__ __forceinline__ uint32_t inf_code(float x) {
  return ((f2u(x) >> 28) & 8u) | (x != 0.0f ? 7u : 0u);
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
    n.x = __builtin_amdgcn_bitop3_b32(hi1, c.y, k0, 0x96);  // three-way xor
    n.y = lo1;
    n.z = __builtin_amdgcn_bitop3_b32(hi0, c.w, k1, 0x96);
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

// Byte offsets in an operand's packing. Row-major: code byte j of row r at
// r * C/2 + j, scale j of scale row s at s * nj + j. K64 (the contraction in
// tiles of 64 elements, each tile holding all rows back to back): code byte
// j of row r at (j / 32) * (R * 32) + r * 32 + j % 32 for R rows; scale j of
// scale row s at (j / n) * (SR * n) + s * n + j % n for SR scale rows and
// n = 64 / block scales per row and tile.
__device__ __forceinline__ int64_t code_offset(int64_t r, int64_t j, int64_t R, int64_t C, bool k64) {
  return k64 ? (j >> 5) * (R << 5) + (r << 5) + (j & 31) : r * (C >> 1) + j;
}
template <int kN>
__device__ __forceinline__ int64_t scale_offset(int64_t s, int64_t j, int64_t SR, int64_t nj, bool k64) {
  return k64 ? (j / kN) * (SR * kN) + s * kN + j % kN : s * nj + j;
}

// bf16 -> fp32 widening of a packed pair.
__device__ __forceinline__ float bf16_lo(uint32_t d) { return u2f(d << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t d) { return u2f(d & 0xFFFF0000u); }

}  // namespace fp4q
