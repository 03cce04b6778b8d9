// Emulated FP4 GEMM: Y[M, N] = (A[M, K] . B[N, K]^T) / (Sa Sb) over the
// decoded operands ("UE5M3 FP4 Block Scaling for Stable Language Model
// Pretraining", §6: the contraction of decoded operands, with the encoded
// tensor-scale product applied after accumulation).
//
// Each decoded element e2m1 * dec has at most 6 significant bits and lies in
// [2^-18, 368640]. The default accumulation decodes it times 2^-5, which is
// exact in binary16 (at most 11520, a multiple of 2^-23), and contracts on
// v_mfma_f32_16x16x32_f16 (v_mfma_f32_32x32x16_f16 where K % 64 != 0 or the
// formats are not the default) with fp32 accumulation; alpha absorbs the
// 2^10.
// The probe-matched mode uses the same binary16 operands (each of its
// 64-wide slice sums, their toward-zero additions and its snap then see
// the values times 2^-10 exactly: no rounding step here depends on a power
// of two scaling); FP4Q_PROBE_F16=0 builds it with a bf16 decode on
// v_mfma_f32_32x32x16_bf16 instead.
//
// Design (gfx950):
//  * A workgroup owns a 256 x 256 output tile; its 8 waves (2 along M x 4
//    along N, two per SIMD) own 128 x 64 sub-tiles (32 MFMA accumulators of
//    16 x 16, or 8 of 32 x 32).
//  * 16 x 16 x 32 MFMAs: the chip runs these GEMMs power-limited, and on
//    the decoded FP4 operands the 16 x 16 x 32 instruction sustains a much
//    higher rate than 32 x 32 x 16 at the same nominal peak (a probe with
//    register-resident operands: 0.94 against 0.78 of it). With it the
//    GEMMs run at a higher clock; its k loop (16 MFMA groups per k tile,
//    fragments read several groups ahead) is described at gemm_tile.
//  * K advances in tiles of 64. FP4 codes (0.5 B/element) and one scale byte
//    per 16 elements are read from global memory two tiles ahead into
//    registers; every thread decodes one 64-element row of the stacked
//    [A tile; B tile] into LDS, double buffered, in pieces placed between
//    the MFMAs that consume the other buffer. Decoding once per workgroup
//    costs (256 + 256) * 64 elements per 256 * 256 * 64 MACs.
//  * The k tile is rotated: the decode ends before the last quarter of the
//    tile's MFMAs, the workgroup barrier (LDS traffic only, so the codes in
//    flight for later tiles are not waited for) comes there, and the next
//    tile's first fragments are read under that quarter's MFMAs.
//  * Decode: v_cvt_scalef32_pk_f16_fp4 (scale 1.0) gives two exact E2M1
//    values as halves and one packed half multiply by the block's scale pair
//    forms the products: two instructions per pair of elements. (A bf16
//    decode, kept for FP4Q_PROBE_F16=0, takes four: a conversion to fp32,
//    two fp32 multiplies and a packing conversion.)
//  * LDS rows are 8 chunks of 16 bytes (8 k each). The 16 x 16 kernels store
//    them chunk-major (chunk c of row r at slot c * rows + r): their
//    fragment reads (16 rows in each of 4 chunks) and the decode writes (64
//    rows, one chunk) then touch consecutive slots and measured free of bank
//    conflicts, where the 144-byte row pitch gave about 4 conflict cycles
//    per fragment read. The 32 x 32 kernels keep the 144-byte pitch (their
//    32-row reads are conflict-free with it, and it measured faster).
//  * Workgroups are numbered so that consecutive ones on one XCD (hardware
//    dispatch is round-robin over the 8 XCDs) cover a compact group of tiles,
//    which keeps their shared A and B rows in that XCD's L2.
//  * A workgroup of the default kernels runs two tiles of that order one
//    after the other where the chip's tile rounds stay as many (fwd, dgrad
//    and wgrad of the FFN shapes): 0.3-0.8% faster steps with 32 x 32 x 16
//    MFMAs, the same with 16 x 16 x 32.
//  * Under sustained load the chip runs power-limited (its clock drops well
//    below the nominal 2.4 GHz); the binary16 decode's fewer VALU
//    instructions measured about 4% faster than the bf16 decode.
//
// One kernel serves fwd (A = X, ROW16; B = W, TILE), dgrad (A = dY, ROW16;
// B = W^T, TILE) and wgrad (A = dY^T, B = X^T, both quantized along tokens):
// both operands are stored contiguous along the contraction.
#include <atomic>
#include <type_traits>

#include "codec.h"
#include "kernels.h"

// Build switches, defaults measured fastest. FP4Q_GEMM_SWZ: LDS layout of
// the default kernels' decoded tiles (3: chunk-major, the 16-byte chunk c of
// row r at c * rows + r; 2: 144-byte padded row pitch; 0 and 1: 128-byte
// rows with the chunk index XORed by row bits; the probe kernels use 2).
// FP4Q_GEMM_ROTATE: the rotated k tile described above (0: decode,
// barrier, then all four k16 steps). FP4Q_PROBE_F16: binary16 operands in
// the probe-matched mode. FP4Q_GEMM_MFMA16: 16 x 16 x 32 MFMAs in the
// default kernels (0: 32 x 32 x 16), scheduled by FP4Q_M16_TAIL (groups
// after the barrier), FP4Q_M16_DIST (A fragments read this many groups
// ahead), FP4Q_M16_BSTART (group reading the first B fragment of the
// second k32 step) and FP4Q_M16_DEC0 / FP4Q_M16_DECSPAN (groups followed
// by the decode pieces; span 0: up to the barrier).
#ifndef FP4Q_GEMM_SWZ
#define FP4Q_GEMM_SWZ 3
#endif
#ifndef FP4Q_GEMM_ROTATE
#define FP4Q_GEMM_ROTATE 1
#endif
#ifndef FP4Q_PROBE_F16
#define FP4Q_PROBE_F16 1
#endif
#ifndef FP4Q_GEMM_MFMA16
#define FP4Q_GEMM_MFMA16 1
#endif
#ifndef FP4Q_M16_TAIL
#define FP4Q_M16_TAIL 4
#endif
#ifndef FP4Q_M16_DIST
#define FP4Q_M16_DIST 5
#endif
#ifndef FP4Q_M16_BSTART
#define FP4Q_M16_BSTART 3
#endif
#ifndef FP4Q_M16_DEC0
#define FP4Q_M16_DEC0 0
#endif
#ifndef FP4Q_M16_DECSPAN
#define FP4Q_M16_DECSPAN 0
#endif

namespace fp4q {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));

constexpr int BM = 256;   // tile of the default kernel
constexpr int BN = 256;
constexpr int BK = 64;    // k tile (also the slice of the probe mode)
constexpr int kPM = 128;  // tile of the probe-mode kernel
constexpr int kThreads = 256;
constexpr int kChunks = BK / 8;              // 16-byte chunks per LDS row
#ifndef FP4Q_GEMM_GROUP_M
#define FP4Q_GEMM_GROUP_M 8
#endif
constexpr int kGroupM = FP4Q_GEMM_GROUP_M;   // M-tiles per scheduling group

// Codes and scales of one 64-element row segment (4 blocks of 16, or 2 of
// 32). The scale bytes are kept as loaded (s0: the first two, s1: the next
// two, unused for blocks of 32) and picked apart only when decoded, so no
// arithmetic waits on the loads where they are issued.
struct RowSeg {
  uint4 c0, c1;    // 32 bytes of codes
  uint32_t s0, s1;
};

// Output tile of grouped position t: kGroupM M-tiles per group, N-tiles
// column by column inside a group.
__device__ __forceinline__ void tile_coords(int t, int tiles_m, int tiles_n, int* tm, int* tn) {
  const int group = t / (kGroupM * tiles_n);
  const int first_m = group * kGroupM;
  const int gm = min(tiles_m - first_m, kGroupM);
  const int in_group = t - group * kGroupM * tiles_n;
  *tm = first_m + in_group % gm;
  *tn = in_group / gm;
}

// Scale code of the 16-element block j (0..3) of a segment. kFmt false:
// blocks of 16 only, and s0 holds all four scale bytes.
template <bool kFmt>
__device__ __forceinline__ uint32_t seg_scale(const RowSeg& g, int j, bool blk32) {
  if (!kFmt) return (g.s0 >> (8 * j)) & 0xFFu;
  const uint32_t w = (blk32 || j < 2) ? g.s0 : g.s1;
  return (w >> (blk32 ? 8 * (j >> 1) : 8 * (j & 1))) & 0xFFu;
}

// K % 64 == 0: a whole segment is in bounds; rows past the end are clamped
// to the last row (their products only reach outputs that are not stored),
// so the load is branch-free. blk32: blocks of 32 (else 16); the second
// 16-bit scale load repeats the first for blocks of 32, so it stays inside
// the row. kK64: the K64 packing, where a segment is the row's 32 bytes of
// k tile k0 / 64 and the workgroup's consecutive rows are adjacent.
template <bool kFmt, bool kK64, bool kNT = false>
__device__ __forceinline__ RowSeg load_seg_full(const uint8_t* __restrict__ codes,
                                                const uint8_t* __restrict__ scales, int64_t rows,
                                                int64_t K, int tile_shift, bool blk32, int64_t r,
                                                int64_t k0) {
  r = r < rows ? r : rows - 1;
  const int64_t kt = k0 / BK;
  const int64_t srows = rows >> tile_shift;
  const uint8_t* cp = kK64 ? codes + kt * (rows * 32) + r * 32 : codes + r * (K / 2) + k0 / 2;
  RowSeg g;
  if constexpr (kNT) {
    g.c0 = load_nt16(cp);
    g.c1 = load_nt16(cp + 16);
  } else {
    g.c0 = *reinterpret_cast<const uint4*>(cp);
    g.c1 = *reinterpret_cast<const uint4*>(cp + 16);
  }
  if (!kFmt) {
    const uint32_t* sp = reinterpret_cast<const uint32_t*>(
        kK64 ? scales + kt * (srows * 4) + (r >> tile_shift) * 4
             : scales + (r >> tile_shift) * (K / 16) + k0 / 16);
    g.s0 = kNT ? __builtin_nontemporal_load(sp) : *sp;
    g.s1 = 0u;
    return g;
  }
  const int sh = blk32 ? 5 : 4;
  const int n = blk32 ? 2 : 4;  // scale bytes per row and k tile
  const uint8_t* sp = kK64 ? scales + kt * (srows * n) + (r >> tile_shift) * n
                           : scales + (r >> tile_shift) * (K >> sh) + (k0 >> sh);
  g.s0 = *reinterpret_cast<const uint16_t*>(sp);
  g.s1 = *reinterpret_cast<const uint16_t*>(blk32 ? sp : sp + 2);
  return g;
}

// General K (a multiple of the block size): blocks at or beyond K read as
// zero codes.
template <bool kFmt>
__device__ __forceinline__ RowSeg load_seg_tail(const uint8_t* __restrict__ codes,
                                                const uint8_t* __restrict__ scales, int64_t rows,
                                                int64_t K, int tile_shift, bool blk32, int64_t r,
                                                int64_t k0) {
  r = r < rows ? r : rows - 1;
  const int bl = blk32 ? 32 : 16;
  const uint8_t* cp = codes + r * (K / 2);
  const uint8_t* sp = scales + (r >> tile_shift) * (K / bl);
  uint2 b[4];
  uint32_t sb[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int64_t kb = k0 + 16 * j;
    if (kb < K) {
      b[j] = *reinterpret_cast<const uint2*>(cp + kb / 2);
      sb[j] = sp[kb / bl];
    } else {
      b[j] = make_uint2(0u, 0u);
      sb[j] = 0u;
    }
  }
  RowSeg g;
  g.c0 = make_uint4(b[0].x, b[0].y, b[1].x, b[1].y);
  g.c1 = make_uint4(b[2].x, b[2].y, b[3].x, b[3].y);
  // same packing as the full path: for blocks of 32, s0 holds the two
  // block codes (blocks 0-1 share code 0, blocks 2-3 code 1)
  if (!kFmt) {
    g.s0 = sb[0] | (sb[1] << 8) | (sb[2] << 16) | (sb[3] << 24);
    g.s1 = 0u;
    return g;
  }
  g.s0 = blk32 ? (sb[0] | (sb[2] << 8)) : (sb[0] | (sb[1] << 8));
  g.s1 = sb[2] | (sb[3] << 8);
  return g;
}

template <bool kFullK, bool kFmt, bool kK64, bool kNT = false>
__device__ __forceinline__ RowSeg load_seg(const uint8_t* __restrict__ codes,
                                           const uint8_t* __restrict__ scales, int64_t rows,
                                           int64_t K, int tile_shift, bool blk32, int64_t r,
                                           int64_t k0) {
  static_assert(kFullK || !kK64, "the K64 packing needs K % 64 == 0");
  return kFullK ? load_seg_full<kFmt, kK64, kNT>(codes, scales, rows, K, tile_shift, blk32, r, k0)
                : load_seg_tail<kFmt>(codes, scales, rows, K, tile_shift, blk32, r, k0);
}

// Nontemporal loads for the B operand (the operand a tile group streams
// through while its A panel stays in the L2).
#ifndef FP4Q_GEMM_NT_B
#define FP4Q_GEMM_NT_B 0
#endif

// 8 codes (one 32-bit word, element e in bits 4e+3:4e) of a block with
// decoded scale dec -> 8 bf16, element order kept.
__device__ __forceinline__ uint4 decode8(uint32_t w, float dec) {
  const f32x2 p0 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 0);
  const f32x2 p1 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 1);
  const f32x2 p2 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 2);
  const f32x2 p3 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 3);
  const bf16x2 b0 = {(__bf16)(p0.x * dec), (__bf16)(p0.y * dec)};
  const bf16x2 b1 = {(__bf16)(p1.x * dec), (__bf16)(p1.y * dec)};
  const bf16x2 b2 = {(__bf16)(p2.x * dec), (__bf16)(p2.y * dec)};
  const bf16x2 b3 = {(__bf16)(p3.x * dec), (__bf16)(p3.y * dec)};
  return make_uint4(__builtin_bit_cast(uint32_t, b0), __builtin_bit_cast(uint32_t, b1),
                    __builtin_bit_cast(uint32_t, b2), __builtin_bit_cast(uint32_t, b3));
}

// The same 8 codes -> 8 halves e2m1 * m, with m = (dec 2^-5, dec 2^-5) the
// block's scale pair from half_scale: v_cvt_scalef32_pk_f16_fp4 (scale 1.0)
// gives the exact E2M1 values and one packed half multiply per pair forms
// the products, which are exact in binary16 (see half_scale).
__device__ __forceinline__ uint4 decode8_h(uint32_t w, f16x2 m) {
  const f16x2 p0 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 0);
  const f16x2 p1 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 1);
  const f16x2 p2 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 2);
  const f16x2 p3 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 3);
  return make_uint4(__builtin_bit_cast(uint32_t, p0 * m), __builtin_bit_cast(uint32_t, p1 * m),
                    __builtin_bit_cast(uint32_t, p2 * m), __builtin_bit_cast(uint32_t, p3 * m));
}

// Scale pair of the binary16 decode: dec 2^-5 in both halves. A UE5M3 code c
// has the value of the half with bit pattern c << 7, so one packed multiply
// by 2^-5 (2^3 for E4M3, whose value is the UE5M3 one times 2^8) gives it,
// exactly: dec 2^-5 lies in [2^-22, 1920] and is a multiple of 2^-24.
// Every product e2m1 * dec 2^-5 is then exact in binary16 as well: it is at
// most 6 * 1920 = 11520, and it is an integer of at most 8 bits times a power
// of two no smaller than 2^-23. The products of two such operands are exact
// in the MFMA's binary32 arithmetic, so the accumulated sums are the bf16
// path's sums times 2^-10, and alpha is taken 2^10 times larger.
__device__ __forceinline__ f16x2 half_scale(uint32_t code, bool e4m3) {
  const f16x2 v = __builtin_bit_cast(f16x2, (code << 7) | (code << 23));
  const _Float16 k = e4m3 ? (_Float16)8.0f : (_Float16)0.03125f;
  return v * f16x2{k, k};
}

__device__ __forceinline__ uint32_t seg_word(const RowSeg& g, int c) {
  switch (c) {
    case 0: return g.c0.x;
    case 1: return g.c0.y;
    case 2: return g.c0.z;
    case 3: return g.c0.w;
    case 4: return g.c1.x;
    case 5: return g.c1.y;
    case 6: return g.c1.z;
    default: return g.c1.w;
  }
}

// LDS slot of 16-byte chunk c of tile row r (8 chunks per row of 64 k) in
// a buffer of kRowsAll rows.
template <int kSwz, int kRowsAll>
__device__ __forceinline__ int slot(int r, int c) {
  if (kSwz == 3) return c * kRowsAll + r;        // chunk-major
  if (kSwz == 2) return r * (kChunks + 1) + c;  // 144-byte row pitch
  return r * kChunks + (kSwz == 0 ? (c ^ (r & 7)) : (c ^ ((r >> 1) & 7)));
}
template <int kSwz>
constexpr int row_pitch() { return kSwz == 2 ? kChunks + 1 : kChunks; }

// The GEMM's LDS: 2 buffers x (A tile + B tile) rows at the LDS row pitch
// (144 KiB for 256 x 256 tiles). kArg: reach it through the caller's
// pointer to the same array, the form the default kernels take (it measured
// 0.5-1.5% faster in their tile loop; the format-generic kernels would
// spill with it).
template <bool kArg>
__device__ __forceinline__ uint4* lds_base(uint4* arg) {
  extern __shared__ uint4 lds_ext[];
  if constexpr (kArg) return arg;
  else return lds_ext;
}

// One output tile: kWavesM x kWavesN waves over a kBM x kBN tile; wave
// tile (kBM / kWavesM) x (kBN / kWavesN) built from 16 x 16 or 32 x 32 MFMA
// blocks. L is the tile's logical workgroup index (see gemm_kernel below).
//
// kProbe: the probe-matched accumulation of the UE5M3 page (§6, Appendix
// B). Each 64-wide k tile is one slice: its MFMAs start from zero, and the
// slice result is added to a running sum with binary32 additions rounded
// toward zero (the MODE register's single-precision rounding field is set
// to round-toward-zero around those additions only); the epilogue
// optionally snaps the sum to multiples of 2^-snap_log2 (ties to even; on
// the 2^-10-scaled binary16 sums, multiples of 2^-(snap_log2 + 10)) before
// applying alpha.
template <int kBM, int kBN, bool kFullK, bool kF32Out, int kWavesM, int kWavesN, int kSwz, bool kProbe,
          bool kFmt, bool kK64, bool kLdsArg>
__device__ __forceinline__ void gemm_tile(
    const uint8_t* __restrict__ a_codes, const uint8_t* __restrict__ a_scales, int a_shift,
    const float* __restrict__ a_S, const uint8_t* __restrict__ b_codes,
    const uint8_t* __restrict__ b_scales, int b_shift, const float* __restrict__ b_S, int64_t M,
    int64_t N, int64_t K, int tiles_m, int tiles_n, int snap_log2, int fmt, int split_local,
    void* __restrict__ y, const int L, const int tid, uint4* lds_arg) {
  // fmt bits: 0 A blocks of 32, 1 A E4M3 scales, 2 B blocks of 32, 3 B E4M3
  // scales; kFmt false compiles the default (blocks of 16, UE5M3) only
  const bool a_blk32 = kFmt && (fmt & 1), a_e4m3 = kFmt && (fmt & 2);
  const bool b_blk32 = kFmt && (fmt & 4), b_e4m3 = kFmt && (fmt & 8);
  constexpr int kT = 64 * kWavesM * kWavesN;  // threads
  constexpr int kTM = kBM / kWavesM;           // wave tile rows
  constexpr int kTN = kBN / kWavesN;           // wave tile cols
  // default kernels with K % 64 == 0: 16 x 16 x 32 MFMA blocks; the
  // others (general K, probe, format-generic): 32 x 32 x 16
  constexpr bool kM16 = FP4Q_GEMM_MFMA16 && !kProbe && !kFmt && kFullK && FP4Q_GEMM_ROTATE;
  constexpr int kEdge = kM16 ? 16 : 32;       // MFMA output block edge
  constexpr int kAccN = kM16 ? 4 : 16;        // accumulators per lane and block
  using acc_t = typename std::conditional<kM16, f32x4, f32x16>::type;
  constexpr int kFM = kTM / kEdge;            // MFMA blocks per wave along M
  // LDS layout: the chunk-major one (3) serves the 16 x 16 fragment reads
  // without bank conflicts; the 32 x 32 path keeps the padded rows (2)
  constexpr int kLay = (!kM16 && kSwz == 3) ? 2 : kSwz;
  constexpr int kFN = kTN / kEdge;            // and along N
  constexpr int kRows = (kBM + kBN) / kT;       // A/B tile rows each thread decodes
  constexpr int kPieces = 2 * kRows;          // decode8 calls per thread per k16 step
  constexpr int kMfmaPerPiece = kFM * kFN / kPieces;
  static_assert(kFM * kFN % kPieces == 0, "MFMA count must split evenly");
  // operands decoded to binary16 (times 2^-5); a bf16 decode for the probe
  // mode if FP4Q_PROBE_F16 is 0
  constexpr bool kF16 = !kProbe || FP4Q_PROBE_F16;

  // ---- XCD-aware tile order: logical workgroup L runs on XCD L % 8 (see
  // gemm_kernel); give each XCD a contiguous range of the grouped tile
  // order.
  // Split tail (split_local >= 0, fp32 output, tile count a multiple of 8):
  // each XCD's tiles from split_local on are run as two workgroups over the
  // two halves of K, so the last round of tiles fills the chip; they add
  // their partial results into an output zeroed beforehand.
  const int ntiles = tiles_m * tiles_n;
  const int per_xcd = (ntiles + 7) / 8;
  const int xcd = L % 8;
  const int local = L / 8;
  int t, half = -1;
  if (split_local >= 0 && local >= split_local) {
    t = xcd * per_xcd + split_local + (local - split_local) / 2;
    half = (local - split_local) & 1;
  } else {
    const int full_xcds = ntiles % 8 ? ntiles % 8 : 8;  // XCDs that receive per_xcd tiles
    t = xcd < full_xcds ? xcd * per_xcd + local
                        : full_xcds * per_xcd + (xcd - full_xcds) * (per_xcd - 1) + local;
  }
  int tm, tn;
  tile_coords(t, tiles_m, tiles_n, &tm, &tn);

  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wm = wave / kWavesN;
  const int wn = wave % kWavesN;
  const int64_t m0 = (int64_t)tm * kBM;
  const int64_t n0 = (int64_t)tn * kBN;

  // rows this thread decodes: tile row q = tid + i * kT of the stacked
  // [A tile; B tile] (A rows 0..255, B rows 256..511)
  auto load_rows = [&](RowSeg* g, int64_t k0) {
#pragma unroll
    for (int i = 0; i < kRows; ++i) {
      const int q = tid + i * kT;
      g[i] = q < kBM
                 ? load_seg<kFullK, kFmt, kK64>(a_codes, a_scales, M, K, a_shift, a_blk32, m0 + q, k0)
                 : load_seg<kFullK, kFmt, kK64, (bool)FP4Q_GEMM_NT_B && !kProbe>(
                       b_codes, b_scales, N, K, b_shift, b_blk32, n0 + (q - kBM), k0);
    }
  };
  // one decode8 piece p (0 .. kPieces-1) of block s into buffer `buf`
  auto decode_piece = [&](uint4* buf, const RowSeg* g, int s, int p) {
    const int i = p >> 1;
    const int q = tid + i * kT;
    const int c = 2 * s + (p & 1);
    const bool is_a = q < kBM;
    const uint32_t code = seg_scale<kFmt>(g[i], s, is_a ? a_blk32 : b_blk32);
    const bool e4m3 = is_a ? a_e4m3 : b_e4m3;
    if constexpr (kF16)
      buf[slot<kLay, kBM + kBN>(q, c)] = decode8_h(seg_word(g[i], c), half_scale(code, e4m3));
    else
      buf[slot<kLay, kBM + kBN>(q, c)] = decode8(seg_word(g[i], c), scale_value(code, e4m3));
  };

  acc_t acc[kFM][kFN];
  f32x16 tot[kProbe ? kFM : 1][kProbe ? kFN : 1];  // running sums of the probe mode
#pragma unroll
  for (int i = 0; i < kFM; ++i)
#pragma unroll
    for (int j = 0; j < kFN; ++j)
#pragma unroll
      for (int e = 0; e < kAccN; ++e) acc[i][j][e] = 0.0f;
#pragma unroll
  for (int i = 0; i < (kProbe ? kFM : 1); ++i)
#pragma unroll
    for (int j = 0; j < (kProbe ? kFN : 1); ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) tot[i][j][e] = 0.0f;

  const int nk_all = (int)((K + BK - 1) / BK);
  // k tiles [k_begin, nk) of this workgroup: all, or one half for a split tile
  const int k_begin = half == 1 ? nk_all / 2 : 0;
  const int nk = half == 0 ? nk_all / 2 : nk_all;
  RowSeg g[kRows];  // codes of tile kt + 1, decoded during iteration kt
  if (nk > k_begin) {
    load_rows(g, (int64_t)k_begin * BK);
#pragma unroll
    for (int s = 0; s < 4; ++s)
#pragma unroll
      for (int p = 0; p < kPieces; ++p) decode_piece(lds_base<kLdsArg>(lds_arg), g, s, p);
    load_rows(g, (int64_t)min(k_begin + 1, nk - 1) * BK);
    lds_barrier();  // the codes just requested are first needed by a decode of the first k tile
  }

  if constexpr (kM16) {
    // 16 x 16 x 32 MFMAs (at the same nominal rate as 32 x 32 x 16, they
    // move half the accumulator data per product and sustain a higher rate
    // under the chip's power limit). A lane's fragment is 8 consecutive k of
    // one row: row lane % 16 of the block, k chunk lane / 16 of the k32 step.
    // A k tile is two k32 steps of kFM groups; group G multiplies A block
    // row G % kFM with the step's kFN B fragments (kFN MFMAs). The B
    // fragments of a step stay in registers for it (the second step's are
    // read from group kBStart on); A fragments are read kDist groups ahead.
    // The next buffer's decode pieces follow groups spread over the first
    // kG - kTail groups; the barrier (LDS traffic only) comes before the
    // last kTail groups, whose fragments are in registers by then, and the
    // next k tile's B fragments and first two A fragments are read from the
    // freshly decoded buffer under those groups' MFMAs.
    const int quad = lane >> 4;
    const int arow = wm * kTM + (lane & 15);
    const int brow = kBM + wn * kTN + (lane & 15);
    constexpr int kG = 2 * kFM;  // A groups per k tile
    constexpr int kTail = FP4Q_M16_TAIL;  // groups after the barrier
    constexpr int kDist = FP4Q_M16_DIST;  // A fragments read this many groups ahead
    constexpr int kBStart = FP4Q_M16_BSTART;  // group that reads the first B fragment of step 1
    // decode pieces follow groups spread over [kDec0, kDec0 + kDecSpan)
    constexpr int kDec0 = FP4Q_M16_DEC0;
    constexpr int kDecSpan = FP4Q_M16_DECSPAN > 0 ? FP4Q_M16_DECSPAN : kG - kTail - kDec0;
    static_assert(kDec0 + kDecSpan <= kG - kTail, "decode pieces precede the barrier");
    static_assert(kFM >= kFN && kG - kTail >= 8 && kBStart + kFN <= kFM && kTail >= 2,
                  "16 x 16 schedule: wave tile shape");
    auto frag = [&](const uint4* buf, int row, int step) {
      return buf[slot<kLay, kBM + kBN>(row, 4 * step + quad)];
    };
    uint4 bq[2][kFN];  // B fragments of the k tile's two k32 steps
    uint4 an[2];       // A fragments of the next k tile's first two groups
    if (nk > k_begin) {
      const uint4* b0 = lds_base<kLdsArg>(lds_arg);
#pragma unroll
      for (int j = 0; j < kFN; ++j) bq[0][j] = frag(b0, brow + 16 * j, 0);
      an[0] = frag(b0, arow, 0);
      an[1] = frag(b0, arow + 16, 0);
    }
    auto k_step16 = [&](int kt, const RowSeg* gd, RowSeg* gl) {
      constexpr int kBuf = (kBM + kBN) * row_pitch<kLay>();
      const uint4* cur_buf = lds_base<kLdsArg>(lds_arg) + ((kt - k_begin) & 1) * kBuf;
      uint4* next_buf = lds_base<kLdsArg>(lds_arg) + ((kt - k_begin + 1) & 1) * kBuf;
      uint4 a[kG];
      a[0] = an[0];
      a[1] = an[1];
#pragma unroll
      for (int G = 0; G < kG; ++G) {
        const int st = G / kFM, i = G % kFM;
        if (G == kG - kTail) {
          // every wave's decode into next_buf and its reads of cur_buf are done
          lds_barrier();
#pragma unroll
          for (int j = 0; j < kFN; ++j) bq[0][j] = frag(next_buf, brow + 16 * j, 0);
          an[0] = frag(next_buf, arow, 0);
          an[1] = frag(next_buf, arow + 16, 0);
          __builtin_amdgcn_sched_barrier(0);
        }
        // A fragment x (2 <= x < kG) is read at group min(max(x - kDist, 0),
        // kG - kTail - 1): every read of cur_buf precedes the barrier
#pragma unroll
        for (int x = 2; x < kG; ++x)
          if (min(max(x - kDist, 0), kG - kTail - 1) == G)
            a[x] = frag(cur_buf, arow + 16 * (x % kFM), x / kFM);
        if (G >= kBStart && G < kBStart + kFN)
          bq[1][G - kBStart] = frag(cur_buf, brow + 16 * (G - kBStart), 1);
#pragma unroll
        for (int j = 0; j < kFN; ++j) {
          acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, a[G]),
                                                             __builtin_bit_cast(f16x8, bq[st][j]), acc[i][j], 0,
                                                             0, 0);
          if (G == 0 && j == 0) {
            // codes of tile kt + 2 (the last tile again near the end: harmless)
            load_rows(gl, (int64_t)min(kt + 2, nk - 1) * BK);
            __builtin_amdgcn_sched_barrier(0);
          }
        }
        // decode piece q (16-byte chunk q of this thread's row) follows
        // group kDec0 + (q + 1) kDecSpan / 8 - 1
#pragma unroll
        for (int q = 0; q < 8; ++q)
          if (kDec0 + (q + 1) * kDecSpan / 8 - 1 == G) {
            decode_piece(next_buf, gd, q >> 1, q & 1);
            __builtin_amdgcn_sched_barrier(0);
          }
        __builtin_amdgcn_sched_barrier(0);
      }
    };
    RowSeg g2[kRows];
    int kt = k_begin;
    for (; kt + 1 < nk; kt += 2) {
      k_step16(kt, g, g2);
      k_step16(kt + 1, g2, g);
    }
    if (kt < nk) k_step16(kt, g, g2);
  } else {
    const int arow0 = wm * kTM + (lane & 31);
    const int brow0 = kBM + wn * kTN + (lane & 31);
    const int hi = lane >> 5;

    // fragments: eight 16-bit values per lane (binary16, or bf16 for a probe
    // mode built with FP4Q_PROBE_F16=0), bit-cast to the MFMA's operand type
    auto load_frags = [&](const uint4* buf, int s, bf16x8* af, bf16x8* bfr) {
      const int ch = 2 * s + hi;
#pragma unroll
      for (int i = 0; i < kFM; ++i)
        af[i] = __builtin_bit_cast(bf16x8, buf[slot<kLay, kBM + kBN>(arow0 + 32 * i, ch)]);
#pragma unroll
      for (int j = 0; j < kFN; ++j)
        bfr[j] = __builtin_bit_cast(bf16x8, buf[slot<kLay, kBM + kBN>(brow0 + 32 * j, ch)]);
    };

    // one k tile: MFMAs on the current buffer while the codes of tile kt + 1
    // (gd) are decoded into the other one and those of tile kt + 2 are loaded
    // into gl. The loop runs two k tiles per trip with gd and gl swapping
    // roles, so no register copy waits for the loads just issued, and the
    // barrier between k tiles (lds_barrier) waits for LDS traffic only, not
    // for the codes in flight for later k tiles.
    // Fragments of the current and the next k16 step. With FP4Q_GEMM_ROTATE
    // the decode of the next buffer ends with the third k16 step, the barrier
    // comes before the fourth, and the next k tile's first fragments are read
    // while the fourth step's MFMAs run (they are in registers when that k
    // tile starts).
    bf16x8 af[2][kFM], bfr[2][kFN];
    if (FP4Q_GEMM_ROTATE && nk > k_begin) load_frags(lds_base<kLdsArg>(lds_arg), 0, af[0], bfr[0]);
    constexpr int kMfma = kFM * kFN;                   // MFMAs per k16 step
    constexpr int kDecStride = kMfma >= 8 ? kMfma / 4 : 1;
    // the rotated schedule's 3 + 3 + 2 decode pieces: one tile row per thread
    static_assert(!FP4Q_GEMM_ROTATE || (kRows == 1 && BK == 64), "rotated k tile: one decoded row per thread");
    auto k_step = [&](int kt, const RowSeg* gd, RowSeg* gl) {
      constexpr int kBuf = (kBM + kBN) * row_pitch<kLay>();
      const uint4* cur_buf = lds_base<kLdsArg>(lds_arg) + ((kt - k_begin) & 1) * kBuf;
      uint4* next_buf = lds_base<kLdsArg>(lds_arg) + ((kt - k_begin + 1) & 1) * kBuf;
      // codes of tile kt + 2 (the last tile again near the end: harmless);
      // in the rotated default kernel they are requested after the first MFMA,
      // so that their address arithmetic issues under it
      constexpr bool kLateLoad = FP4Q_GEMM_ROTATE && !kProbe;
      if (!kLateLoad) load_rows(gl, (int64_t)min(kt + 2, nk - 1) * BK);
      if (!FP4Q_GEMM_ROTATE) load_frags(cur_buf, 0, af[0], bfr[0]);
#pragma unroll
      for (int s = 0; s < BK / 16; ++s) {
        const int cb = s & 1;
        if (s + 1 < BK / 16) {
          load_frags(cur_buf, s + 1, af[cb ^ 1], bfr[cb ^ 1]);
        } else if (FP4Q_GEMM_ROTATE) {
          // every wave's decode into next_buf and its reads of this step's
          // fragments are done: the next k tile's first fragments can be read
          lds_barrier();
          load_frags(next_buf, 0, af[cb ^ 1], bfr[cb ^ 1]);
        }
        if (FP4Q_GEMM_ROTATE) {
          // the 2 * (BK / 16) decode pieces of the next buffer over the first
          // three k16 steps (3, 3, 2), each after kDecStride MFMAs
          constexpr int kQ = 2 * (BK / 16);
          const int q0 = s == 0 ? 0 : s == 1 ? 3 : s == 2 ? 6 : kQ;
          const int q1 = s == 0 ? 3 : s == 1 ? 6 : kQ;
#pragma unroll
          for (int f = 0; f < kMfma; ++f) {
            const int i = f / kFN, j = f % kFN;
            if constexpr (kF16)
              acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(
                  __builtin_bit_cast(f16x8, af[cb][i]), __builtin_bit_cast(f16x8, bfr[cb][j]),
                  (kProbe && s == 0) ? f32x16{} : acc[i][j], 0, 0, 0);
            else
              acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                  af[cb][i], bfr[cb][j], (kProbe && s == 0) ? f32x16{} : acc[i][j], 0, 0, 0);
            const int q = q0 + f / kDecStride;
            if ((f + 1) % kDecStride == 0 && q < q1) {
              decode_piece(next_buf, gd, q >> 1, q & 1);
              __builtin_amdgcn_sched_barrier(0);
            }
            if (kLateLoad && s == 0 && f == 0) {
              load_rows(gl, (int64_t)min(kt + 2, nk - 1) * BK);
              __builtin_amdgcn_sched_barrier(0);
            }
          }
          __builtin_amdgcn_sched_barrier(0);
        } else {
          // block s of the next tile is decoded in kPieces pieces, each after
          // kMfmaPerPiece MFMAs, so that the VALU work issues while the matrix
          // core is busy
#pragma unroll
          for (int p = 0; p < kPieces; ++p) {
#pragma unroll
            for (int u = 0; u < kMfmaPerPiece; ++u) {
              const int f = p * kMfmaPerPiece + u;
              const int i = f / kFN, j = f % kFN;
              if constexpr (kF16)
                acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(
                    __builtin_bit_cast(f16x8, af[cb][i]), __builtin_bit_cast(f16x8, bfr[cb][j]),
                    (kProbe && s == 0) ? f32x16{} : acc[i][j], 0, 0, 0);
              else
                acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                    af[cb][i], bfr[cb][j], (kProbe && s == 0) ? f32x16{} : acc[i][j], 0, 0, 0);
            }
            decode_piece(next_buf, gd, s, p);
            __builtin_amdgcn_sched_barrier(0);
          }
        }
      }
      if constexpr (kProbe) {
        // add the slice partials to the running sums with round-toward-zero.
        // The MODE rounding field governs these VALU additions only: MFMA
        // results are the same under either mode (checked on 65536 random
        // outputs). The compiler does not model the additions' dependence on
        // MODE (a plain fp32 add may legally move across a MODE write, and
        // one k tile's additions of each unrolled pair did), so the two MODE
        // writes and every addition are volatile asm statements, which keep
        // their order: all 64 additions run inside the window. The asm hides
        // the additions' reads of the matrix core's results from the
        // compiler's hazard tracking, so the window opens with 24 wait states
        // (more than a 16-pass MFMA result needs before a VALU read, and the
        // MODE write's own two).
        __builtin_amdgcn_sched_barrier(0);
        asm volatile("s_setreg_imm32_b32 hwreg(HW_REG_MODE, 0, 2), 3\n\ts_nop 7\n\ts_nop 7\n\ts_nop 7" ::
                         : "memory");
#pragma unroll
        for (int i = 0; i < kFM; ++i)
#pragma unroll
          for (int j = 0; j < kFN; ++j)
#pragma unroll
            for (int e = 0; e < 16; ++e) {
              float t;
              asm volatile("v_add_f32 %0, %1, %2" : "=v"(t) : "v"(tot[i][j][e]), "v"(acc[i][j][e]));
              tot[i][j][e] = t;
            }
        asm volatile("s_setreg_imm32_b32 hwreg(HW_REG_MODE, 0, 2), 0\n\ts_nop 1" ::: "memory");
        __builtin_amdgcn_sched_barrier(0);
      }
      if (!FP4Q_GEMM_ROTATE) lds_barrier();
    };
    RowSeg g2[kRows];
    int kt = k_begin;
    for (; kt + 1 < nk; kt += 2) {
      k_step(kt, g, g2);
      k_step(kt + 1, g2, g);
    }
    if (kt < nk) k_step(kt, g, g2);
  }
  if constexpr (kProbe) {
    // sums of binary16 operands carry 2^-10 (alpha restores it): the snap
    // grid moves by the same 10 bits
    constexpr int kSnapShift = kF16 ? 10 : 0;
#pragma unroll
    for (int i = 0; i < kFM; ++i)
#pragma unroll
      for (int j = 0; j < kFN; ++j)
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const float t = tot[i][j][e];
          acc[i][j][e] = snap_log2 > 0
                             ? __builtin_ldexpf(__builtin_rintf(__builtin_ldexpf(t, snap_log2 + kSnapShift)),
                                                -snap_log2 - kSnapShift)
                             : t;
        }
  }

  // epilogue: y = acc * alpha, alpha = 1 / (Sa Sb). Interior tiles (and a
  // normal fp32 alpha) take a branch-free path: a uniform tile base plus
  // 32-bit in-tile offsets, two rows per step.
  const double alpha_d = (kF16 ? 1024.0 : 1.0) / ((double)*a_S * (double)*b_S);
  const float alpha = (float)alpha_d;
  const bool alpha_normal = alpha >= 1.17549435e-38f && alpha <= 3.40282347e+38f;
  constexpr int es = kF32Out ? 4 : 2;
  // accumulator e of block (i, j): in-tile row i kEdge + erow(e) + lrow,
  // column j kEdge + (lane % kEdge) (32 x 32 blocks: rows 8 (e / 4) + e % 4
  // + 4 (lane / 32); 16 x 16 blocks: rows e + 4 (lane / 16))
  const int lrow = kM16 ? 4 * (lane >> 4) : 4 * (lane >> 5);
  const int lcol = lane & (kEdge - 1);
  auto erow = [](int e) { return kM16 ? e : 8 * (e >> 2) + (e & 3); };
  if (kF32Out && half >= 0) {
    // one half of a split tile: add into the zeroed output (two additions
    // onto zero give the same sum in either order)
#pragma unroll
    for (int i = 0; i < kFM; ++i)
#pragma unroll
      for (int j = 0; j < kFN; ++j) {
        const int64_t c = n0 + wn * kTN + j * kEdge + lcol;
#pragma unroll
        for (int e = 0; e < kAccN; ++e) {
          const int64_t r = m0 + wm * kTM + i * kEdge + erow(e) + lrow;
          const float v = alpha_normal ? acc[i][j][e] * alpha : (float)((double)acc[i][j][e] * alpha_d);
          if (r < M && c < N) unsafeAtomicAdd(static_cast<float*>(y) + r * N + c, v);
        }
      }
    return;
  }
  const bool full_tile = m0 + kBM <= M && n0 + kBN <= N;
  if (full_tile && alpha_normal && N * es * kBM < 0xFFFFFFFFll) {
    char* tile_base = static_cast<char*>(y) + (m0 * N + n0) * es;
    const uint32_t lane_off = (uint32_t)(((wm * kTM + lrow) * N + wn * kTN + lcol) * es);
#pragma unroll
    for (int i = 0; i < kFM; ++i)
#pragma unroll
      for (int j = 0; j < kFN; ++j)
#pragma unroll
        for (int e = 0; e < kAccN; e += 2) {
          const uint32_t r0 = (uint32_t)(i * kEdge + erow(e));
          const uint32_t o0 = lane_off + (uint32_t)((r0 * N + j * kEdge) * es);
          const uint32_t o1 = o0 + (uint32_t)(N * es);
          const float v0 = acc[i][j][e] * alpha, v1 = acc[i][j][e + 1] * alpha;
          if (kF32Out) {
            *reinterpret_cast<float*>(tile_base + o0) = v0;
            *reinterpret_cast<float*>(tile_base + o1) = v1;
          } else {
            *reinterpret_cast<__bf16*>(tile_base + o0) = (__bf16)v0;
            *reinterpret_cast<__bf16*>(tile_base + o1) = (__bf16)v1;
          }
        }
    return;
  }
#pragma unroll
  for (int i = 0; i < kFM; ++i)
#pragma unroll
    for (int j = 0; j < kFN; ++j) {
      const int64_t c = n0 + wn * kTN + j * kEdge + lcol;
#pragma unroll
      for (int e = 0; e < kAccN; ++e) {
        const int64_t r = m0 + wm * kTM + i * kEdge + erow(e) + lrow;
        const float v = alpha_normal ? acc[i][j][e] * alpha : (float)((double)acc[i][j][e] * alpha_d);
        if (r < M && c < N) {
          if (kF32Out) {
            static_cast<float*>(y)[r * N + c] = v;
          } else {
            static_cast<__bf16*>(y)[r * N + c] = (__bf16)v;
          }
        }
      }
    }
}

// A workgroup runs the logical workgroups blockIdx.x, blockIdx.x + G, ...
// below nwg (G = gridDim.x, a multiple of 8). Hardware dispatch sends
// workgroup b to XCD b % 8, so each logical workgroup L still runs on XCD
// L % 8. Two tiles per workgroup save a dispatch and the workgroup's start
// per tile; the launcher picks that only where it keeps the number of tile
// rounds, and only for the default-format kernels.
template <int kBM, int kBN, bool kFullK, bool kF32Out, int kWavesM, int kWavesN, int kSwz, bool kProbe,
          bool kFmt, bool kK64>
__global__ __launch_bounds__(64 * kWavesM * kWavesN) void gemm_kernel(
    const uint8_t* __restrict__ a_codes, const uint8_t* __restrict__ a_scales, int a_shift,
    const float* __restrict__ a_S, const uint8_t* __restrict__ b_codes,
    const uint8_t* __restrict__ b_scales, int b_shift, const float* __restrict__ b_S, int64_t M,
    int64_t N, int64_t K, int tiles_m, int tiles_n, int snap_log2, int fmt, int split_local,
    void* __restrict__ y, int nwg) {
  if constexpr (kFmt || kProbe) {
    // one tile per workgroup (the format-generic kernel would pass 256
    // VGPRs inside a tile loop); the grid is rounded up to a multiple of 8,
    // so workgroups past the last logical one have no tile
    if ((int)blockIdx.x >= nwg) return;
    gemm_tile<kBM, kBN, kFullK, kF32Out, kWavesM, kWavesN, kSwz, kProbe, kFmt, kK64, false>(
        a_codes, a_scales, a_shift, a_S, b_codes, b_scales, b_shift, b_S, M, N, K, tiles_m, tiles_n,
        snap_log2, fmt, split_local, y, (int)blockIdx.x, (int)threadIdx.x, nullptr);
  } else {
    extern __shared__ uint4 lds[];
    for (int L = blockIdx.x; L < nwg; L += gridDim.x) {
      // the thread index, opaque per tile, keeps the lane arithmetic inside
      // the loop (hoisted out of it, its values stay live through the k
      // loop and spill)
      int tid = threadIdx.x;
      asm volatile("" : "+v"(tid));
      gemm_tile<kBM, kBN, kFullK, kF32Out, kWavesM, kWavesN, kSwz, kProbe, kFmt, kK64, true>(
          a_codes, a_scales, a_shift, a_S, b_codes, b_scales, b_shift, b_S, M, N, K, tiles_m, tiles_n,
          snap_log2, fmt, split_local, y, L, tid, lds);
      lds_barrier();  // every wave is done with this tile's LDS buffers
    }
  }
}

// Zeroes the fp32 output tiles that split workgroups add into: workgroup j
// takes split tile j (nsplit of them per XCD range); each wave writes whole
// tile rows, 16 bytes per lane (y is 16-byte aligned and N % 4 == 0).
__global__ __launch_bounds__(256) void zero_split_tiles(float* __restrict__ y, int64_t M, int64_t N,
                                                        int tiles_m, int tiles_n, int per_xcd,
                                                        int split_local, int nsplit, int bm, int bn) {
  const int xcd = blockIdx.x / nsplit;
  const int t = xcd * per_xcd + split_local + (int)(blockIdx.x % nsplit);
  int tm, tn;
  tile_coords(t, tiles_m, tiles_n, &tm, &tn);
  const int64_t m0 = (int64_t)tm * bm;
  const int64_t c = (int64_t)tn * bn + 4 * (threadIdx.x & 63);
  const bool cv = c < N && 4 * (int)(threadIdx.x & 63) < bn;
  for (int r = threadIdx.x >> 6; r < bm; r += 4) {
    if (cv && m0 + r < M)
      *reinterpret_cast<float4*>(y + (m0 + r) * N + c) = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
  }
}

}  // namespace

// Kernel configuration, chosen at build time: 2 x 4 waves (two per SIMD, so
// one wave's MFMAs overlap the other's decode and LDS traffic; 128 x 64
// accumulators each) and the padded 144-byte LDS row pitch, the fastest of
// the measured variants (2x2 / 2x4 / 4x2 waves; XOR or padded layouts).
#ifndef FP4Q_GEMM_WAVES_M
#define FP4Q_GEMM_WAVES_M 2
#endif
#ifndef FP4Q_GEMM_WAVES_N
#define FP4Q_GEMM_WAVES_N 4
#endif

namespace {

// Per-device facts the launcher needs, looked up once per device and kept
// in lock-free caches (a race only repeats an idempotent lookup).
constexpr int kMaxDevices = 64;

// Workgroups of the default kernel that run at once on device dev: one per
// compute unit (its LDS use allows one per CU).
int concurrent_workgroups(int dev) {
  static std::atomic<int> cache[kMaxDevices];
  if (dev < 0 || dev >= kMaxDevices) dev = 0;
  int cus = cache[dev].load(std::memory_order_relaxed);
  if (cus > 0) return cus;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0)
    cus = 256;
  cache[dev].store(cus, std::memory_order_relaxed);
  return cus;
}

// The dynamic LDS limit of kernel fn on device dev, raised once per
// (kernel, device): one bit per device in a mask kept per kernel.
hipError_t allow_lds(const void* fn, int dev, int bytes) {
  struct Entry {
    std::atomic<const void*> fn;
    std::atomic<uint64_t> devs;
  };
  static Entry table[64];
  const uint64_t bit = (dev >= 0 && dev < kMaxDevices) ? (uint64_t(1) << dev) : 0;
  Entry* e = nullptr;
  for (Entry& t : table) {
    const void* cur = t.fn.load(std::memory_order_acquire);
    if (cur == fn) { e = &t; break; }
    if (cur == nullptr) {
      const void* expected = nullptr;
      if (t.fn.compare_exchange_strong(expected, fn, std::memory_order_acq_rel) || expected == fn) {
        e = &t;
        break;
      }
    }
  }
  if (e && bit && (e->devs.load(std::memory_order_acquire) & bit)) return hipSuccess;
  const hipError_t err = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, bytes);
  if (err == hipSuccess && e && bit) e->devs.fetch_or(bit, std::memory_order_acq_rel);
  return err;
}

template <int kBM, int kBN, int kWM, int kWN, int kSW, bool kProbe, bool kFmt>
hipError_t launch_kernel(const QOperand& a, const QOperand& b, void* y, int y_es, int snap_log2,
                         int fmt, hipStream_t s) {
  // operands share the packing (checked by the caller); K64 implies K % 64 == 0
  const bool k64 = a.pack != 0;
  const int64_t M = a.rows, N = b.rows, K = a.cols;
  const int tiles_m = (int)((M + kBM - 1) / kBM);
  const int tiles_n = (int)((N + kBN - 1) / kBN);
  const bool full_k = K % BK == 0;
  // layouts 2 and 3 (whose 32 x 32 kernels use 2) take the padded size
  const size_t lds_bytes = 2 * (kBM + kBN) * (kSW >= 2 ? kChunks + 1 : kChunks) * sizeof(uint4);
  const void* fn;
  if (k64)
    fn = y_es == 4 ? (const void*)gemm_kernel<kBM, kBN, true, true, kWM, kWN, kSW, kProbe, kFmt, true>
                   : (const void*)gemm_kernel<kBM, kBN, true, false, kWM, kWN, kSW, kProbe, kFmt, true>;
  else if (full_k)
    fn = y_es == 4 ? (const void*)gemm_kernel<kBM, kBN, true, true, kWM, kWN, kSW, kProbe, kFmt, false>
                   : (const void*)gemm_kernel<kBM, kBN, true, false, kWM, kWN, kSW, kProbe, kFmt, false>;
  else
    fn = y_es == 4 ? (const void*)gemm_kernel<kBM, kBN, false, true, kWM, kWN, kSW, kProbe, kFmt, false>
                   : (const void*)gemm_kernel<kBM, kBN, false, false, kWM, kWN, kSW, kProbe, kFmt, false>;
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  e = allow_lds(fn, dev, (int)lds_bytes);
  if (e != hipSuccess) return e;
  // split tail: when the tiles fill the last round of workgroups at most
  // half way, run each of those tiles as two K halves (fp32 output only)
  const int ntiles = tiles_m * tiles_n;
  const int nk = (int)((K + BK - 1) / BK);
  const int per_xcd = (ntiles + 7) / 8;
  int split_local = -1;
  const int cwg = (!kProbe && y_es == 4) ? concurrent_workgroups(dev) : 1;  // one per CU
  const int rem = ntiles % cwg;
#ifndef FP4Q_NO_SPLIT_TAIL
  if (!kProbe && y_es == 4 && ntiles % 8 == 0 && rem > 0 && rem % 8 == 0 && 2 * rem <= cwg && nk >= 2 &&
      reinterpret_cast<uintptr_t>(y) % 16 == 0 && N % 4 == 0 && kBN <= 256)
    split_local = per_xcd - rem / 8;
#endif
  const int nwg = split_local < 0 ? ntiles : 8 * (split_local + 2 * (per_xcd - split_local));
  if (split_local >= 0) {
    const int nsplit = per_xcd - split_local;
    hipLaunchKernelGGL(zero_split_tiles, dim3((uint32_t)(8 * nsplit)), dim3(256), 0, s,
                       static_cast<float*>(y), M, N, tiles_m, tiles_n, per_xcd, split_local, nsplit,
                       kBM, kBN);
  }
  // two tiles per workgroup where the tile rounds stay as many (one
  // workgroup of this kernel per CU at a time)
  int rep = 1;
  if (!kProbe && !kFmt) {
    const int64_t cw = concurrent_workgroups(dev);
    const int64_t rounds1 = (nwg + cw - 1) / cw;
    const int64_t phys2 = 8 * (((nwg + 7) / 8 + 1) / 2);
    if (2 * ((phys2 + cw - 1) / cw) <= rounds1) rep = 2;
  }
  const int per_xcd_wg = (nwg + 7) / 8;
  const dim3 grid((uint32_t)(8 * ((per_xcd_wg + rep - 1) / rep))), block(64 * kWM * kWN);
  const int a_shift = a.tile ? (a.block == 32 ? 5 : 4) : 0;
  const int b_shift = b.tile ? (b.block == 32 ? 5 : 4) : 0;
#define FP4Q_GEMM(FK, F32, K64)                                                                     \
  hipLaunchKernelGGL((gemm_kernel<kBM, kBN, FK, F32, kWM, kWN, kSW, kProbe, kFmt, K64>), grid, block, \
                     lds_bytes, s, a.codes, a.scales, a_shift, a.enc_scale, b.codes, b.scales,         \
                     b_shift, b.enc_scale, M, N, K, tiles_m, tiles_n, snap_log2, fmt, split_local, y, nwg)
  if (k64) {
    if (y_es == 4) FP4Q_GEMM(true, true, true);
    else FP4Q_GEMM(true, false, true);
  } else if (full_k) {
    if (y_es == 4) FP4Q_GEMM(true, true, false);
    else FP4Q_GEMM(true, false, false);
  } else {
    if (y_es == 4) FP4Q_GEMM(false, true, false);
    else FP4Q_GEMM(false, false, false);
  }
#undef FP4Q_GEMM
  return hipGetLastError();
}

// Operands in the default format (blocks of 16, UE5M3) take kernels
// compiled for it; any other combination takes the format-generic ones.
template <int kBM, int kBN, int kWM, int kWN, int kSW, bool kProbe>
hipError_t launch_tiled(const QOperand& a, const QOperand& b, void* y, int y_es, int snap_log2,
                        hipStream_t s) {
  if (a.rows == 0 || b.rows == 0) return hipSuccess;
  const int fmt = (a.block == 32 ? 1 : 0) | (a.scale_fmt ? 2 : 0) | (b.block == 32 ? 4 : 0) |
                  (b.scale_fmt ? 8 : 0);
  if (fmt == 0) return launch_kernel<kBM, kBN, kWM, kWN, kSW, kProbe, false>(a, b, y, y_es, snap_log2, 0, s);
  return launch_kernel<kBM, kBN, kWM, kWN, kSW, kProbe, true>(a, b, y, y_es, snap_log2, fmt, s);
}

}  // namespace

hipError_t launch_gemm(const QOperand& a, const QOperand& b, void* y, int y_es, hipStream_t s) {
  return launch_tiled<BM, BN, FP4Q_GEMM_WAVES_M, FP4Q_GEMM_WAVES_N, FP4Q_GEMM_SWZ, false>(a, b, y, y_es,
                                                                                         0, s);
}

// Probe mode: 128 x 128 tiles of 2 x 2 waves (64 x 64 each), so that the
// slice accumulators and the running sums both stay in registers.
hipError_t launch_gemm_probe(const QOperand& a, const QOperand& b, void* y, int y_es, int snap_log2,
                             hipStream_t s) {
  return launch_tiled<kPM, kPM, 2, 2, 2, true>(a, b, y, y_es, snap_log2, s);
}

}  // namespace fp4q
