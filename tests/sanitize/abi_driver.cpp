// Drives every entry point of the C ABI (include/fp4q.h), built for the host
// with the launchers stubbed out, through valid calls and every class of
// invalid argument: NULL pointers, unknown enums, misaligned pointers and
// strides, negative, ragged and huge sizes (up to and past the 2^40 / 2^44
// limits, where products of sizes would overflow 64 bits without the
// validation's guards). Device pointers are fake addresses: the validation
// layer checks them, it never dereferences them. Expected statuses are
// asserted; the sanitizers report any overflow or out-of-range access in the
// validation arithmetic.
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <initializer_list>

#include "fp4q.h"

extern int g_launches;

static int g_fail = 0;
static void expect(fp4q_status got, fp4q_status want, const char* what) {
  if (got != want) {
    std::fprintf(stderr, "%s: status %d (%s), expected %d\n", what, (int)got, fp4q_status_str(got), (int)want);
    g_fail = 1;
  }
}

static void* fake(uintptr_t a) { return reinterpret_cast<void*>(a); }

static fp4q_qtensor operand(int64_t rows, int64_t cols, fp4q_layout layout, int32_t block = 16,
                            int32_t pack = FP4Q_PACK_ROWS) {
  fp4q_qtensor q;
  q.codes = static_cast<const uint8_t*>(fake(0x100000));
  q.scales = static_cast<const uint8_t*>(fake(0x200000));
  q.enc_scale = static_cast<const float*>(fake(0x300000));
  q.rows = rows;
  q.cols = cols;
  q.layout = layout;
  q.block = block;
  q.scale_fmt = FP4Q_UE5M3;
  q.pack = pack;
  return q;
}

int main() {
  const void* x = fake(0x400000);
  float* amax = static_cast<float*>(fake(0x500000));
  uint8_t* codes = static_cast<uint8_t*>(fake(0x600000));
  uint8_t* scales = static_cast<uint8_t*>(fake(0x700000));
  uint8_t* codes_t = static_cast<uint8_t*>(fake(0x800000));
  uint8_t* scales_t = static_cast<uint8_t*>(fake(0x900000));
  void* y = fake(0xA00000);
  const int64_t big = int64_t(1) << 40, huge = int64_t(1) << 62, neg = -16;

  expect(fp4q_abi_version() == FP4Q_ABI_VERSION ? FP4Q_OK : FP4Q_E_ARG, FP4Q_OK, "abi version");
  for (int s = -1; s <= 8; ++s) (void)fp4q_status_str((fp4q_status)s);

  // ---- amax
  expect(fp4q_amax(x, FP4Q_BF16, 64, 256, 256, amax, nullptr), FP4Q_OK, "amax");
  expect(fp4q_amax(x, FP4Q_F32, 0, 0, 0, amax, nullptr), FP4Q_OK, "amax empty");
  expect(fp4q_amax(x, (fp4q_dtype)7, 64, 256, 256, amax, nullptr), FP4Q_E_DTYPE, "amax dtype");
  expect(fp4q_amax(nullptr, FP4Q_BF16, 64, 256, 256, amax, nullptr), FP4Q_E_NULL, "amax x");
  expect(fp4q_amax(x, FP4Q_BF16, 64, 256, 256, nullptr, nullptr), FP4Q_E_NULL, "amax out");
  expect(fp4q_amax(x, FP4Q_BF16, 64, 256, 128, amax, nullptr), FP4Q_E_SHAPE, "amax ld < cols");
  expect(fp4q_amax(x, FP4Q_BF16, neg, 256, 256, amax, nullptr), FP4Q_E_SHAPE, "amax negative rows");
  expect(fp4q_amax(x, FP4Q_BF16, big, big, big, amax, nullptr), FP4Q_E_SHAPE, "amax 2^80 elements");
  expect(fp4q_amax(x, FP4Q_BF16, huge, 16, 16, amax, nullptr), FP4Q_E_SHAPE, "amax 2^62 rows");
  expect(fp4q_amax(x, FP4Q_BF16, 16, huge, huge, amax, nullptr), FP4Q_E_SHAPE, "amax 2^62 cols");
  expect(fp4q_amax(fake(0x400002), FP4Q_BF16, 64, 256, 256, amax, nullptr), FP4Q_E_ALIGN, "amax x align");
  expect(fp4q_amax(x, FP4Q_BF16, 64, 252, 252, amax, nullptr), FP4Q_E_ALIGN, "amax row bytes");
  expect(fp4q_amax(x, FP4Q_BF16, 64, 256, 256, static_cast<float*>(fake(0x500002)), nullptr), FP4Q_E_ALIGN,
         "amax out align");

  // ---- quantize: every layout, rounding, block, format and packing, then
  // each invalid argument in turn
  const fp4q_layout layouts[] = {FP4Q_ROW16, FP4Q_COL16, FP4Q_TILE16x16};
  for (fp4q_layout L : layouts)
    for (int rnd = 0; rnd < 2; ++rnd)
      for (int32_t blk : {16, 32})
        for (int fmt = 0; fmt < 2; ++fmt)
          for (int32_t pack : {FP4Q_PACK_ROWS, FP4Q_PACK_K64})
            for (int dt = 0; dt < 2; ++dt) {
              const bool second = L != FP4Q_COL16;
              expect(fp4q_quantize_fmt(x, (fp4q_dtype)dt, 128, 256, 264, amax, 448.0f, L, blk, (fp4q_scale_fmt)fmt,
                                       pack, (fp4q_round)rnd, 7, 3, codes, scales, amax,
                                       second ? codes_t : nullptr, second ? scales_t : nullptr,
                                       reinterpret_cast<int32_t*>(fake(0xB00000)), nullptr),
                     FP4Q_OK, "quantize valid");
            }
  auto q = [&](int64_t r, int64_t c, int64_t ld, fp4q_layout L, int32_t blk, int32_t pack, const void* xx,
               uint8_t* ct, uint8_t* st, float T = 448.0f) {
    return fp4q_quantize_fmt(xx, FP4Q_BF16, r, c, ld, amax, T, L, blk, FP4Q_UE5M3, pack, FP4Q_RNE, 0, 0, codes,
                             scales, nullptr, ct, st, nullptr, nullptr);
  };
  expect(q(0, 0, 0, FP4Q_ROW16, 16, 0, x, nullptr, nullptr), FP4Q_OK, "quantize empty");
  expect(q(48, 1040, 1040, FP4Q_ROW16, 16, 0, x, nullptr, nullptr), FP4Q_OK, "quantize ragged rows");
  expect(q(48, 1048, 1048, FP4Q_COL16, 16, 0, x, nullptr, nullptr), FP4Q_OK, "quantize col16 ragged cols");
  expect(q(48, 1048, 1048, FP4Q_ROW16, 16, 0, x, nullptr, nullptr), FP4Q_E_SHAPE, "row16 ragged cols");
  expect(q(40, 1040, 1040, FP4Q_TILE16x16, 16, 0, x, nullptr, nullptr), FP4Q_E_SHAPE, "tile ragged rows");
  expect(q(48, 1040, 1040, FP4Q_ROW16, 16, 0, x, codes_t, scales_t), FP4Q_OK, "row16 + col16");
  expect(q(40, 1040, 1040, FP4Q_ROW16, 16, 0, x, codes_t, scales_t), FP4Q_E_SHAPE, "row16 + col16 ragged rows");
  expect(q(48, 1040, 1040, FP4Q_ROW16, 16, 0, x, codes_t, nullptr), FP4Q_E_ARG, "codes_t without scales_t");
  expect(q(48, 1040, 1040, FP4Q_COL16, 16, 0, x, codes_t, scales_t), FP4Q_E_ARG, "col16 with a second output");
  expect(q(64, 1040, 1040, FP4Q_ROW16, 16, FP4Q_PACK_K64, x, nullptr, nullptr), FP4Q_E_SHAPE, "k64 ragged K");
  expect(q(48, 1024, 1024, FP4Q_ROW16, 16, FP4Q_PACK_K64, x, codes_t, scales_t), FP4Q_E_SHAPE, "k64 ragged M");
  expect(q(48, 1040, 1040, FP4Q_ROW16, 24, 0, x, nullptr, nullptr), FP4Q_E_ARG, "block 24");
  expect(q(48, 1040, 1040, FP4Q_ROW16, 16, 5, x, nullptr, nullptr), FP4Q_E_ARG, "packing 5");
  expect(q(48, 1040, 1040, (fp4q_layout)9, 16, 0, x, nullptr, nullptr), FP4Q_E_ARG, "layout 9");
  expect(q(48, 1040, 1040, FP4Q_ROW16, 16, 0, x, nullptr, nullptr, 0.0f), FP4Q_E_ARG, "target 0");
  expect(q(48, 1040, 1040, FP4Q_ROW16, 16, 0, x, nullptr, nullptr, -1.0f), FP4Q_E_ARG, "target < 0");
  expect(q(48, 1040, 1040, FP4Q_ROW16, 16, 0, x, nullptr, nullptr, 1.0f / 0.0f), FP4Q_E_ARG, "target inf");
  expect(q(48, 1040, 1032, FP4Q_ROW16, 16, 0, x, nullptr, nullptr), FP4Q_E_SHAPE, "ld < cols");
  expect(q(48, 1040, 1041, FP4Q_ROW16, 16, 0, x, nullptr, nullptr), FP4Q_E_ALIGN, "odd ld");
  expect(q(48, 1040, 1040, FP4Q_ROW16, 16, 0, fake(0x400008), nullptr, nullptr), FP4Q_E_ALIGN, "x align");
  expect(q(48, 1040, 1040, FP4Q_ROW16, 16, 0, nullptr, nullptr, nullptr), FP4Q_E_NULL, "x null");
  expect(q(big, big, big, FP4Q_ROW16, 16, 0, x, nullptr, nullptr), FP4Q_E_SHAPE, "2^80 elements");
  expect(q(huge, 16, 16, FP4Q_ROW16, 16, 0, x, nullptr, nullptr), FP4Q_E_SHAPE, "2^62 rows");
  expect(q(16, huge, huge, FP4Q_COL16, 16, 0, x, nullptr, nullptr), FP4Q_E_SHAPE, "2^62 cols");
  expect(q(int64_t(1) << 30, int64_t(1) << 13, int64_t(1) << 13, FP4Q_ROW16, 16, 0, x, nullptr, nullptr),
         FP4Q_E_SHAPE, "grid beyond 2^31 threads");
  expect(q(neg, 64, 64, FP4Q_ROW16, 16, 0, x, nullptr, nullptr), FP4Q_E_SHAPE, "negative rows");
  expect(fp4q_quantize_fmt(x, FP4Q_BF16, 48, 1040, 1040, nullptr, 448.0f, FP4Q_ROW16, 16, FP4Q_UE5M3, 0,
                           FP4Q_RNE, 0, 0, codes, scales, nullptr, nullptr, nullptr, nullptr, nullptr),
         FP4Q_E_NULL, "held amax null");
  expect(fp4q_quantize_fmt(x, FP4Q_BF16, 48, 1040, 1040, static_cast<const float*>(fake(0x500001)), 448.0f,
                           FP4Q_ROW16, 16, FP4Q_UE5M3, 0, FP4Q_RNE, 0, 0, codes, scales, nullptr, nullptr,
                           nullptr, nullptr, nullptr),
         FP4Q_E_ALIGN, "held amax align");
  expect(fp4q_quantize_fmt(x, FP4Q_BF16, 48, 1040, 1040, amax, 448.0f, FP4Q_ROW16, 16, (fp4q_scale_fmt)4, 0,
                           FP4Q_RNE, 0, 0, codes, scales, nullptr, nullptr, nullptr, nullptr, nullptr),
         FP4Q_E_ARG, "scale format 4");
  expect(fp4q_quantize_fmt(x, FP4Q_BF16, 48, 1040, 1040, amax, 448.0f, FP4Q_ROW16, 16, FP4Q_UE5M3, 0,
                           (fp4q_round)3, 0, 0, codes, scales, nullptr, nullptr, nullptr, nullptr, nullptr),
         FP4Q_E_ARG, "rounding 3");
  expect(fp4q_quantize(x, FP4Q_F32, 48, 1040, 1040, amax, 448.0f, FP4Q_TILE16x16, FP4Q_SR, 1, 2, codes, scales,
                       amax, codes_t, scales_t, reinterpret_cast<int32_t*>(fake(0xB00002)), nullptr),
         FP4Q_E_ALIGN, "diag align");

  // ---- dequant
  fp4q_qtensor a = operand(300, 1040, FP4Q_ROW16);
  expect(fp4q_dequant(&a, y, FP4Q_BF16, nullptr), FP4Q_OK, "dequant");
  expect(fp4q_dequant(nullptr, y, FP4Q_BF16, nullptr), FP4Q_E_NULL, "dequant null operand");
  expect(fp4q_dequant(&a, nullptr, FP4Q_BF16, nullptr), FP4Q_E_NULL, "dequant null output");
  expect(fp4q_dequant(&a, fake(0xA00004), FP4Q_F32, nullptr), FP4Q_E_ALIGN, "dequant output align");
  expect(fp4q_dequant(&a, y, (fp4q_dtype)5, nullptr), FP4Q_E_DTYPE, "dequant dtype");
  fp4q_qtensor hb = operand(big, big, FP4Q_ROW16);
  expect(fp4q_dequant(&hb, y, FP4Q_F32, nullptr), FP4Q_E_SHAPE, "dequant 2^80 elements");

  // ---- GEMMs
  for (int32_t pack : {FP4Q_PACK_ROWS, FP4Q_PACK_K64}) {
    fp4q_qtensor xa = operand(300, 1088, FP4Q_ROW16, 16, pack), wb = operand(272, 1088, FP4Q_TILE16x16, 16, pack);
    for (int yt = 0; yt < 2; ++yt) {
      expect(fp4q_linear_fwd(&xa, &wb, y, (fp4q_dtype)yt, nullptr), FP4Q_OK, "fwd");
      expect(fp4q_linear_dgrad(&xa, &wb, y, (fp4q_dtype)yt, nullptr), FP4Q_OK, "dgrad");
      expect(fp4q_linear_wgrad(&xa, &wb, y, (fp4q_dtype)yt, nullptr), FP4Q_OK, "wgrad");
      for (int32_t snap : {0, 10, 30}) expect(fp4q_linear_probe(&xa, &wb, y, (fp4q_dtype)yt, snap, nullptr), FP4Q_OK, "probe");
    }
  }
  fp4q_qtensor xa = operand(300, 1088, FP4Q_ROW16), wb = operand(272, 1088, FP4Q_TILE16x16);
  fp4q_qtensor wk = operand(272, 1024, FP4Q_TILE16x16);
  expect(fp4q_linear_fwd(&xa, &wk, y, FP4Q_BF16, nullptr), FP4Q_E_SHAPE, "contraction mismatch");
  fp4q_qtensor xr = operand(300, 1040, FP4Q_ROW16), wp = operand(272, 1040, FP4Q_TILE16x16, 16, FP4Q_PACK_K64);
  expect(fp4q_linear_fwd(&xr, &wp, y, FP4Q_BF16, nullptr), FP4Q_E_SHAPE, "k64 ragged contraction");
  fp4q_qtensor wp2 = operand(272, 1024, FP4Q_TILE16x16, 16, FP4Q_PACK_K64), xa2 = operand(300, 1024, FP4Q_ROW16);
  expect(fp4q_linear_fwd(&xa2, &wp2, y, FP4Q_BF16, nullptr), FP4Q_E_ARG, "packing mismatch");
  expect(fp4q_linear_fwd(&xa, &wb, nullptr, FP4Q_BF16, nullptr), FP4Q_E_NULL, "null output");
  expect(fp4q_linear_fwd(nullptr, &wb, y, FP4Q_BF16, nullptr), FP4Q_E_NULL, "null operand");
  expect(fp4q_linear_fwd(&xa, &wb, fake(0xA00002), FP4Q_F32, nullptr), FP4Q_E_ALIGN, "output align");
  expect(fp4q_linear_fwd(&xa, &wb, y, (fp4q_dtype)3, nullptr), FP4Q_E_DTYPE, "output dtype");
  expect(fp4q_linear_probe(&xa, &wb, y, FP4Q_F32, 31, nullptr), FP4Q_E_ARG, "snap 31");
  expect(fp4q_linear_probe(&xa, &wb, y, FP4Q_F32, -1, nullptr), FP4Q_E_ARG, "snap -1");
  fp4q_qtensor t40 = operand(40, 1088, FP4Q_TILE16x16);
  expect(fp4q_linear_fwd(&xa, &t40, y, FP4Q_F32, nullptr), FP4Q_E_SHAPE, "tile rows not whole blocks");
  fp4q_qtensor b32 = operand(272, 1040, FP4Q_ROW16, 32);
  expect(fp4q_linear_fwd(&xr, &b32, y, FP4Q_F32, nullptr), FP4Q_E_SHAPE, "block 32 ragged contraction");
  fp4q_qtensor bad = operand(272, 1088, FP4Q_ROW16);
  bad.codes = static_cast<const uint8_t*>(fake(0x100004));
  expect(fp4q_linear_fwd(&xa, &bad, y, FP4Q_F32, nullptr), FP4Q_E_ALIGN, "codes align");
  bad = operand(272, 1088, FP4Q_ROW16);
  bad.enc_scale = nullptr;
  expect(fp4q_linear_fwd(&xa, &bad, y, FP4Q_F32, nullptr), FP4Q_E_NULL, "null tensor scale");
  bad = operand(272, 1088, FP4Q_ROW16);
  bad.layout = FP4Q_COL16;
  expect(fp4q_linear_fwd(&xa, &bad, y, FP4Q_F32, nullptr), FP4Q_E_ARG, "col16 operand");
  fp4q_qtensor hx = operand(big, 1088, FP4Q_ROW16), hw = operand(big, 1088, FP4Q_ROW16);
  expect(fp4q_linear_fwd(&hx, &hw, y, FP4Q_F32, nullptr), FP4Q_E_SHAPE, "2^80 tiles");
  fp4q_qtensor ha = operand(huge, huge, FP4Q_ROW16);
  expect(fp4q_linear_fwd(&ha, &ha, y, FP4Q_F32, nullptr), FP4Q_E_SHAPE, "2^62 x 2^62 operand");
  fp4q_qtensor e0 = operand(0, 1088, FP4Q_ROW16);
  expect(fp4q_linear_fwd(&e0, &wb, nullptr, FP4Q_F32, nullptr), FP4Q_OK, "empty M with no output");

  if (g_launches == 0) {
    std::fprintf(stderr, "no launcher was reached\n");
    g_fail = 1;
  }
  std::printf("abi driver: %d launches, %s\n", g_launches, g_fail ? "FAILED" : "ok");
  return g_fail;
}
