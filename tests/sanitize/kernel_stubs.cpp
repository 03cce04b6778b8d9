// Host-only stand-ins for the launchers of libfp4q.so's kernels, so that the
// C ABI layer (csrc/api.cpp) can be built for the host alone under the
// address and undefined-behaviour sanitizers and driven with every kind of
// argument. Each stub checks what the validation layer guarantees to its
// launcher and counts its calls; nothing is launched.
#include <cstdio>
#include <cstdlib>

#include "kernels.h"

int g_launches = 0;

static void require(bool ok, const char* what) {
  if (!ok) {
    std::fprintf(stderr, "launcher precondition violated: %s\n", what);
    std::abort();
  }
}

namespace fp4q {

hipError_t launch_amax(const void* x, int es, int64_t rows, int64_t cols, int64_t ld, float* out, hipStream_t) {
  require(es == 2 || es == 4, "amax element size");
  require(rows >= 0 && cols >= 0 && ld >= cols, "amax shape");
  require(out != nullptr, "amax output");
  require(rows == 0 || cols == 0 || x != nullptr, "amax input");
  ++g_launches;
  return hipSuccess;
}

hipError_t launch_quantize(const QuantArgs& a, hipStream_t) {
  require(a.es == 2 || a.es == 4, "quantize element size");
  require(a.rows >= 0 && a.cols >= 0 && a.ld >= a.cols, "quantize shape");
  require(a.block == 16 || a.block == 32, "quantize block");
  require(a.layout >= 0 && a.layout <= 2, "quantize layout");
  require(a.amax_held != nullptr, "quantize held amax");
  require(a.rows == 0 || a.cols == 0 || (a.x && a.codes && a.scales), "quantize buffers");
  ++g_launches;
  return hipSuccess;
}

hipError_t launch_dequant(const QOperand& q, void* out, int out_es, hipStream_t) {
  require(out_es == 2 || out_es == 4, "dequant element size");
  require(q.rows == 0 || q.cols == 0 || (out && q.codes && q.scales), "dequant buffers");
  ++g_launches;
  return hipSuccess;
}

hipError_t launch_gemm(const QOperand& a, const QOperand& b, void* y, int y_es, hipStream_t) {
  require(a.cols == b.cols, "gemm contraction");
  require(y_es == 2 || y_es == 4, "gemm element size");
  require(a.rows == 0 || b.rows == 0 || y != nullptr, "gemm output");
  ++g_launches;
  return hipSuccess;
}

hipError_t launch_gemm_probe(const QOperand& a, const QOperand& b, void* y, int y_es, int snap_log2,
                             hipStream_t s) {
  require(snap_log2 >= 0 && snap_log2 <= 30, "probe snap");
  return launch_gemm(a, b, y, y_es, s);
}

}  // namespace fp4q
