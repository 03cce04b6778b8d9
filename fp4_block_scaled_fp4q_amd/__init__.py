"""MI355X-native block-scaled FP4 (E2M1 + UE5M3 + FP32 tensor scale) linear layer.

The computation lives in libfp4q.so (HIP kernels for gfx950 behind the C ABI
of include/fp4q.h). ``api`` is its torch-facing binding; ``inputs`` holds the
seeded synthetic workload generators. The library is loaded on first use, so
importing the package works on a machine without a GPU.
"""
__all__ = ["api", "inputs"]
