"""ctypes binding of libfp4q.so (the C ABI declared in include/fp4q.h).

Argument marshalling only: torch tensors supply device pointers, strides and
the current HIP stream; every step of the computation runs in the HIP
kernels of the library. There is no fallback: if the library is missing or
cannot be loaded, every call raises.
"""
from __future__ import annotations

import ctypes
import os

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libfp4q.so")

# status codes (fp4q_status)
OK, E_NULL, E_SHAPE, E_ALIGN, E_DTYPE, E_ARG, E_HIP = range(7)
# enums
F32, BF16 = 0, 1
RNE, SR = 0, 1
ROW16, COL16, TILE16x16 = 0, 1, 2
UE5M3, E4M3 = 0, 1
PACK_ROWS, PACK_K64 = 0, 1

# every entry point include/fp4q.h declares
EXPORTS = ("fp4q_abi_version", "fp4q_status_str", "fp4q_amax", "fp4q_quantize", "fp4q_quantize_fmt",
           "fp4q_dequant", "fp4q_linear_fwd", "fp4q_linear_dgrad", "fp4q_linear_wgrad",
           "fp4q_linear_probe")


class QTensorC(ctypes.Structure):
    """fp4q_qtensor."""
    _fields_ = [("codes", ctypes.c_void_p), ("scales", ctypes.c_void_p),
                ("enc_scale", ctypes.c_void_p), ("rows", ctypes.c_int64),
                ("cols", ctypes.c_int64), ("layout", ctypes.c_int32), ("block", ctypes.c_int32),
                ("scale_fmt", ctypes.c_int32), ("pack", ctypes.c_int32)]


class Fp4qError(RuntimeError):
    def __init__(self, fn: str, status: int, msg: str):
        super().__init__(f"{fn}: {msg} (status {status})")
        self.status = status


_lib = None


def lib() -> ctypes.CDLL:
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is not built; run __graft_entry__.build() "
                          "(or python -m fp4_block_scaled_fp4q_amd.build)")
    L = ctypes.CDLL(LIB_PATH)
    p, i64, i32, u64, u32, f = (ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32, ctypes.c_uint64,
                                ctypes.c_uint32, ctypes.c_float)
    qp = ctypes.POINTER(QTensorC)
    L.fp4q_abi_version.restype = ctypes.c_int
    L.fp4q_abi_version.argtypes = []
    L.fp4q_status_str.restype = ctypes.c_char_p
    L.fp4q_status_str.argtypes = [ctypes.c_int]
    L.fp4q_amax.restype = ctypes.c_int
    L.fp4q_amax.argtypes = [p, ctypes.c_int, i64, i64, i64, p, p]
    L.fp4q_quantize.restype = ctypes.c_int
    L.fp4q_quantize.argtypes = [p, ctypes.c_int, i64, i64, i64, p, f, ctypes.c_int, ctypes.c_int,
                                u64, u32, p, p, p, p, p, p, p]
    L.fp4q_quantize_fmt.restype = ctypes.c_int
    L.fp4q_quantize_fmt.argtypes = [p, ctypes.c_int, i64, i64, i64, p, f, ctypes.c_int, i32, ctypes.c_int,
                                    i32, ctypes.c_int, u64, u32, p, p, p, p, p, p, p]
    L.fp4q_dequant.restype = ctypes.c_int
    L.fp4q_dequant.argtypes = [qp, p, ctypes.c_int, p]
    for name in ("fp4q_linear_fwd", "fp4q_linear_dgrad", "fp4q_linear_wgrad"):
        fn = getattr(L, name)
        fn.restype = ctypes.c_int
        fn.argtypes = [qp, qp, p, ctypes.c_int, p]
    L.fp4q_linear_probe.restype = ctypes.c_int
    L.fp4q_linear_probe.argtypes = [qp, qp, p, ctypes.c_int, ctypes.c_int32, p]
    _lib = L
    return L


def check(fn: str, status: int) -> None:
    if status != OK:
        msg = lib().fp4q_status_str(status).decode()
        raise Fp4qError(fn, status, msg)
