"""fp4q oracle: plain CPU reference for the block-scaled FP4 linear layer.

TEST INFRASTRUCTURE ONLY. The test suite, the package smoke check and the
benchmark's CPU-baseline leg are the only callers. Nothing in the product
package imports this module, and it imports nothing from the product package.

The codec (amax, tensor scale, UE5M3 block scales, E2M1 RNE/SR payloads,
Philox4x32-10, dequant) lives in ``fp4q_oracle.c`` (scalar binary32, no FMA
contraction). The GEMM is the plain definition of the emulated FP4 linear of
"UE5M3 FP4 Block Scaling for Stable Language Model Pretraining", §6: the
contraction of the exactly decoded operands, here in float64 with numpy, then
divided by the product of the two tensor scales.

Every function is pinned by tests under ``tests/test_oracle_*.py`` against
values the pages print, closed forms, library routines (numpy float16,
torch float8_e4m3fn) and brute force; see those files for which pin covers
which function.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from dataclasses import dataclass

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "fp4q_oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")

F32, BF16 = 0, 1
ROW16, COL16, TILE16 = 0, 1, 2   # blocks along a row, down a column, square tiles
RNE, SR = 0, 1
UE5M3, E4M3 = 0, 1               # block-scale formats


def build(force: bool = True) -> str:
    """Compile the oracle with gcc (plain IEEE binary32, no FMA contraction)."""
    stale = os.path.exists(_LIB) and os.path.getmtime(_SRC) > os.path.getmtime(_LIB)
    if force or stale or not os.path.exists(_LIB):
        tmp = _LIB + ".tmp"
        cmd = ["gcc", "-O2", "-std=gnu11", "-ffp-contract=off", "-fno-fast-math", "-frounding-math",
               "-fPIC", "-shared", "-o", tmp, _SRC, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _LIB)
    return _LIB


_lib = None


def lib():
    global _lib
    if _lib is None:
        path = build(force=False)
        L = ctypes.CDLL(path)
        c_i64, c_f, c_d, c_p = ctypes.c_int64, ctypes.c_float, ctypes.c_double, ctypes.c_void_p
        L.oracle_e2m1_decode.restype = c_d
        L.oracle_e2m1_decode.argtypes = [ctypes.c_int]
        L.oracle_ue5m3_decode.restype = c_d
        L.oracle_ue5m3_decode.argtypes = [ctypes.c_int]
        L.oracle_ue5m3_encode.restype = ctypes.c_int
        L.oracle_ue5m3_encode.argtypes = [c_f, ctypes.POINTER(ctypes.c_int)]
        L.oracle_ue5m3_nearest.restype = ctypes.c_int
        L.oracle_ue5m3_nearest.argtypes = [c_f]
        L.oracle_e4m3_decode.restype = c_d
        L.oracle_e4m3_decode.argtypes = [ctypes.c_int]
        L.oracle_e4m3_encode.restype = ctypes.c_int
        L.oracle_e4m3_encode.argtypes = [c_f, ctypes.POINTER(ctypes.c_int)]
        L.oracle_e2m1_encode_rne.restype = ctypes.c_int
        L.oracle_e2m1_encode_rne.argtypes = [c_f, ctypes.c_int]
        L.oracle_e2m1_encode_sr.restype = ctypes.c_int
        L.oracle_e2m1_encode_sr.argtypes = [c_f, ctypes.c_int, ctypes.c_uint32]
        L.oracle_philox4x32_10.restype = None
        L.oracle_philox4x32_10.argtypes = [c_p, c_p, c_p]
        L.oracle_sr_word.restype = ctypes.c_uint32
        L.oracle_sr_word.argtypes = [ctypes.c_uint64, ctypes.c_uint32, ctypes.c_uint64]
        L.oracle_amax.restype = c_f
        L.oracle_amax.argtypes = [c_p, ctypes.c_int, c_i64, c_i64, c_i64]
        L.oracle_tensor_scale.restype = c_f
        L.oracle_tensor_scale.argtypes = [c_f, c_f]
        L.oracle_quantize.restype = ctypes.c_int
        L.oracle_quantize.argtypes = [c_p, ctypes.c_int, c_i64, c_i64, c_i64, c_f, c_f,
                                      ctypes.c_int, ctypes.c_int, ctypes.c_uint64, ctypes.c_uint32,
                                      c_i64, c_i64, c_i64, c_p, c_p, c_p, c_p, c_p, c_p]
        L.oracle_quantize_fmt.restype = ctypes.c_int
        L.oracle_quantize_fmt.argtypes = [c_p, ctypes.c_int, c_i64, c_i64, c_i64, c_f, c_f, ctypes.c_int,
                                          ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_uint64,
                                          ctypes.c_uint32, c_i64, c_i64, c_i64, c_p, c_p, c_p, c_p, c_p, c_p]
        L.oracle_decode_f64_fmt.restype = None
        L.oracle_decode_f64_fmt.argtypes = [c_p, c_p, c_i64, c_i64, ctypes.c_int, ctypes.c_int, ctypes.c_int, c_p]
        L.oracle_dequant_f32_fmt.restype = None
        L.oracle_dequant_f32_fmt.argtypes = [c_p, c_p, c_i64, c_i64, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                             c_f, c_p]
        L.oracle_decode_f64.restype = None
        L.oracle_decode_f64.argtypes = [c_p, c_p, c_i64, c_i64, ctypes.c_int, c_p]
        L.oracle_dequant_f32.restype = None
        L.oracle_dequant_f32.argtypes = [c_p, c_p, c_i64, c_i64, ctypes.c_int, c_f, c_p]
        L.oracle_gemm_f64_loops.restype = None
        L.oracle_gemm_f64_loops.argtypes = [c_p, c_p, c_i64, c_i64, c_i64, c_d, c_d, c_p]
        L.oracle_gemm_probe.restype = ctypes.c_int
        L.oracle_gemm_probe.argtypes = [c_p, c_p, c_i64, c_i64, c_i64, c_f, c_f, ctypes.c_int, c_p]
        _lib = L
    return _lib


def _ptr(a: np.ndarray):
    return a.ctypes.data_as(ctypes.c_void_p)


def _as_input(x: np.ndarray):
    """float32 arrays are binary32 inputs; uint16 arrays are raw bfloat16 bits."""
    if x.dtype == np.float32:
        return np.ascontiguousarray(x), F32
    if x.dtype == np.uint16:
        return np.ascontiguousarray(x), BF16
    raise TypeError(f"oracle input must be float32 or bfloat16 bits (uint16), got {x.dtype}")


# --------------------------------------------------------------------- scalars
def e2m1_decode(code: int) -> float:
    return lib().oracle_e2m1_decode(int(code))


def ue5m3_decode(code: int) -> float:
    return lib().oracle_ue5m3_decode(int(code))


def ue5m3_encode(raw: float):
    """(code after repair, flags): flags bit0 zero-rounded, bit1 saturated."""
    f = ctypes.c_int(0)
    c = lib().oracle_ue5m3_encode(float(raw), ctypes.byref(f))
    return c, f.value


def ue5m3_nearest(raw: float) -> int:
    """Pre-repair nearest code; 0xF8 means above the largest finite value."""
    return lib().oracle_ue5m3_nearest(float(raw))


def e2m1_encode_rne(v: float, negative: bool | None = None) -> int:
    if negative is None:
        negative = bool(np.signbit(np.float32(v)))
    return lib().oracle_e2m1_encode_rne(float(v), int(negative))


def e2m1_encode_sr(v: float, word: int, negative: bool | None = None) -> int:
    if negative is None:
        negative = bool(np.signbit(np.float32(v)))
    return lib().oracle_e2m1_encode_sr(float(v), int(negative), int(word))


def philox4x32_10(ctr, key):
    c = np.asarray(ctr, dtype=np.uint32).copy()
    k = np.asarray(key, dtype=np.uint32).copy()
    out = np.zeros(4, dtype=np.uint32)
    lib().oracle_philox4x32_10(_ptr(c), _ptr(k), _ptr(out))
    return out


def sr_word(seed: int, subseq: int, index: int) -> int:
    return lib().oracle_sr_word(int(seed), int(subseq), int(index))


def e4m3_decode(code: int) -> float:
    return lib().oracle_e4m3_decode(int(code))


def e4m3_encode(raw: float) -> tuple[int, int]:
    """(code, flags) of the E4M3 block-scale encode with repair."""
    f = ctypes.c_int(0)
    c = lib().oracle_e4m3_encode(float(raw), ctypes.byref(f))
    return c, f.value


def tensor_scale(amax: float, T: float) -> np.float32:
    return np.float32(lib().oracle_tensor_scale(float(amax), float(T)))


# --------------------------------------------------------------------- tensors
def amax(x: np.ndarray) -> np.float32:
    xc, dt = _as_input(x)
    rows, cols = xc.shape
    return np.float32(lib().oracle_amax(_ptr(xc), dt, rows, cols, cols))


@dataclass
class QTensor:
    """A quantized operand stored contiguous along its contraction (cols)."""
    codes: np.ndarray      # uint8 [rows, cols/2]
    scales: np.ndarray     # uint8 ROW16 [rows, cols/block]; TILE16 [rows/block, cols/block]
    S: np.float32          # tensor (encode) scale
    rows: int
    cols: int
    layout: int            # ROW16 or TILE16
    block: int = 16        # block size (16, or 32 for the block-32 variant)
    scale_fmt: int = UE5M3  # UE5M3, or E4M3 (NVFP4's scale format)


@dataclass
class Quantized:
    q: QTensor                     # for ROW16/TILE16: [rows, cols]; for COL16: the transpose
    qt: QTensor | None             # TILE16 only: the transposed copy
    diag: np.ndarray               # [zero-rounded, saturated] block counts


def quantize(x: np.ndarray, amax_held: float, T: float = 448.0, layout: int = ROW16,
             rnd: int = RNE, seed: int = 0, subseq: int = 0, transposed: bool = False,
             origin: tuple | None = None, block: int = 16, scale_fmt: int = UE5M3) -> Quantized:
    """Quantize x. ``origin = (row0, col0, full_cols)`` places x inside a
    larger logical tensor for the SR word index (default: x is the whole
    tensor). ``block`` (16 or 32) and ``scale_fmt`` (UE5M3 or E4M3) select
    the block geometry and the block-scale format."""
    xc, dt = _as_input(x)
    rows, cols = xc.shape
    B = block
    row0, col0, full_cols = origin if origin is not None else (0, 0, cols)
    if B not in (16, 32) or (layout != COL16 and cols % B) or (layout != ROW16 and rows % B):
        raise ValueError("the blocked dimension(s) must be multiples of the block size (16 or 32)")
    if layout == COL16:
        codes = np.zeros((cols, rows // 2), np.uint8)
        scales = np.zeros((cols, rows // B), np.uint8)
    else:
        codes = np.zeros((rows, cols // 2), np.uint8)
        scales = np.zeros((rows, cols // B) if layout == ROW16 else (rows // B, cols // B), np.uint8)
    codes_t = scales_t = None
    if layout == TILE16 and transposed:
        codes_t = np.zeros((cols, rows // 2), np.uint8)
        scales_t = np.zeros((cols // B, rows // B), np.uint8)
    S = np.zeros(1, np.float32)
    diag = np.zeros(2, np.int32)
    rc = lib().oracle_quantize_fmt(_ptr(xc), dt, rows, cols, cols, float(amax_held), float(T), layout,
                                   B, scale_fmt, rnd, int(seed), int(subseq), int(row0), int(col0),
                                   int(full_cols), _ptr(codes), _ptr(scales), _ptr(S),
                                   _ptr(codes_t) if codes_t is not None else None,
                                   _ptr(scales_t) if scales_t is not None else None, _ptr(diag))
    if rc != 0:
        raise ValueError("oracle_quantize: bad shape or format")
    if layout == COL16:
        q = QTensor(codes, scales, S[0], cols, rows, ROW16, B, scale_fmt)
    else:
        q = QTensor(codes, scales, S[0], rows, cols, layout, B, scale_fmt)
    qt = None
    if codes_t is not None:
        qt = QTensor(codes_t, scales_t, S[0], cols, rows, TILE16, B, scale_fmt)
    return Quantized(q, qt, diag)


def decode_f64(q: QTensor) -> np.ndarray:
    """e2m1(code) * dec(scale) per element, exact in float64 (no tensor scale)."""
    out = np.zeros((q.rows, q.cols), np.float64)
    lib().oracle_decode_f64_fmt(_ptr(np.ascontiguousarray(q.codes)), _ptr(np.ascontiguousarray(q.scales)),
                                q.rows, q.cols, q.layout, q.block, q.scale_fmt, _ptr(out))
    return out


def dequant_f32(q: QTensor) -> np.ndarray:
    """x_hat = RN_f32((e2m1 * dec) / S)."""
    out = np.zeros((q.rows, q.cols), np.float32)
    lib().oracle_dequant_f32_fmt(_ptr(np.ascontiguousarray(q.codes)), _ptr(np.ascontiguousarray(q.scales)),
                                 q.rows, q.cols, q.layout, q.block, q.scale_fmt, float(q.S), _ptr(out))
    return out


def gemm(a: QTensor, b: QTensor) -> np.ndarray:
    """Y[i, j] = (sum_k A[i, k] B[j, k]) / (Sa Sb) over exactly decoded operands, float64.

    The emulated FP4 linear ("UE5M3 FP4 Block Scaling ...", §6): contraction of
    decoded operands with the tensor-scale product applied after it. fwd is
    Y = Xq Wq^T, dgrad is dX = dYq (Wq^T)^T with the transposed weight copy,
    wgrad is dW = (dYq^T)(Xq^T)^T with both operands quantized along tokens.
    """
    if a.cols != b.cols:
        raise ValueError("contraction lengths differ")
    A = decode_f64(a)
    B = decode_f64(b)
    return (A @ B.T) / (np.float64(a.S) * np.float64(b.S))


def gemm_probe(a: QTensor, b: QTensor, snap_log2: int = 0) -> np.ndarray:
    """The probe-matched GEMM numerics ("UE5M3 FP4 Block Scaling ...", §6 and
    Appendix B): exact 64-wide slice dot products rounded once to binary32,
    slice partials added in order with binary32 additions rounded toward
    zero, an optional snap of the accumulator to multiples of 2^-snap_log2
    (ties to even), then the binary32 product with alpha = 1 / (Sa Sb).
    Returns float32 [a.rows, b.rows]."""
    if a.cols != b.cols:
        raise ValueError("contraction lengths differ")
    A = np.ascontiguousarray(decode_f64(a))
    B = np.ascontiguousarray(decode_f64(b))
    y = np.zeros((a.rows, b.rows), np.float32)
    rc = lib().oracle_gemm_probe(_ptr(A), _ptr(B), a.rows, b.rows, a.cols, float(a.S), float(b.S),
                                 int(snap_log2), _ptr(y))
    if rc != 0:
        raise ValueError("decoded operand off the 2^-18 lattice")
    return y


def gemm_probe_decoded(A: np.ndarray, B: np.ndarray, Sa: float = 1.0, Sb: float = 1.0,
                       snap_log2: int = 0) -> np.ndarray:
    """gemm_probe on already decoded float64 operands (multiples of 2^-18)."""
    A = np.ascontiguousarray(A, np.float64)
    B = np.ascontiguousarray(B, np.float64)
    y = np.zeros((A.shape[0], B.shape[0]), np.float32)
    rc = lib().oracle_gemm_probe(_ptr(A), _ptr(B), A.shape[0], B.shape[0], A.shape[1], float(Sa),
                                 float(Sb), int(snap_log2), _ptr(y))
    if rc != 0:
        raise ValueError("decoded operand off the 2^-18 lattice")
    return y


def gemm_loops(a: QTensor, b: QTensor) -> np.ndarray:
    """The same contraction as plain triple loops in C (small cases only)."""
    A = decode_f64(a)
    B = decode_f64(b)
    y = np.zeros((a.rows, b.rows), np.float64)
    lib().oracle_gemm_f64_loops(_ptr(A), _ptr(B), a.rows, b.rows, a.cols,
                                float(a.S), float(b.S), _ptr(y))
    return y
