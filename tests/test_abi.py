"""The C ABI library on a machine without a GPU: it loads, exports every
entry point include/fp4q.h declares, and rejects bad arguments with the
documented status codes before touching the device (no call here launches a
kernel)."""
import ctypes
import os
import re

import pytest

from fp4_block_scaled_fp4q_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "fp4q.h")

FAKE = ctypes.c_void_p(0x10000)       # a 64 KiB-aligned non-null address (never dereferenced)
FAKE_ODD = ctypes.c_void_p(0x10004)   # 4-byte aligned only


def declared_functions():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(fp4q_\w+)\s*\(", text, re.M)))


def test_library_exports_every_declared_function():
    L = _lib.lib()
    names = declared_functions()
    assert set(names) == set(_lib.EXPORTS), names
    for n in names:
        assert hasattr(L, n), n
    assert L.fp4q_abi_version() == 3
    for s in range(7):
        assert L.fp4q_status_str(s)


def q(rows, cols, layout=_lib.ROW16, codes=FAKE, scales=FAKE, S=FAKE, block=16, fmt=_lib.UE5M3,
      pack=_lib.PACK_ROWS):
    return _lib.QTensorC(codes.value if codes else None, scales.value if scales else None,
                         S.value if S else None, rows, cols, layout, block, fmt, pack)


def quant(**kw):
    a = dict(x=FAKE, xt=_lib.BF16, rows=32, cols=64, ld=64, amax=FAKE, target=448.0,
             layout=_lib.ROW16, rnd=_lib.RNE, codes=FAKE, scales=FAKE, S=None, ct=None, st=None,
             diag=None)
    a.update(kw)
    return _lib.lib().fp4q_quantize(a["x"], a["xt"], a["rows"], a["cols"], a["ld"], a["amax"],
                                    a["target"], a["layout"], a["rnd"], 0, 0, a["codes"],
                                    a["scales"], a["S"], a["ct"], a["st"], a["diag"], None)


def test_quantize_validation():
    assert quant(xt=5) == _lib.E_DTYPE
    assert quant(layout=9) == _lib.E_ARG
    assert quant(rnd=4) == _lib.E_ARG
    assert quant(target=0.0) == _lib.E_ARG
    assert quant(target=float("inf")) == _lib.E_ARG
    assert quant(target=float("nan")) == _lib.E_ARG
    assert quant(ct=FAKE) == _lib.E_ARG                       # codes_t without scales_t
    assert quant(ct=FAKE, st=FAKE, layout=_lib.COL16) == _lib.E_ARG  # no second orientation for COL16
    assert quant(ct=FAKE, st=FAKE, rows=24) == _lib.E_SHAPE   # ROW16 + COL16 needs rows % 16
    assert quant(amax=None) == _lib.E_NULL
    assert quant(x=None) == _lib.E_NULL
    assert quant(codes=None) == _lib.E_NULL
    assert quant(cols=24, ld=24) == _lib.E_SHAPE              # ROW16 needs cols % 16
    assert quant(rows=-1) == _lib.E_SHAPE
    assert quant(ld=32) == _lib.E_SHAPE                       # ld < cols
    assert quant(rows=24, layout=_lib.TILE16x16) == _lib.E_SHAPE
    assert quant(rows=24, layout=_lib.COL16) == _lib.E_SHAPE
    assert quant(cols=12, ld=16, layout=_lib.COL16) == _lib.E_ALIGN
    assert quant(x=FAKE_ODD) == _lib.E_ALIGN
    assert quant(ld=68) == _lib.E_ALIGN                       # 136-byte bf16 rows
    assert quant(codes=FAKE_ODD) == _lib.E_ALIGN
    assert quant(amax=ctypes.c_void_p(0x10002)) == _lib.E_ALIGN


def test_amax_validation():
    L = _lib.lib()
    assert L.fp4q_amax(FAKE, 3, 16, 16, 16, FAKE, None) == _lib.E_DTYPE
    assert L.fp4q_amax(FAKE, _lib.BF16, 16, 16, 16, None, None) == _lib.E_NULL
    assert L.fp4q_amax(None, _lib.BF16, 16, 16, 16, FAKE, None) == _lib.E_NULL
    assert L.fp4q_amax(FAKE, _lib.BF16, 16, 16, 8, FAKE, None) == _lib.E_SHAPE
    assert L.fp4q_amax(FAKE, _lib.BF16, 16, 12, 16, FAKE, None) == _lib.E_ALIGN
    assert L.fp4q_amax(FAKE_ODD, _lib.F32, 16, 16, 16, FAKE, None) == _lib.E_ALIGN


def test_gemm_and_dequant_validation():
    L = _lib.lib()
    for fn in (L.fp4q_linear_fwd, L.fp4q_linear_dgrad, L.fp4q_linear_wgrad):
        a, b = q(32, 64), q(48, 64, _lib.TILE16x16)
        assert fn(None, b, FAKE, _lib.BF16, None) == _lib.E_NULL
        assert fn(a, b, FAKE, 7, None) == _lib.E_DTYPE
        assert fn(a, q(48, 80, _lib.TILE16x16), FAKE, _lib.BF16, None) == _lib.E_SHAPE
        assert fn(a, q(40, 64, _lib.TILE16x16), FAKE, _lib.BF16, None) == _lib.E_SHAPE
        assert fn(q(32, 72), b, FAKE, _lib.BF16, None) == _lib.E_SHAPE
        assert fn(a, q(48, 64, 5), FAKE, _lib.BF16, None) == _lib.E_ARG
        assert fn(a, q(48, 64, _lib.COL16), FAKE, _lib.BF16, None) == _lib.E_ARG
        assert fn(a, b, None, _lib.BF16, None) == _lib.E_NULL
        assert fn(a, b, ctypes.c_void_p(0x10001), _lib.BF16, None) == _lib.E_ALIGN
        assert fn(a, b, ctypes.c_void_p(0x10002), _lib.F32, None) == _lib.E_ALIGN
        assert fn(q(32, 64, S=None), b, FAKE, _lib.BF16, None) == _lib.E_NULL
        assert fn(q(32, 64, codes=FAKE_ODD), b, FAKE, _lib.BF16, None) == _lib.E_ALIGN
        assert fn(a, q(48, 64, _lib.TILE16x16, scales=ctypes.c_void_p(0x10002)), FAKE, _lib.BF16,
                  None) == _lib.E_ALIGN
    assert L.fp4q_dequant(q(32, 64), None, _lib.F32, None) == _lib.E_NULL
    assert L.fp4q_dequant(q(32, 64), FAKE_ODD, _lib.F32, None) == _lib.E_ALIGN
    assert L.fp4q_dequant(q(32, 64), FAKE, 9, None) == _lib.E_DTYPE


def test_probe_gemm_validation():
    L = _lib.lib()
    a, b = q(32, 64), q(48, 64, _lib.TILE16x16)
    assert L.fp4q_linear_probe(a, b, FAKE, _lib.F32, -1, None) == _lib.E_ARG
    assert L.fp4q_linear_probe(a, b, FAKE, _lib.F32, 31, None) == _lib.E_ARG
    assert L.fp4q_linear_probe(None, b, FAKE, _lib.F32, 0, None) == _lib.E_NULL
    assert L.fp4q_linear_probe(a, q(48, 80, _lib.TILE16x16), FAKE, _lib.F32, 10, None) == _lib.E_SHAPE
    assert L.fp4q_linear_probe(a, b, FAKE, 7, 10, None) == _lib.E_DTYPE
    assert L.fp4q_linear_probe(a, b, None, _lib.BF16, 10, None) == _lib.E_NULL
    assert L.fp4q_linear_probe(a, b, ctypes.c_void_p(0x10002), _lib.F32, 10, None) == _lib.E_ALIGN


def test_format_validation():
    L = _lib.lib()
    a, b = q(32, 64), q(48, 64, _lib.TILE16x16)
    # operand block size / scale format
    assert L.fp4q_linear_fwd(q(32, 64, block=8), b, FAKE, _lib.BF16, None) == _lib.E_ARG
    assert L.fp4q_linear_fwd(a, q(48, 64, _lib.TILE16x16, fmt=2), FAKE, _lib.BF16, None) == _lib.E_ARG
    assert L.fp4q_linear_fwd(q(32, 48, block=32), q(48, 48), FAKE, _lib.BF16, None) == _lib.E_SHAPE
    assert L.fp4q_linear_fwd(a, q(48, 64, _lib.TILE16x16, block=32), FAKE, _lib.BF16, None) == _lib.E_SHAPE
    assert L.fp4q_dequant(q(32, 48, block=32), FAKE, _lib.F32, None) == _lib.E_SHAPE

    def qf(rows=64, cols=64, layout=_lib.ROW16, block=32, fmt=_lib.E4M3, ct=None, st=None):
        return L.fp4q_quantize_fmt(FAKE, _lib.BF16, rows, cols, cols, FAKE, 448.0, layout, block, fmt,
                                   _lib.PACK_ROWS, _lib.RNE, 0, 0, FAKE, FAKE, None, ct, st, None, None)
    assert qf(block=24) == _lib.E_ARG
    assert qf(fmt=3) == _lib.E_ARG
    assert qf(cols=48) == _lib.E_SHAPE                       # ROW blocks of 32
    assert qf(rows=48, layout=_lib.COL16) == _lib.E_SHAPE    # COL blocks of 32
    assert qf(rows=48, layout=_lib.TILE16x16) == _lib.E_SHAPE
    assert qf(rows=48, ct=FAKE, st=FAKE) == _lib.E_SHAPE     # ROW + COL needs rows % 32


def test_packing_validation():
    L = _lib.lib()

    def qp(rows=128, cols=128, layout=_lib.ROW16, pack=_lib.PACK_K64, ct=None, st=None):
        return L.fp4q_quantize_fmt(FAKE, _lib.BF16, rows, cols, cols, FAKE, 448.0, layout, 16, _lib.UE5M3,
                                   pack, _lib.RNE, 0, 0, FAKE, FAKE, None, ct, st, None, None)
    assert qp(pack=2) == _lib.E_ARG
    assert qp(pack=-1) == _lib.E_ARG
    # K64 needs every output's contraction length to be a multiple of 64
    assert qp(cols=96) == _lib.E_SHAPE                                  # ROW16: cols
    assert qp(cols=96, layout=_lib.TILE16x16) == _lib.E_SHAPE           # TILE: cols
    assert qp(rows=96, layout=_lib.COL16) == _lib.E_SHAPE               # COL16: rows
    assert qp(rows=96, ct=FAKE, st=FAKE) == _lib.E_SHAPE                # ROW16 + COL16: rows too
    assert qp(rows=96, layout=_lib.TILE16x16, ct=FAKE, st=FAKE) == _lib.E_SHAPE  # transposed tile copy
    # operands: K64 needs cols % 64; the two GEMM operands must share the packing
    k = _lib.PACK_K64
    assert L.fp4q_dequant(q(32, 96, pack=k), FAKE, _lib.F32, None) == _lib.E_SHAPE
    assert L.fp4q_dequant(q(32, 64, pack=3), FAKE, _lib.F32, None) == _lib.E_ARG
    assert L.fp4q_linear_fwd(q(32, 64, pack=k), q(48, 64), FAKE, _lib.BF16, None) == _lib.E_ARG
    assert L.fp4q_linear_wgrad(q(32, 96, pack=k), q(48, 96, pack=k), FAKE, _lib.F32, None) == _lib.E_SHAPE


def test_oversized_grids_are_rejected():
    # shapes whose launch would exceed the grid limits come back as
    # FP4Q_E_SHAPE before anything is enqueued (nothing is dereferenced)
    L = _lib.lib()
    huge = 1 << 40
    assert L.fp4q_quantize(FAKE, _lib.BF16, huge, 4096, 4096, FAKE, 448.0, _lib.ROW16, _lib.RNE, 0, 0,
                           FAKE, FAKE, None, None, None, None, None) == _lib.E_SHAPE
    assert L.fp4q_quantize(FAKE, _lib.BF16, huge, 4096, 4096, FAKE, 448.0, _lib.TILE16x16, _lib.RNE, 0,
                           0, FAKE, FAKE, None, None, None, None, None) == _lib.E_SHAPE
    assert L.fp4q_quantize(FAKE, _lib.BF16, huge, 4096, 4096, FAKE, 448.0, _lib.COL16, _lib.RNE, 0, 0,
                           FAKE, FAKE, None, None, None, None, None) == _lib.E_SHAPE
    # ROW16 alone: one 64-lane workgroup per 64 blocks of a row, so 2^25 rows
    # of 64 columns are one workgroup past 2^31 threads
    assert L.fp4q_quantize(FAKE, _lib.BF16, 1 << 25, 64, 64, FAKE, 448.0, _lib.ROW16, _lib.RNE, 0, 0,
                           FAKE, FAKE, None, None, None, None, None) == _lib.E_SHAPE
    assert L.fp4q_linear_fwd(q(huge, 64), q(huge, 64), FAKE, _lib.F32, None) == _lib.E_SHAPE
    assert L.fp4q_dequant(q(huge, 4096), FAKE, _lib.F32, None) == _lib.E_SHAPE
    # negative sizes
    assert L.fp4q_amax(FAKE, _lib.BF16, -1, 16, 16, FAKE, None) == _lib.E_SHAPE
    assert L.fp4q_linear_fwd(q(-16, 64), q(16, 64), FAKE, _lib.F32, None) == _lib.E_SHAPE
