"""Python face of the C ABI: the same entry points, taking torch tensors.

Each ``fp4q_*`` function checks that its tensors are CUDA (HIP) tensors of
the right dtype and layout, passes their device pointers, row strides and the
current stream to libfp4q.so, and raises ``Fp4qError`` on a non-OK status.
``quantize`` additionally allocates the output tensors with torch (device
memory is torch's job here) before calling ``fp4q_quantize``.
"""
from __future__ import annotations

from dataclasses import dataclass

import torch

from . import _lib
from ._lib import (BF16, COL16, E4M3, F32, PACK_K64, PACK_ROWS, QTensorC, RNE, ROW16, SR, TILE16x16,
                   UE5M3, check, lib)

__all__ = ["QTensor", "fp4q_amax", "fp4q_quantize", "fp4q_quantize_fmt", "fp4q_dequant",
           "fp4q_linear_fwd", "fp4q_linear_dgrad", "fp4q_linear_wgrad", "fp4q_linear_probe",
           "quantize", "amax", "dequant", "ROW16", "COL16", "TILE16x16", "RNE", "SR", "F32", "BF16",
           "UE5M3", "E4M3", "PACK_ROWS", "PACK_K64"]


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return BF16
    if t.dtype == torch.float32:
        return F32
    raise TypeError(f"fp4q: unsupported dtype {t.dtype} (bfloat16 or float32)")


def _torch_dtype(code: int) -> torch.dtype:
    return torch.bfloat16 if code == BF16 else torch.float32


def _stream() -> int:
    return torch.cuda.current_stream().cuda_stream


def _dev2d(t: torch.Tensor, name: str) -> None:
    if not t.is_cuda:
        raise ValueError(f"fp4q: {name} must be a device tensor")
    if t.dim() != 2 or (t.numel() > 0 and t.shape[1] > 1 and t.stride(1) != 1):
        raise ValueError(f"fp4q: {name} must be 2-D with unit column stride")


def _ld(t: torch.Tensor) -> int:
    """Row stride in elements (an empty tensor's strides are arbitrary)."""
    return t.stride(0) if t.numel() > 0 else t.shape[1]


def _ptr(t: torch.Tensor | None) -> int | None:
    return None if t is None else t.data_ptr()


@dataclass
class QTensor:
    """A quantized operand on the device (see fp4q_qtensor).

    Row-major packing: codes uint8 [rows, cols/2], scales [SR, cols/B] with
    SR = rows (ROW16) or rows/B (TILE), B = block. K64 packing: the same
    bytes as [cols/64, rows, 32] codes and [cols/64, SR, 64/B] scales."""
    codes: torch.Tensor
    scales: torch.Tensor
    enc_scale: torch.Tensor  # float32 [1]: the tensor scale S
    rows: int
    cols: int
    layout: int              # ROW16 or TILE16x16
    block: int = 16          # 16, or 32 for the block-32 variant
    scale_fmt: int = UE5M3   # UE5M3, or E4M3 (NVFP4's scale format)
    pack: int = PACK_ROWS    # PACK_ROWS or PACK_K64

    def c(self) -> QTensorC:
        return QTensorC(self.codes.data_ptr(), self.scales.data_ptr(), self.enc_scale.data_ptr(),
                        self.rows, self.cols, self.layout, self.block, self.scale_fmt, self.pack)


# ---------------------------------------------------------------- entry points
def fp4q_amax(x: torch.Tensor, amax_out: torch.Tensor) -> None:
    _dev2d(x, "x")
    check("fp4q_amax", lib().fp4q_amax(x.data_ptr(), _dtype_code(x), x.shape[0], x.shape[1],
                                       _ld(x), amax_out.data_ptr(), _stream()))


def fp4q_quantize(x: torch.Tensor, amax_held: torch.Tensor, target: float, layout: int, rnd: int,
                  seed: int, subseq: int, codes: torch.Tensor, scales: torch.Tensor,
                  enc_scale_out: torch.Tensor | None = None, codes_t: torch.Tensor | None = None,
                  scales_t: torch.Tensor | None = None, diag: torch.Tensor | None = None) -> None:
    _dev2d(x, "x")
    st = lib().fp4q_quantize(x.data_ptr(), _dtype_code(x), x.shape[0], x.shape[1], _ld(x),
                             amax_held.data_ptr(), float(target), int(layout), int(rnd),
                             int(seed) & (2 ** 64 - 1), int(subseq) & 0xFFFFFFFF,
                             codes.data_ptr(), scales.data_ptr(), _ptr(enc_scale_out),
                             _ptr(codes_t), _ptr(scales_t), _ptr(diag), _stream())
    check("fp4q_quantize", st)


def fp4q_quantize_fmt(x: torch.Tensor, amax_held: torch.Tensor, target: float, layout: int,
                      block: int, scale_fmt: int, pack: int, rnd: int, seed: int, subseq: int,
                      codes: torch.Tensor, scales: torch.Tensor,
                      enc_scale_out: torch.Tensor | None = None, codes_t: torch.Tensor | None = None,
                      scales_t: torch.Tensor | None = None, diag: torch.Tensor | None = None) -> None:
    _dev2d(x, "x")
    st = lib().fp4q_quantize_fmt(x.data_ptr(), _dtype_code(x), x.shape[0], x.shape[1], _ld(x),
                                 amax_held.data_ptr(), float(target), int(layout), int(block),
                                 int(scale_fmt), int(pack), int(rnd), int(seed) & (2 ** 64 - 1),
                                 int(subseq) & 0xFFFFFFFF, codes.data_ptr(), scales.data_ptr(),
                                 _ptr(enc_scale_out), _ptr(codes_t), _ptr(scales_t), _ptr(diag),
                                 _stream())
    check("fp4q_quantize_fmt", st)


def fp4q_dequant(q: QTensor, out: torch.Tensor) -> None:
    qc = q.c()
    check("fp4q_dequant", lib().fp4q_dequant(qc, out.data_ptr(), _dtype_code(out), _stream()))


def _gemm(name: str, a: QTensor, b: QTensor, y: torch.Tensor) -> None:
    if not y.is_contiguous():
        raise ValueError(f"{name}: output must be contiguous")
    if tuple(y.shape) != (a.rows, b.rows):
        raise ValueError(f"{name}: output shape {tuple(y.shape)} != {(a.rows, b.rows)}")
    ac, bc = a.c(), b.c()
    check(name, getattr(lib(), name)(ac, bc, y.data_ptr(), _dtype_code(y), _stream()))


def fp4q_linear_fwd(xq: QTensor, wq: QTensor, y: torch.Tensor) -> None:
    """y[M, N] = Xq . Wq^T (X ROW16 [M, K], W TILE16x16 [N, K])."""
    _gemm("fp4q_linear_fwd", xq, wq, y)


def fp4q_linear_dgrad(dyq: QTensor, wqt: QTensor, dx: torch.Tensor) -> None:
    """dx[M, K] = dYq . Wq (dY ROW16 [M, N], W's transposed copy [K, N])."""
    _gemm("fp4q_linear_dgrad", dyq, wqt, dx)


def fp4q_linear_wgrad(dyqt: QTensor, xqt: QTensor, dw: torch.Tensor) -> None:
    """dw[N, K] = dYq^T . Xq (dY COL16 stored [N, M], X COL16 stored [K, M])."""
    _gemm("fp4q_linear_wgrad", dyqt, xqt, dw)


def fp4q_linear_probe(a: QTensor, b: QTensor, y: torch.Tensor, snap_log2: int = 0) -> None:
    """y[M, N] = A . B^T with the probe-matched accumulation (64-wide slices,
    round-toward-zero addition of the slice sums, optional snap to multiples
    of 2^-snap_log2)."""
    if not y.is_contiguous():
        raise ValueError("fp4q_linear_probe: output must be contiguous")
    if tuple(y.shape) != (a.rows, b.rows):
        raise ValueError(f"fp4q_linear_probe: output shape {tuple(y.shape)} != {(a.rows, b.rows)}")
    ac, bc = a.c(), b.c()
    check("fp4q_linear_probe", lib().fp4q_linear_probe(ac, bc, y.data_ptr(), _dtype_code(y), int(snap_log2),
                                                       _stream()))


# ---------------------------------------------------------------- helpers
def amax(x: torch.Tensor) -> torch.Tensor:
    out = torch.empty(1, dtype=torch.float32, device=x.device)
    fp4q_amax(x, out)
    return out


def operand_buffers(rows: int, cols: int, tile: bool, block: int = 16, pack: int = PACK_ROWS,
                    device: torch.device | str = "cuda"):
    """Allocate (codes, scales) of an operand with `rows` rows contiguous
    along `cols`, shaped for its packing (see QTensor)."""
    u8 = dict(dtype=torch.uint8, device=device)
    SR = rows // block if tile else rows
    if pack == PACK_K64:
        return (torch.empty((cols // 64, rows, 32), **u8),
                torch.empty((cols // 64, SR, 64 // block), **u8))
    return torch.empty((rows, cols // 2), **u8), torch.empty((SR, cols // block), **u8)


def quantize(x: torch.Tensor, amax_held: torch.Tensor, target: float = 448.0, layout: int = ROW16,
             rnd: int = RNE, seed: int = 0, subseq: int = 0, transposed: bool = False,
             with_diag: bool = False, block: int = 16, scale_fmt: int = UE5M3,
             pack: int = PACK_ROWS):
    """Allocate outputs and run fp4q_quantize_fmt.

    Returns (q, qt, diag): q is the operand as the GEMMs read it (for COL16,
    the [cols, rows] transpose stored ROW16); with transposed=True, qt is the
    other orientation (TILE: the transposed tile copy; ROW16: the COL16
    operand [cols, rows] of the same tensor), else None; diag the int32[2]
    repair counts or None. block (16 or 32) and scale_fmt (UE5M3 or E4M3)
    select the variant, pack the memory packing of every output.
    """
    _dev2d(x, "x")
    R, C = x.shape
    B = block
    dev = x.device
    S = torch.empty(1, dtype=torch.float32, device=dev)
    if layout == COL16:
        codes, scales = operand_buffers(C, R, False, B, pack, dev)
    else:
        codes, scales = operand_buffers(R, C, layout == TILE16x16, B, pack, dev)
    codes_t = scales_t = None
    if transposed:
        codes_t, scales_t = operand_buffers(C, R, layout == TILE16x16, B, pack, dev)
    diag = torch.empty(2, dtype=torch.int32, device=dev) if with_diag else None
    fp4q_quantize_fmt(x, amax_held, target, layout, block, scale_fmt, pack, rnd, seed, subseq, codes,
                      scales, S, codes_t, scales_t, diag)
    if layout == COL16:
        q = QTensor(codes, scales, S, C, R, ROW16, B, scale_fmt, pack)
    else:
        q = QTensor(codes, scales, S, R, C, layout, B, scale_fmt, pack)
    qt = QTensor(codes_t, scales_t, S, C, R, layout, B, scale_fmt, pack) if transposed else None
    return q, qt, diag


def dequant(q: QTensor, dtype: torch.dtype = torch.float32) -> torch.Tensor:
    out = torch.empty((q.rows, q.cols), dtype=dtype, device=q.codes.device)
    fp4q_dequant(q, out)
    return out
