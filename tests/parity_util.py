"""Shared helpers of the GPU parity tests: run one step through the C ABI
(via the thin torch binding) and the same step through the oracle, on the
same seeded host inputs, and compare."""
from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np
import torch

import oracle
from fp4_block_scaled_fp4q_amd import api, inputs

DEV = "cuda"
LAYOUTS = {"row16": (api.ROW16, oracle.ROW16), "col16": (api.COL16, oracle.COL16),
           "tile": (api.TILE16x16, oracle.TILE16)}


def host_view(t: torch.Tensor) -> np.ndarray:
    """The oracle's input form of a CPU tensor: float32, or bf16 bits."""
    t = t.contiguous()
    return t.numpy() if t.dtype == torch.float32 else inputs.bf16_bits(t)


def dev_scalar(v: float) -> torch.Tensor:
    return torch.tensor([v], dtype=torch.float32, device=DEV)


def unpack_k64(a: np.ndarray) -> np.ndarray:
    """Row-major view of a K64-packed code or scale array: [tiles, rows, n]
    (n bytes of each row per 64-element tile) -> [rows, tiles * n]."""
    t, r, n = a.shape
    return np.ascontiguousarray(a.transpose(1, 0, 2)).reshape(r, t * n)


def host_rows(t: torch.Tensor, pack: int) -> np.ndarray:
    """A device code or scale tensor as a row-major numpy array."""
    a = t.cpu().numpy()
    return unpack_k64(a) if pack == api.PACK_K64 else a


def quant_both(x: torch.Tensor, amax_held: float, layout: str, rnd: int = 0, T: float = 448.0,
               seed: int = 0, subseq: int = 0, transposed: bool = False, ld_pad: int = 0,
               block: int = 16, scale_fmt: int = 0, pack: int = 0):
    """Quantize the CPU tensor x on the GPU and with the oracle.

    Returns (gpu dict of numpy arrays, oracle Quantized). ld_pad > 0 stores x
    on the device inside a wider buffer (row stride cols + ld_pad). pack
    selects the GPU outputs' packing; the numpy arrays are row-major either
    way (K64 outputs are unpacked by index permutation only)."""
    lay_g, lay_o = LAYOUTS[layout]
    if ld_pad:
        buf = torch.zeros((x.shape[0], x.shape[1] + ld_pad), dtype=x.dtype)
        buf[:, :x.shape[1]] = x
        xd = buf.to(DEV)[:, :x.shape[1]]
    else:
        xd = x.to(DEV)
    q, qt, diag = api.quantize(xd, dev_scalar(amax_held), T, lay_g, rnd, seed, subseq,
                               transposed=transposed, with_diag=True, block=block, scale_fmt=scale_fmt,
                               pack=pack)
    torch.cuda.synchronize()
    g = dict(codes=host_rows(q.codes, pack), scales=host_rows(q.scales, pack),
             S=q.enc_scale.cpu().numpy()[0], diag=diag.cpu().numpy(), q=q, qt=qt)
    if qt is not None:
        g["codes_t"] = host_rows(qt.codes, pack)
        g["scales_t"] = host_rows(qt.scales, pack)
    o = oracle.quantize(host_view(x), amax_held, T, lay_o, rnd, seed, subseq, transposed=transposed,
                        block=block, scale_fmt=scale_fmt)
    if layout == "row16" and transposed:
        # the second orientation of a ROW16 call is the COL16 quantization
        oc = oracle.quantize(host_view(x), amax_held, T, oracle.COL16, rnd, seed, subseq, block=block,
                             scale_fmt=scale_fmt)
        o.qt = oc.q
        o.diag = o.diag + oc.diag
    return g, o


def assert_quant_equal(g, o, what=""):
    assert g["S"].view(np.uint32) == np.float32(o.q.S).view(np.uint32), what
    np.testing.assert_array_equal(g["scales"], o.q.scales, err_msg=f"scales {what}")
    np.testing.assert_array_equal(g["codes"], o.q.codes, err_msg=f"codes {what}")
    np.testing.assert_array_equal(g["diag"], o.diag, err_msg=f"diag {what}")
    if o.qt is not None:
        np.testing.assert_array_equal(g["scales_t"], o.qt.scales, err_msg=f"scales_t {what}")
        np.testing.assert_array_equal(g["codes_t"], o.qt.codes, err_msg=f"codes_t {what}")


def rel_fro(got: np.ndarray, ref: np.ndarray) -> float:
    got = got.astype(np.float64)
    ref = ref.astype(np.float64)
    den = np.linalg.norm(ref)
    return float(np.linalg.norm(got - ref) / den) if den > 0 else float(np.linalg.norm(got))


def round_out(y: np.ndarray, dtype: torch.dtype) -> np.ndarray:
    """RN_out of the fp64 reference: to fp32, then (bf16 outputs) to bf16."""
    t = torch.from_numpy(y.astype(np.float32))
    if dtype == torch.bfloat16:
        t = t.to(torch.bfloat16).float()
    return t.numpy().astype(np.float64)


GEMM_TOL = 2e-3


# ---------------------------------------------------------------- large cases
def _workers() -> int:
    return max(1, min(16, len(os.sched_getaffinity(0))))


def oracle_quantize_par(x: np.ndarray, amax_held: float, layout: int, rnd: int = 0, T: float = 448.0,
                        seed: int = 0, subseq: int = 0, transposed: bool = False, chunk: int = 512,
                        block: int = 16, scale_fmt: int = 0):
    """oracle.quantize of a large tensor, run as independent chunks on host
    threads (the oracle's C calls release the GIL). Under a held amax a ROW16
    (or TILE) row band and a COL16 column band depend on their own elements
    only, and SR takes the chunk's origin in the whole tensor, so the
    concatenated chunks equal one call on the whole tensor. Returns
    (q, qt) oracle QTensors; qt is the TILE transposed copy when asked."""
    rows, cols = x.shape
    col = layout == oracle.COL16
    n = cols if col else rows
    starts = list(range(0, n, chunk))

    def run(s):
        e = min(n, s + chunk)
        part = np.ascontiguousarray(x[:, s:e] if col else x[s:e])
        origin = (0, s, cols) if col else (s, 0, cols)
        return oracle.quantize(part, amax_held, T, layout, rnd, seed, subseq, transposed=transposed,
                               origin=origin, block=block, scale_fmt=scale_fmt)

    with ThreadPoolExecutor(_workers()) as ex:
        parts = list(ex.map(run, starts))
    S = parts[0].q.S
    codes = np.concatenate([p.q.codes for p in parts], axis=0)
    if layout == oracle.TILE16:
        scales = np.concatenate([p.q.scales for p in parts], axis=0)
        q = oracle.QTensor(codes, scales, S, rows, cols, oracle.TILE16, block, scale_fmt)
        qt = None
        if transposed:
            qt = oracle.QTensor(np.concatenate([p.qt.codes for p in parts], axis=1),
                                np.concatenate([p.qt.scales for p in parts], axis=1), S, cols, rows,
                                oracle.TILE16, block, scale_fmt)
        return q, qt
    scales = np.concatenate([p.q.scales for p in parts], axis=0)
    if col:
        return oracle.QTensor(codes, scales, S, cols, rows, oracle.ROW16, block, scale_fmt), None
    return oracle.QTensor(codes, scales, S, rows, cols, oracle.ROW16, block, scale_fmt), None


def sub_operand(q: oracle.QTensor, r0: int, n: int) -> oracle.QTensor:
    """Rows [r0, r0+n) of an oracle operand (n and r0 multiples of the block
    size for TILE)."""
    if q.layout == oracle.TILE16:
        b = q.block
        return oracle.QTensor(q.codes[r0:r0 + n], q.scales[r0 // b:(r0 + n) // b], q.S, n, q.cols,
                              q.layout, q.block, q.scale_fmt)
    return oracle.QTensor(q.codes[r0:r0 + n], q.scales[r0:r0 + n], q.S, n, q.cols, q.layout, q.block,
                          q.scale_fmt)


def gemm_ref_and_bound(a: oracle.QTensor, b: oracle.QTensor, out: torch.dtype):
    """The oracle's contraction (fp64) and an elementwise bound on what an
    fp32-accumulated evaluation of it may differ by:
        2 K 2^-24 (|A| |B|^T) / (Sa Sb)   (at most K - 1 fp32 roundings of
                                            partial sums, each within 2^-24
                                            of a partial sum of |products|;
                                            doubled for the matrix core's
                                            grouped additions)
      + 2^-22 |Y|                          (alpha's rounding and the fp32 product)
      + for bf16 outputs, 2^-8 of the fp32 value (RNE to 8 significant bits).
    |A| |B|^T is taken in fp64 from the oracle's exactly decoded operands."""
    A = oracle.decode_f64(a)
    B = oracle.decode_f64(b)
    s = np.float64(a.S) * np.float64(b.S)
    ref = (A @ B.T) / s
    absp = (np.abs(A) @ np.abs(B).T) / s
    del A, B
    K = a.cols
    bound = 2.0 * K * 2.0 ** -24 * absp + 2.0 ** -22 * np.abs(ref) + 1e-37
    if out == torch.bfloat16:
        bound += 2.0 ** -8 * (np.abs(ref) + bound)
    return ref, bound


def check_gemm_elementwise(got: torch.Tensor, ref: np.ndarray, bound: np.ndarray, what: str):
    """Every element within its bound, and the 2e-3 relative Frobenius bar
    against RN_out of the fp64 reference."""
    g = got.float().cpu().numpy().astype(np.float64)
    assert np.isfinite(g).all(), f"{what}: non-finite output"
    err = np.abs(g - ref)
    bad = err > bound
    if bad.any():
        i = np.argwhere(bad)[0]
        raise AssertionError(f"{what}: {int(bad.sum())} elements beyond the bound, first at {tuple(i)}: "
                             f"got {g[tuple(i)]!r}, ref {ref[tuple(i)]!r}, bound {bound[tuple(i)]!r}")
    fro = rel_fro(g, round_out(ref, got.dtype))
    assert fro <= GEMM_TOL, f"{what}: rel Frobenius {fro:.3e}"
    return fro


def lsb_exp(x: np.ndarray) -> np.ndarray:
    """Exponent of the lowest set bit of each nonzero (binary-fraction)
    float64 value; a large number (2^20) for zeros."""
    ax = np.abs(x)
    nz = ax > 0
    m, e = np.frexp(np.where(nz, ax, 1.0))
    v = (m * 2.0 ** 53).astype(np.int64)
    tz = np.zeros(v.shape, np.int64)
    for _ in range(53):
        z = ((v & 1) == 0) & nz
        tz += z
        v = np.where(z, v >> 1, v)
    return np.where(nz, e - 53 + tz, 1 << 20)


def probe_exact_condition(A: np.ndarray, B: np.ndarray) -> np.ndarray:
    """Per output of A B^T (decoded operands, fp64): whether in every 64-wide
    slice all products A[i, k] B[j, k] are integer multiples of a common 2^g
    and their absolute sum is below 2^(g + 24), the condition under which
    the probe-matched mode's slice sums are exact on the matrix core and its
    outputs equal the oracle's bit for bit."""
    la, lb = lsb_exp(A), lsb_exp(B)
    ok = np.ones((A.shape[0], B.shape[0]), bool)
    for s0 in range(0, A.shape[1], 64):
        g = (la[:, None, s0:s0 + 64] + lb[None, :, s0:s0 + 64]).min(axis=2)
        tot = np.abs(A[:, s0:s0 + 64]) @ np.abs(B[:, s0:s0 + 64]).T
        ok &= (tot == 0) | (tot < np.ldexp(1.0, np.minimum(g, 1000) + 24))
    return ok
