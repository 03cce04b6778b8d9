"""Shared helpers of the GPU parity tests: run one step through the C ABI
(via the thin torch binding) and the same step through the oracle, on the
same seeded host inputs, and compare."""
from __future__ import annotations

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
