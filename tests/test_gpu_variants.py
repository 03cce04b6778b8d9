"""The block-32 and E4M3-scale variants through the C ABI against the oracle:
quantize (every layout, both roundings, bf16 and fp32 inputs) bit for bit,
dequant bit for bit, and the three GEMMs (plus the probe-matched mode) on
variant operands within the GEMM bound ("UE5M3 FP4 Block Scaling for Stable
Language Model Pretraining": NVFP4's E4M3 scales, §3; block 32, §7.3)."""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
from fp4_block_scaled_fp4q_amd import api, inputs
from parity_util import DEV, GEMM_TOL, assert_quant_equal, host_view, quant_both, rel_fro, round_out

pytestmark = pytest.mark.gpu

FORMATS = [(32, api.UE5M3), (16, api.E4M3), (32, api.E4M3)]


def data(shape, kind, dtype, seed):
    rng = np.random.default_rng(seed)
    R, C = shape
    if kind == "act":
        x = inputs.activation(rng, R, C, inputs.outlier_columns(rng, C))
    elif kind == "grad":
        x = inputs.loguniform_grad(rng, R, C)
    else:
        x = inputs.gaussian(rng, R, C, 0.02)
    t = torch.from_numpy(x)
    return t.to(torch.bfloat16) if dtype == torch.bfloat16 else t


def held(x: torch.Tensor) -> float:
    return float(oracle.amax(host_view(x)))


CASES = [  # layout, shape, transposed
    ("row16", (40, 1056), False),
    ("col16", (192, 1032), False),
    ("tile", (192, 544), True),
    ("row16", (224, 608), True),   # ROW + COL in one pass
]


@pytest.mark.parametrize("block,fmt", FORMATS)
@pytest.mark.parametrize("layout,shape,transposed", CASES)
@pytest.mark.parametrize("rnd", [api.RNE, api.SR])
@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_quantize_variants(block, fmt, layout, shape, transposed, rnd, dtype):
    x = data(shape, "grad" if rnd == api.SR else "act", dtype, block + fmt + shape[0])
    g, o = quant_both(x, held(x), layout, rnd, seed=7, subseq=3, transposed=transposed,
                      block=block, scale_fmt=fmt)
    assert_quant_equal(g, o, f"{layout} block {block} fmt {fmt}")


@pytest.mark.parametrize("block,fmt", FORMATS)
@pytest.mark.parametrize("factor", [1e-3, 30.0])
def test_quantize_variants_repairs(block, fmt, factor):
    # a stale held amax (far too small or too large) drives scales into
    # saturation or zero-rounding; the repaired codes and counts must match
    x = data((64, 512), "act", torch.bfloat16, 11)
    A = held(x) * factor
    for layout in ("row16", "tile"):
        g, o = quant_both(x, A, layout, block=block, scale_fmt=fmt)
        assert_quant_equal(g, o, f"{layout} factor {factor}")
    if factor < 1:
        assert o.diag[1] > 0  # saturated blocks present


@pytest.mark.parametrize("block,fmt", FORMATS)
def test_dequant_variants(block, fmt):
    x = data((96, 320), "act", torch.bfloat16, 5)
    for layout in ("row16", "tile"):
        g, o = quant_both(x, held(x), layout, block=block, scale_fmt=fmt)
        for dt in (torch.float32, torch.bfloat16):
            out = api.dequant(g["q"], dt)
            torch.cuda.synchronize()
            ref = oracle.dequant_f32(o.q)
            if dt == torch.bfloat16:
                ref = torch.from_numpy(ref).to(torch.bfloat16).float().numpy()
            np.testing.assert_array_equal(out.float().cpu().numpy(), ref)


@pytest.mark.parametrize("block,fmt", FORMATS)
@pytest.mark.parametrize("M,N,K", [(224, 96, 352), (64, 320, 1024)])
def test_linear_variants(block, fmt, M, N, K):
    X = data((M, K), "act", torch.bfloat16, 1)
    W = data((N, K), "weight", torch.bfloat16, 2)
    dY = data((M, N), "grad", torch.bfloat16, 3)
    kw = dict(block=block, scale_fmt=fmt)
    gx, ox = quant_both(X, held(X), "row16", transposed=True, **kw)
    gw, ow = quant_both(W, held(W), "tile", transposed=True, **kw)
    gd, od = quant_both(dY, held(dY), "row16", api.SR, seed=5, transposed=True, **kw)
    Y = torch.empty((M, N), dtype=torch.bfloat16, device=DEV)
    dX = torch.empty((M, K), dtype=torch.bfloat16, device=DEV)
    dW = torch.empty((N, K), dtype=torch.float32, device=DEV)
    api.fp4q_linear_fwd(gx["q"], gw["q"], Y)
    api.fp4q_linear_dgrad(gd["q"], gw["qt"], dX)
    api.fp4q_linear_wgrad(gd["qt"], gx["qt"], dW)
    Yp = torch.empty((M, N), dtype=torch.float32, device=DEV)
    api.fp4q_linear_probe(gx["q"], gw["q"], Yp, 10)
    torch.cuda.synchronize()
    for got, ref, what in ((Y, oracle.gemm(ox.q, ow.q), "fwd"), (dX, oracle.gemm(od.q, ow.qt), "dgrad"),
                           (dW, oracle.gemm(od.qt, ox.qt), "wgrad")):
        err = rel_fro(got.float().cpu().numpy(), round_out(ref, got.dtype))
        assert err <= GEMM_TOL, f"{what}: {err:.3e}"
    refp = oracle.gemm_probe(ox.q, ow.q, 10).astype(np.float64)
    assert rel_fro(Yp.cpu().numpy().astype(np.float64), refp) < 1e-6


def test_mixed_operand_formats():
    # block-32 E4M3 activations against block-16 UE5M3 weights
    X = data((128, 512), "act", torch.bfloat16, 21)
    W = data((64, 512), "weight", torch.bfloat16, 22)
    gx, ox = quant_both(X, held(X), "row16", block=32, scale_fmt=api.E4M3)
    gw, ow = quant_both(W, held(W), "tile")
    Y = torch.empty((128, 64), dtype=torch.float32, device=DEV)
    api.fp4q_linear_fwd(gx["q"], gw["q"], Y)
    torch.cuda.synchronize()
    assert rel_fro(Y.cpu().numpy(), round_out(oracle.gemm(ox.q, ow.q), torch.float32)) <= GEMM_TOL
