"""Parity at the full workload sizes, in the launch configuration the
benchmark times: the quantize-only tensor (8192x4096), the linear forward
(8192x4096x4096), the linear backward (dY 8192x4096 with SR) and the FFN
up-projection refresh step (16384x14336x4096, K64-packed operands, two
output tiles per workgroup and the split-K tail of the fp32 wgrad, exactly
as the benchmark runs it).

Codes, scales, tensor scales and amax are compared bit for bit over whole
tensors (the oracle runs in independent row or column chunks on host
threads; stochastic rounding takes each chunk's origin, so its Philox words
are the whole tensor's). GEMM outputs are compared against the oracle's fp64
contraction of its own quantizations: whole outputs for the 8192-token
linear layer, and for the FFN step one full-width row band and one
full-height column band of each GEMM. Every compared element must lie within
the elementwise fp32-accumulation bound of parity_util.gemm_ref_and_bound,
and each compared block within the 2e-3 relative Frobenius bar."""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
from fp4_block_scaled_fp4q_amd import api, inputs
from parity_util import (DEV, check_gemm_elementwise, gemm_ref_and_bound, host_rows,
                         oracle_quantize_par, probe_exact_condition, sub_operand)

pytestmark = pytest.mark.gpu

T = 448.0
BAND = 256


def npy(t: torch.Tensor) -> np.ndarray:
    return t.cpu().numpy()


def f32_bits(v) -> int:
    return int(np.float32(v).view(np.uint32))


def held_pair(tensor: inputs.Tensor):
    """The held amax of a workload tensor: the amax of its companion draw,
    on the GPU (through the C ABI) and in the oracle; asserted identical."""
    g = api.amax(tensor.held_from.to(DEV))
    o = oracle.amax(tensor.held_oracle_view)
    assert f32_bits(npy(g)[0]) == f32_bits(o)
    return g, o


def check_q(gq: api.QTensor, oq: oracle.QTensor, what: str):
    """Bit-exact codes/scales/S of a whole GPU operand (either packing)
    against an oracle operand."""
    assert f32_bits(npy(gq.enc_scale)[0]) == f32_bits(oq.S), what
    np.testing.assert_array_equal(host_rows(gq.scales, gq.pack), oq.scales, err_msg=f"scales {what}")
    np.testing.assert_array_equal(host_rows(gq.codes, gq.pack), oq.codes, err_msg=f"codes {what}")


def test_quantize_full_size():
    """8192x4096 bf16 activations, ROW16 RNE under a held amax: whole tensor."""
    wl = inputs.make("quantize")
    X = wl.tensors["X"]
    held, held_o = held_pair(X)
    q, _, diag = api.quantize(X.t.to(DEV), held, T, api.ROW16, api.RNE, with_diag=True)
    o = oracle.quantize(X.oracle_view, held_o, T, oracle.ROW16)
    check_q(q, o.q, "X ROW16")
    np.testing.assert_array_equal(npy(diag), o.diag)


def test_linear_fwd_full_size():
    """X 8192x4096 ROW16, W 4096x4096 TILE16x16 with its transposed copy
    (whole tensors); the whole bf16 output Y = Xq Wq^T."""
    wl = inputs.make("linear_fwd")
    X, W = wl.tensors["X"], wl.tensors["W"]
    hx, hx_o = held_pair(X)
    hw, hw_o = held_pair(W)
    xq, _, _ = api.quantize(X.t.to(DEV), hx, T, api.ROW16)
    wq, wqt, _ = api.quantize(W.t.to(DEV), hw, T, api.TILE16x16, transposed=True)
    M, N = xq.rows, wq.rows
    Y = torch.empty((M, N), dtype=torch.bfloat16, device=DEV)
    api.fp4q_linear_fwd(xq, wq, Y)
    torch.cuda.synchronize()

    ox, _ = oracle_quantize_par(X.oracle_view, hx_o, oracle.ROW16)
    ow, owt = oracle_quantize_par(W.oracle_view, hw_o, oracle.TILE16, transposed=True)
    check_q(xq, ox, "X ROW16")
    check_q(wq, ow, "W TILE")
    check_q(wqt, owt, "W TILE transposed copy")
    ref, bound = gemm_ref_and_bound(ox, ow, Y.dtype)
    check_gemm_elementwise(Y, ref, bound, "fwd, whole output")


def test_linear_bwd_full_size():
    """dY 8192x4096 SR (ROW16 + COL16 in one pass, seed 0), X ROW16 + COL16,
    W TILE + transposed; the whole dgrad output (bf16) and the whole wgrad
    output (fp32, contraction over the 8192 tokens)."""
    wl = inputs.make("linear_bwd")
    X, W, dY = wl.tensors["X"], wl.tensors["W"], wl.tensors["dY"]
    hx, hx_o = held_pair(X)
    hw, hw_o = held_pair(W)
    hd, hd_o = held_pair(dY)
    seed = 0
    xq, xqt, _ = api.quantize(X.t.to(DEV), hx, T, api.ROW16, transposed=True)
    wq, wqt, _ = api.quantize(W.t.to(DEV), hw, T, api.TILE16x16, transposed=True)
    dyq, dyqt, _ = api.quantize(dY.t.to(DEV), hd, T, api.ROW16, api.SR, seed, 0, transposed=True)
    M, N, K = dyq.rows, dyq.cols, xq.cols
    dX = torch.empty((M, K), dtype=torch.bfloat16, device=DEV)
    dW = torch.empty((N, K), dtype=torch.float32, device=DEV)
    api.fp4q_linear_dgrad(dyq, wqt, dX)
    api.fp4q_linear_wgrad(dyqt, xqt, dW)
    torch.cuda.synchronize()

    ody, _ = oracle_quantize_par(dY.oracle_view, hd_o, oracle.ROW16, oracle.SR, seed=seed)
    odyt, _ = oracle_quantize_par(dY.oracle_view, hd_o, oracle.COL16, oracle.SR, seed=seed)
    ox, _ = oracle_quantize_par(X.oracle_view, hx_o, oracle.ROW16)
    oxt, _ = oracle_quantize_par(X.oracle_view, hx_o, oracle.COL16)
    _, owt = oracle_quantize_par(W.oracle_view, hw_o, oracle.TILE16, transposed=True)
    check_q(dyq, ody, "dY ROW16 SR")
    check_q(dyqt, odyt, "dY COL16 SR")
    check_q(xq, ox, "X ROW16")
    check_q(xqt, oxt, "X COL16")
    check_q(wqt, owt, "W transposed copy")
    ref, bound = gemm_ref_and_bound(ody, owt, dX.dtype)
    check_gemm_elementwise(dX, ref, bound, "dgrad, whole output")
    ref, bound = gemm_ref_and_bound(odyt, oxt, dW.dtype)
    check_gemm_elementwise(dW, ref, bound, "wgrad, whole output")


def _step_gpu(wl, pack):
    """The benchmark's refresh step on the device in the given packing:
    amax of each operand, its quantization, then fwd, dgrad and wgrad."""
    X, W, dY = (wl.tensors[k] for k in ("X", "W", "dY"))
    Xd, Wd, dYd = X.t.to(DEV), W.t.to(DEV), dY.t.to(DEV)
    am = {k: api.amax(t) for k, t in (("X", Xd), ("W", Wd), ("dY", dYd))}
    xq, xqt, _ = api.quantize(Xd, am["X"], T, api.ROW16, transposed=True, pack=pack)
    wq, wqt, _ = api.quantize(Wd, am["W"], T, api.TILE16x16, transposed=True, pack=pack)
    dyq, dyqt, _ = api.quantize(dYd, am["dY"], T, api.ROW16, api.SR, 0, 0, transposed=True, pack=pack)
    M, N, K = xq.rows, wq.rows, xq.cols
    Y = torch.full((M, N), float("nan"), dtype=torch.bfloat16, device=DEV)
    dX = torch.full((M, K), float("nan"), dtype=torch.bfloat16, device=DEV)
    dW = torch.full((N, K), float("nan"), dtype=torch.float32, device=DEV)
    api.fp4q_linear_fwd(xq, wq, Y)
    api.fp4q_linear_dgrad(dyq, wqt, dX)
    api.fp4q_linear_wgrad(dyqt, xqt, dW)
    torch.cuda.synchronize()
    return dict(amax=am, xq=xq, xqt=xqt, wq=wq, wqt=wqt, dyq=dyq, dyqt=dyqt, Y=Y, dX=dX, dW=dW,
                M=M, N=N, K=K)


@pytest.fixture(scope="module")
def ffn_step():
    """The benchmark's step on the FFN up-projection shape (K64 packing),
    run once; the row-major packing's outputs are checked against it bit
    for bit and then dropped."""
    wl = inputs.make("ffn_up_step")
    s = _step_gpu(wl, api.PACK_K64)
    r = _step_gpu(wl, api.PACK_ROWS)
    for k in ("Y", "dX", "dW"):
        assert torch.equal(s[k].view(torch.uint8), r[k].view(torch.uint8)), f"{k}: K64 != row-major packing"
    del r
    torch.cuda.empty_cache()
    s["wl"] = wl
    return s


@pytest.fixture(scope="module")
def ffn_oracle(ffn_step):
    """The oracle's amax and whole quantizations of the step's operands
    (the refresh step holds each operand's own amax)."""
    wl = ffn_step["wl"]
    X, W, dY = (wl.tensors[k].oracle_view for k in ("X", "W", "dY"))
    a = {k: float(oracle.amax(wl.tensors[k].oracle_view)) for k in ("X", "W", "dY")}
    o = dict(amax=a)
    o["xq"], _ = oracle_quantize_par(X, a["X"], oracle.ROW16)
    o["xqt"], _ = oracle_quantize_par(X, a["X"], oracle.COL16)
    o["wq"], o["wqt"] = oracle_quantize_par(W, a["W"], oracle.TILE16, transposed=True)
    o["dyq"], _ = oracle_quantize_par(dY, a["dY"], oracle.ROW16, oracle.SR)
    o["dyqt"], _ = oracle_quantize_par(dY, a["dY"], oracle.COL16, oracle.SR)
    return o


def test_ffn_step_amax(ffn_step, ffn_oracle):
    """Refresh step: each operand's amax is taken from itself, bit-exact."""
    for k in ("X", "W", "dY"):
        assert f32_bits(npy(ffn_step["amax"][k])[0]) == f32_bits(ffn_oracle["amax"][k]), k


@pytest.mark.parametrize("name", ["xq", "xqt", "wq", "wqt", "dyq", "dyqt"])
def test_ffn_step_quantize_whole(ffn_step, ffn_oracle, name):
    """Every K64-packed operand of the step (X ROW16 and COL16, W TILE and
    its transposed copy, dY ROW16 and COL16 under SR), whole."""
    check_q(ffn_step[name], ffn_oracle[name], name)


# GEMMs of the step: (output, A operand, B operand)
STEP_GEMMS = {"fwd": ("Y", "xq", "wq"), "dgrad": ("dX", "dyq", "wqt"), "wgrad": ("dW", "dyqt", "xqt")}


@pytest.mark.parametrize("gemm", list(STEP_GEMMS))
@pytest.mark.parametrize("band", ["rows", "cols"])
def test_ffn_step_gemm_band(ffn_step, ffn_oracle, gemm, band):
    """One full-width row band (the last 256 output rows: for wgrad these
    are the split-K tail tiles of the last XCD range) and one full-height
    column band (256 columns in the middle of the output, crossing tile
    rounds, XCD ranges and, for wgrad, split and unsplit tiles) of each
    GEMM over its full contraction (4096, 14336 and 16384)."""
    out, an, bn = STEP_GEMMS[gemm]
    y = ffn_step[out]
    a, b = ffn_oracle[an], ffn_oracle[bn]
    if band == "rows":
        r0 = a.rows - BAND
        ref, bound = gemm_ref_and_bound(sub_operand(a, r0, BAND), b, y.dtype)
        got = y[r0:r0 + BAND]
    else:
        c0 = (b.rows // 2 // BAND) * BAND - BAND // 2 if gemm != "wgrad" else 12 * BAND + BAND // 2
        ref, bound = gemm_ref_and_bound(a, sub_operand(b, c0, BAND), y.dtype)
        got = y[:, c0:c0 + BAND]
    check_gemm_elementwise(got, ref, bound, f"{gemm} {band} band")


def test_ffn_step_probe_band(ffn_step, ffn_oracle):
    """The probe-matched forward GEMM on the step's K64 operands at the full
    FFN shape (16384 x 14336 x 4096, 128 x 128 tiles) with the 1/1024 snap,
    as the benchmark times it: a 32-row by 256-column block crossing tile
    boundaries in both directions against the oracle's probe rule. Every
    output whose slices meet the exactness condition equals the oracle bit
    for bit; the rest stay within 1024 units in the last place."""
    xq, wq = ffn_step["xq"], ffn_step["wq"]
    y = torch.empty((xq.rows, wq.rows), dtype=torch.float32, device=DEV)
    api.fp4q_linear_probe(xq, wq, y, 10)
    torch.cuda.synchronize()
    r0, c0 = 8192 - 16, 7168 - 128
    got = y[r0:r0 + 32, c0:c0 + 256].cpu().numpy()
    del y
    a = sub_operand(ffn_oracle["xq"], r0, 32)
    b = sub_operand(ffn_oracle["wq"], c0, 256)
    ref = oracle.gemm_probe(a, b, 10)
    ok = probe_exact_condition(oracle.decode_f64(a), oracle.decode_f64(b))
    assert ok.mean() > 0.9, ok.mean()
    eq = got.view(np.uint32) == ref.view(np.uint32)
    assert eq[ok].all(), f"{int((~eq[ok]).sum())} outputs meeting the condition differ"
    rest = ~ok & ~eq
    if rest.any():
        ulps = np.abs(got[rest].view(np.int32).astype(np.int64) - ref[rest].view(np.int32).astype(np.int64))
        assert ulps.max() <= 1024


# the block-32 and E4M3-scale variants as the benchmark times them
VARIANTS = [(32, 0, "block32_ue5m3"), (16, 1, "block16_e4m3"), (32, 1, "block32_e4m3")]


@pytest.mark.parametrize("block,fmt,tag", VARIANTS)
def test_quantize_full_size_variants(block, fmt, tag):
    """The quantize-only workload (8192x4096 bf16 ROW16 RNE, held amax,
    row-major packing) in each variant: whole tensor."""
    wl = inputs.make("quantize")
    X = wl.tensors["X"]
    held, held_o = held_pair(X)
    q, _, _ = api.quantize(X.t.to(DEV), held, T, api.ROW16, api.RNE, block=block, scale_fmt=fmt)
    o = oracle.quantize(X.oracle_view, held_o, T, oracle.ROW16, block=block, scale_fmt=fmt)
    check_q(q, o.q, f"X ROW16 {tag}")


@pytest.mark.parametrize("block,fmt,tag", VARIANTS)
def test_ffn_step_variant_fwd_band(ffn_step, block, fmt, tag):
    """The forward GEMM of the FFN shape on variant operands (X ROW16 and W
    TILE, K64 packing, the step's refresh maxima): W whole and the last 256
    output rows, every element within the elementwise bound."""
    wl = ffn_step["wl"]
    X, W = wl.tensors["X"], wl.tensors["W"]
    am = ffn_step["amax"]
    xv, _, _ = api.quantize(X.t.to(DEV), am["X"], T, api.ROW16, block=block, scale_fmt=fmt, pack=api.PACK_K64)
    wv, _, _ = api.quantize(W.t.to(DEV), am["W"], T, api.TILE16x16, block=block, scale_fmt=fmt,
                            pack=api.PACK_K64)
    M, N = xv.rows, wv.rows
    y = torch.empty((M, N), dtype=torch.bfloat16, device=DEV)
    api.fp4q_linear_fwd(xv, wv, y)
    torch.cuda.synchronize()
    r0 = M - BAND
    got = y[r0:r0 + BAND].clone()
    del y, xv
    ax, aw = float(npy(am["X"])[0]), float(npy(am["W"])[0])
    ow, _ = oracle_quantize_par(W.oracle_view, aw, oracle.TILE16, block=block, scale_fmt=fmt)
    check_q(wv, ow, f"W TILE {tag}")
    ox = oracle.quantize(np.ascontiguousarray(X.oracle_view[r0:r0 + BAND]), ax, T, oracle.ROW16, block=block,
                         scale_fmt=fmt).q
    ref, bound = gemm_ref_and_bound(ox, ow, got.dtype)
    check_gemm_elementwise(got, ref, bound, f"fwd {tag}, last {BAND} rows")


def test_ffn_step_fp4linear_bands(ffn_step, ffn_oracle):
    """The FP4Linear module's refresh step (step 0: fp32 master weight,
    bf16 activations, seed 0) on the FFN shape, as the benchmark runs it,
    against the oracle's quantizations of the same tensors (each under its
    own maximum; dY with Philox seed 0, subsequence 0): the last 256 rows of
    the output, of dX and of dW, every element within the elementwise
    bound."""
    from fp4_block_scaled_fp4q_amd.recipe import FP4Linear, Fp4Recipe
    wl = ffn_step["wl"]
    X, W, dY = (wl.tensors[k].t for k in ("X", "W", "dY"))
    M, K = X.shape
    N = W.shape[0]
    layer = FP4Linear(K, N, Fp4Recipe(refresh_period=50), device=DEV)
    with torch.no_grad():
        layer.weight.copy_(W.to(DEV).float())
    xin = X.to(DEV).requires_grad_(True)
    y = layer(xin)
    y.backward(dY.to(DEV))
    torch.cuda.synchronize()
    o = ffn_oracle
    got = {"y": y.detach()[M - BAND:].clone(), "dx": xin.grad[M - BAND:].clone(),
           "dw": layer.weight.grad[N - BAND:].clone()}
    del layer, xin, y
    torch.cuda.empty_cache()
    cases = {"y": (sub_operand(o["xq"], M - BAND, BAND), o["wq"]),
             "dx": (sub_operand(o["dyq"], M - BAND, BAND), o["wqt"]),
             "dw": (sub_operand(o["dyqt"], N - BAND, BAND), o["xqt"])}
    for k, (a, b) in cases.items():
        ref, bound = gemm_ref_and_bound(a, b, got[k].dtype)
        check_gemm_elementwise(got[k], ref, bound, f"FP4Linear {k}, last {BAND} rows")
    assert got["dw"].dtype == torch.float32 and got["dx"].dtype == torch.bfloat16
