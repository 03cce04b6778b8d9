"""Parity at the full workload sizes, in the launch configuration the
benchmark times: the quantize-only tensor (8192x4096), the linear forward
(8192x4096x4096), the linear backward (dY 8192x4096 with SR) and the FFN
up-projection refresh step (16384x14336x4096).

Codes, scales, tensor scales and amax are compared bit for bit: whole
tensors where the oracle finishes in seconds, and 256-row / 256-column bands
of the step's tensors otherwise (the oracle quantizes the band on its own;
stochastic rounding takes the band's origin so its Philox words are the
whole tensor's). GEMM outputs are compared on blocks of rows and columns that
the oracle computes from its own quantizations of exactly the operand rows
they need, within the 2e-3 relative Frobenius bound."""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
from fp4_block_scaled_fp4q_amd import api, inputs
from parity_util import DEV, GEMM_TOL, rel_fro, round_out

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


def check_q(gq: api.QTensor, oq: oracle.QTensor, what: str, rows=None, scale_rows=None):
    """Bit-exact codes/scales/S of a GPU operand (optionally a row slice)
    against an oracle operand."""
    codes = npy(gq.codes if rows is None else gq.codes[rows])
    scales = npy(gq.scales if scale_rows is None else gq.scales[scale_rows])
    assert f32_bits(npy(gq.enc_scale)[0]) == f32_bits(oq.S), what
    np.testing.assert_array_equal(scales, oq.scales, err_msg=f"scales {what}")
    np.testing.assert_array_equal(codes, oq.codes, err_msg=f"codes {what}")


def sub_rows(q: oracle.QTensor, r0: int, n: int) -> oracle.QTensor:
    """Rows [r0, r0+n) of a ROW16 oracle operand."""
    assert q.layout == oracle.ROW16
    return oracle.QTensor(q.codes[r0:r0 + n], q.scales[r0:r0 + n], q.S, n, q.cols, q.layout)


def check_gemm(got: torch.Tensor, ref: np.ndarray, what: str):
    g = npy(got.float()).astype(np.float64)
    err = rel_fro(g, round_out(ref, got.dtype))
    assert err <= GEMM_TOL, f"{what}: rel Frobenius {err:.3e}"


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
    (whole tensors); Y = Xq Wq^T in bf16 on 256 sampled rows."""
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

    ox = oracle.quantize(X.oracle_view, hx_o, T, oracle.ROW16).q
    ow = oracle.quantize(W.oracle_view, hw_o, T, oracle.TILE16, transposed=True)
    check_q(xq, ox, "X ROW16")
    check_q(wq, ow.q, "W TILE")
    check_q(wqt, ow.qt, "W TILE transposed copy")
    for r0 in (0, M - BAND):
        ref = oracle.gemm(sub_rows(ox, r0, BAND), ow.q)
        check_gemm(Y[r0:r0 + BAND], ref, f"fwd rows {r0}..")


def test_linear_bwd_full_size():
    """dY 8192x4096 SR (ROW16 + COL16 in one pass, seed 0), X ROW16 + COL16,
    W TILE + transposed; dgrad and wgrad (contraction 8192 tokens) on sampled
    rows."""
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

    ody = oracle.quantize(dY.oracle_view, hd_o, T, oracle.ROW16, oracle.SR, seed).q
    odyt = oracle.quantize(dY.oracle_view, hd_o, T, oracle.COL16, oracle.SR, seed).q
    oxt = oracle.quantize(X.oracle_view, hx_o, T, oracle.COL16).q
    ow = oracle.quantize(W.oracle_view, hw_o, T, oracle.TILE16, transposed=True)
    check_q(dyq, ody, "dY ROW16 SR")
    check_q(dyqt, odyt, "dY COL16 SR")
    check_q(xqt, oxt, "X COL16")
    check_q(wqt, ow.qt, "W transposed copy")
    ox_band = oracle.quantize(X.oracle_view[:BAND], hx_o, T, oracle.ROW16).q
    check_q(xq, ox_band, "X ROW16 first rows", rows=slice(0, BAND), scale_rows=slice(0, BAND))
    for r0 in (0, M - BAND):
        check_gemm(dX[r0:r0 + BAND], oracle.gemm(sub_rows(ody, r0, BAND), ow.qt), f"dgrad rows {r0}..")
    for n0 in (0, N - BAND):
        check_gemm(dW[n0:n0 + BAND], oracle.gemm(sub_rows(odyt, n0, BAND), oxt), f"wgrad rows {n0}..")


@pytest.fixture(scope="module")
def ffn_step():
    """The benchmark's step on the FFN up-projection shape, run once."""
    wl = inputs.make("ffn_up_step")
    X, W, dY = (wl.tensors[k] for k in ("X", "W", "dY"))
    Xd, Wd, dYd = X.t.to(DEV), W.t.to(DEV), dY.t.to(DEV)
    am = {k: api.amax(t) for k, t in (("X", Xd), ("W", Wd), ("dY", dYd))}
    xq, xqt, _ = api.quantize(Xd, am["X"], T, api.ROW16, transposed=True)
    wq, wqt, _ = api.quantize(Wd, am["W"], T, api.TILE16x16, transposed=True)
    dyq, dyqt, _ = api.quantize(dYd, am["dY"], T, api.ROW16, api.SR, 0, 0, transposed=True)
    M, N, K = xq.rows, wq.rows, xq.cols
    Y = torch.empty((M, N), dtype=torch.bfloat16, device=DEV)
    dX = torch.empty((M, K), dtype=torch.bfloat16, device=DEV)
    dW = torch.empty((N, K), dtype=torch.float32, device=DEV)
    api.fp4q_linear_fwd(xq, wq, Y)
    api.fp4q_linear_dgrad(dyq, wqt, dX)
    api.fp4q_linear_wgrad(dyqt, xqt, dW)
    torch.cuda.synchronize()
    del Xd, Wd, dYd
    return dict(wl=wl, amax=am, xq=xq, xqt=xqt, wq=wq, wqt=wqt, dyq=dyq, dyqt=dyqt, Y=Y, dX=dX, dW=dW,
                M=M, N=N, K=K)


@pytest.fixture(scope="module")
def ffn_oracle_amax(ffn_step):
    """The oracle's amax of each step operand (the refresh step holds these)."""
    return {k: float(oracle.amax(ffn_step["wl"].tensors[k].oracle_view)) for k in ("X", "W", "dY")}


def test_ffn_step_amax(ffn_step, ffn_oracle_amax):
    """Refresh step: each operand's amax is taken from itself, bit-exact."""
    for k in ("X", "W", "dY"):
        assert f32_bits(npy(ffn_step["amax"][k])[0]) == f32_bits(ffn_oracle_amax[k]), k


def test_ffn_step_quantize_bands(ffn_step, ffn_oracle_amax):
    """256-row bands of X (ROW16 + COL16), dY (ROW16 + COL16, SR) and W (TILE
    + transposed copy), quantized by the oracle on their own."""
    s = ffn_step
    wl = s["wl"]
    X, W, dY = (wl.tensors[k] for k in ("X", "W", "dY"))
    ax, aw, ady = (ffn_oracle_amax[k] for k in ("X", "W", "dY"))
    M, N = s["M"], s["N"]
    for r0 in (0, M // 2 + 16 * 7, M - BAND):
        band = slice(r0, r0 + BAND)
        half = slice(r0 // 2, (r0 + BAND) // 2)
        sixteenth = slice(r0 // 16, (r0 + BAND) // 16)
        o = oracle.quantize(X.oracle_view[band], ax, T, oracle.ROW16).q
        check_q(s["xq"], o, f"X ROW16 rows {r0}..", rows=band, scale_rows=band)
        o = oracle.quantize(X.oracle_view[band], ax, T, oracle.COL16).q
        np.testing.assert_array_equal(npy(s["xqt"].codes[:, half]), o.codes, err_msg=f"X COL16 rows {r0}..")
        np.testing.assert_array_equal(npy(s["xqt"].scales[:, sixteenth]), o.scales)
        for lay, gq in ((oracle.ROW16, s["dyq"]), (oracle.COL16, s["dyqt"])):
            o = oracle.quantize(dY.oracle_view[band], ady, T, lay, oracle.SR, 0, 0, origin=(r0, 0, N)).q
            if lay == oracle.ROW16:
                check_q(gq, o, f"dY ROW16 SR rows {r0}..", rows=band, scale_rows=band)
            else:
                np.testing.assert_array_equal(npy(gq.codes[:, half]), o.codes, err_msg=f"dY COL16 rows {r0}..")
                np.testing.assert_array_equal(npy(gq.scales[:, sixteenth]), o.scales)
    for n0 in (0, N - BAND):
        band = slice(n0, n0 + BAND)
        o = oracle.quantize(W.oracle_view[band], aw, T, oracle.TILE16, transposed=True)
        check_q(s["wq"], o.q, f"W TILE rows {n0}..", rows=band, scale_rows=slice(n0 // 16, (n0 + BAND) // 16))
        np.testing.assert_array_equal(npy(s["wqt"].codes[:, n0 // 2:(n0 + BAND) // 2]), o.qt.codes)
        np.testing.assert_array_equal(npy(s["wqt"].scales[:, n0 // 16:(n0 + BAND) // 16]), o.qt.scales)


def test_ffn_step_gemm_blocks(ffn_step, ffn_oracle_amax):
    """256x256 output blocks of fwd, dgrad and wgrad (full contraction
    lengths 4096, 14336 and 16384) against the oracle's own operands; the
    column-band quantizations the oracle needs for them are also compared
    with the GPU's, bit for bit."""
    s = ffn_step
    wl = s["wl"]
    X, W, dY = (wl.tensors[k] for k in ("X", "W", "dY"))
    ax, aw, ady = (ffn_oracle_amax[k] for k in ("X", "W", "dY"))
    M, N, K = s["M"], s["N"], s["K"]
    r0, n0, k0 = M - BAND - 16 * 5, N // 2, K - BAND
    rows, ncols, kcols = slice(r0, r0 + BAND), slice(n0, n0 + BAND), slice(k0, k0 + BAND)

    xr = oracle.quantize(X.oracle_view[rows], ax, T, oracle.ROW16).q
    wr = oracle.quantize(W.oracle_view[ncols], aw, T, oracle.TILE16).q
    check_gemm(s["Y"][rows, ncols], oracle.gemm(xr, wr), "fwd block")

    dyr = oracle.quantize(dY.oracle_view[rows], ady, T, oracle.ROW16, oracle.SR, 0, 0, origin=(r0, 0, N)).q
    # W's transposed copy, rows k0.. (W columns k0.., all N rows)
    wk = oracle.quantize(np.ascontiguousarray(W.oracle_view[:, kcols]), aw, T, oracle.TILE16,
                         transposed=True).qt
    np.testing.assert_array_equal(npy(s["wqt"].codes[kcols]), wk.codes, err_msg="W transposed copy rows k0..")
    np.testing.assert_array_equal(npy(s["wqt"].scales[k0 // 16:(k0 + BAND) // 16]), wk.scales)
    check_gemm(s["dX"][rows, kcols], oracle.gemm(dyr, wk), "dgrad block")

    # COL16 operands of wgrad: dY columns n0.. and X columns k0.., all M tokens
    dyc = oracle.quantize(np.ascontiguousarray(dY.oracle_view[:, ncols]), ady, T, oracle.COL16, oracle.SR,
                          0, 0, origin=(0, n0, N)).q
    xc = oracle.quantize(np.ascontiguousarray(X.oracle_view[:, kcols]), ax, T, oracle.COL16).q
    check_q(s["dyqt"], dyc, "dY COL16 SR columns n0..", rows=ncols, scale_rows=ncols)
    check_q(s["xqt"], xc, "X COL16 columns k0..", rows=kcols, scale_rows=kcols)
    check_gemm(s["dW"][ncols, kcols], oracle.gemm(dyc, xc), "wgrad block")
