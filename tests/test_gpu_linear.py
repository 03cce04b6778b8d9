"""GPU parity of the emulated FP4 linear layer (fwd, dgrad, wgrad) against the
oracle's fp64 contraction of the decoded operands: relative Frobenius error
<= 2e-3 against the oracle rounded to the output dtype; the quantized
operands themselves are compared bit-exactly first.

Covers the tiny fp32 case (64x128x256), ragged shapes (tails in M, N and K
that are not multiples of the 128x128x64 tile) and the bf16 workloads at
their full sizes (8192x4096x4096 fwd and bwd; 16384x14336x4096 FFN step),
where GEMM outputs are checked on sampled rows."""
import numpy as np
import pytest
import torch

import oracle
from fp4_block_scaled_fp4q_amd import api, inputs
from parity_util import (DEV, GEMM_TOL, assert_quant_equal, dev_scalar, host_view, quant_both,
                         rel_fro, round_out)

pytestmark = pytest.mark.gpu


def _gemm_check(y_dev: torch.Tensor, ref: np.ndarray, rows=None):
    y = y_dev.float().cpu().numpy() if rows is None else y_dev[rows].float().cpu().numpy()
    err = rel_fro(y, round_out(ref, y_dev.dtype))
    assert err <= GEMM_TOL, err
    return err


def test_tiny_fwd_fp32():
    wl = inputs.make("tiny_fwd")
    X, W = wl.tensors["X"].t, wl.tensors["W"].t
    ax = float(oracle.amax(host_view(X)))
    aw = float(oracle.amax(host_view(W)))
    gx, ox = quant_both(X, ax, "row16")
    gw, ow = quant_both(W, aw, "tile", transposed=True)
    assert_quant_equal(gx, ox)
    assert_quant_equal(gw, ow)
    y = torch.empty((64, 128), dtype=torch.float32, device=DEV)
    api.fp4q_linear_fwd(gx["q"], gw["q"], y)
    ref = oracle.gemm(ox.q, ow.q)
    err = _gemm_check(y, ref)
    assert err < 1e-6  # fp32 output of a short fp32-accumulated sum


@pytest.mark.parametrize("M,N,K", [(100, 48, 80), (130, 144, 1040), (1, 16, 16), (256, 256, 4096),
                                   (129, 272, 208), (0, 16, 32), (16, 16, 0)])
@pytest.mark.parametrize("btile", [False, True])
@pytest.mark.parametrize("out", [torch.float32, torch.bfloat16])
def test_gemm_shapes(M, N, K, btile, out):
    rng = np.random.default_rng(M * 7 + N * 3 + K)
    A = torch.from_numpy(inputs.activation(rng, M, K, inputs.outlier_columns(rng, K)) if M and K
                         else np.zeros((M, K), np.float32))
    B = torch.from_numpy(inputs.gaussian(rng, N, K, 0.02) if K else np.zeros((N, K), np.float32))
    aa = float(oracle.amax(host_view(A))) if A.numel() else 1.0
    ab = float(oracle.amax(host_view(B))) if B.numel() else 1.0
    ga, oa = quant_both(A, aa, "row16")
    gb, ob = quant_both(B, ab, "tile" if btile else "row16")
    y = torch.full((M, N), float("nan"), dtype=out, device=DEV)
    api.fp4q_linear_fwd(ga["q"], gb["q"], y)
    torch.cuda.synchronize()
    if M and N:
        if K == 0:
            assert torch.all(y == 0)
        else:
            _gemm_check(y, oracle.gemm(oa.q, ob.q))


def test_linear_small_fwd_dgrad_wgrad():
    rng = np.random.default_rng(11)
    M, N, K = 272, 192, 320
    X = inputs.to_bf16(inputs.activation(rng, M, K, inputs.outlier_columns(rng, K)))
    W = inputs.to_bf16(inputs.gaussian(rng, N, K, 0.02))
    dY = inputs.to_bf16(inputs.loguniform_grad(rng, M, N))
    ax, aw, ady = (float(oracle.amax(host_view(t))) for t in (X, W, dY))
    gx, ox = quant_both(X, ax, "row16")
    gw, ow = quant_both(W, aw, "tile", transposed=True)
    gdy, ody = quant_both(dY, ady, "row16", rnd=1, seed=5, transposed=True)  # + COL16 in one pass
    gdyt, odyt = quant_both(dY, ady, "col16", rnd=1, seed=5)
    gxt, oxt = quant_both(X, ax, "col16")
    for g, o in ((gx, ox), (gw, ow), (gdy, ody), (gdyt, odyt), (gxt, oxt)):
        assert_quant_equal(g, o)
    # the dual pass's COL16 output equals the COL16-only call
    np.testing.assert_array_equal(gdy["codes_t"], gdyt["codes"])
    y = torch.empty((M, N), dtype=torch.bfloat16, device=DEV)
    dx = torch.empty((M, K), dtype=torch.bfloat16, device=DEV)
    dw = torch.empty((N, K), dtype=torch.float32, device=DEV)
    api.fp4q_linear_fwd(gx["q"], gw["q"], y)
    api.fp4q_linear_dgrad(gdy["q"], gw["qt"], dx)
    api.fp4q_linear_wgrad(gdyt["q"], gxt["q"], dw)
    _gemm_check(y, oracle.gemm(ox.q, ow.q))
    _gemm_check(dx, oracle.gemm(ody.q, ow.qt))
    _gemm_check(dw, oracle.gemm(odyt.q, oxt.q))


def _rows(q: oracle.QTensor, idx):
    """The operand restricted to some rows (ROW16 layout only)."""
    return oracle.QTensor(q.codes[idx], q.scales[idx], q.S, len(idx), q.cols, q.layout)


def test_gemm_deterministic_and_launch_independent():
    rng = np.random.default_rng(12)
    A = torch.from_numpy(inputs.activation(rng, 512, 1024, inputs.outlier_columns(rng, 1024))).to(DEV)
    B = torch.from_numpy(inputs.gaussian(rng, 384, 1024, 0.02)).to(DEV)
    qa = api.quantize(A, api.amax(A))[0]
    qb = api.quantize(B, api.amax(B), layout=api.TILE16x16)[0]
    y1 = torch.empty((512, 384), device=DEV)
    y2 = torch.empty((512, 384), device=DEV)
    api.fp4q_linear_fwd(qa, qb, y1)
    api.fp4q_linear_fwd(qa, qb, y2)
    assert torch.equal(y1, y2)
    # a row-slice of A gives the same rows of Y (tile position does not matter)
    sub = api.QTensor(qa.codes[128:256], qa.scales[128:256], qa.enc_scale, 128, 1024, api.ROW16)
    y3 = torch.empty((128, 384), device=DEV)
    api.fp4q_linear_fwd(sub, qb, y3)
    assert torch.equal(y3, y1[128:256])


@pytest.mark.parametrize("M,N,K,out,pack", [
    (8292, 4144, 128, torch.float32, api.PACK_ROWS),  # 561 tiles, edge tiles
    (8292, 4144, 192, torch.bfloat16, api.PACK_K64),
    (8192, 4096, 64, torch.bfloat16, api.PACK_ROWS),  # 512 tiles
])
def test_gemm_many_tiles(M, N, K, out, pack):
    # More 256 x 256 output tiles than compute units, a tile count that does
    # not divide evenly over the eight XCD ranges, and partial edge tiles:
    # the whole output is within the GEMM bound of the oracle, and every
    # tile equals what a launch over a 256-row slice of A computes for it,
    # bit for bit (a tile's result does not depend on its position in the
    # launch).
    rng = np.random.default_rng(M + N + K)
    A = torch.from_numpy(inputs.activation(rng, M, K, inputs.outlier_columns(rng, K)))
    B = torch.from_numpy(inputs.gaussian(rng, N, K, 0.02))
    ga, oa = quant_both(A, float(oracle.amax(host_view(A))), "row16", pack=pack)
    gb, ob = quant_both(B, float(oracle.amax(host_view(B))), "tile", pack=pack)
    assert_quant_equal(ga, oa)
    assert_quant_equal(gb, ob)
    y = torch.full((M, N), float("nan"), dtype=out, device=DEV)
    api.fp4q_linear_fwd(ga["q"], gb["q"], y)
    torch.cuda.synchronize()
    _gemm_check(y, oracle.gemm(oa.q, ob.q))
    if pack == api.PACK_K64:
        # the same product from row-major operands, bit for bit
        ra, _ = quant_both(A, float(oracle.amax(host_view(A))), "row16")
        rb, _ = quant_both(B, float(oracle.amax(host_view(B))), "tile")
        yr = torch.full((M, N), float("nan"), dtype=out, device=DEV)
        api.fp4q_linear_fwd(ra["q"], rb["q"], yr)
        torch.cuda.synchronize()
        assert torch.equal(y, yr)
        return
    qa = ga["q"]
    for r0 in (0, 256 * 17, (M // 256) * 256):
        rows = min(256, M - r0)
        sub = api.QTensor(qa.codes[r0:r0 + rows], qa.scales[r0:r0 + rows], qa.enc_scale, rows, K, api.ROW16)
        ys = torch.full((rows, N), float("nan"), dtype=out, device=DEV)
        api.fp4q_linear_fwd(sub, gb["q"], ys)
        torch.cuda.synchronize()
        assert torch.equal(ys, y[r0:r0 + rows]), r0


@pytest.mark.parametrize("M,N,K", [(512, 1024, 1024), (500, 1000, 1040), (2048, 1024, 512)])
def test_split_tail_fp32_gemm(M, N, K):
    # fp32 outputs whose tile count leaves the last round of workgroups at
    # most half full run those tiles as two K halves added into a zeroed
    # output (here: 8, 8 and 32 tiles of 256 x 256); results stay within the
    # GEMM bound and are identical from run to run
    rng = np.random.default_rng(M + N + K)
    a = torch.from_numpy(rng.standard_normal((M, K)).astype(np.float32))
    b = torch.from_numpy((0.02 * rng.standard_normal((N, K))).astype(np.float32))
    ga, oa = quant_both(a, float(np.abs(a.numpy()).max()), "row16")
    gb, ob = quant_both(b, float(np.abs(b.numpy()).max()), "row16")
    y1 = torch.full((M, N), float("nan"), dtype=torch.float32, device=DEV)
    y2 = torch.full((M, N), float("nan"), dtype=torch.float32, device=DEV)
    api.fp4q_linear_wgrad(ga["q"], gb["q"], y1)
    api.fp4q_linear_wgrad(ga["q"], gb["q"], y2)
    torch.cuda.synchronize()
    assert torch.equal(y1, y2)
    ref = oracle.gemm(oa.q, ob.q)
    assert rel_fro(y1.cpu().numpy(), round_out(ref, torch.float32)) <= GEMM_TOL
    # an output that is not 16-byte aligned takes the unsplit path
    buf = torch.full((M * N + 1,), float("nan"), dtype=torch.float32, device=DEV)
    y3 = buf[1:].view(M, N)
    api.fp4q_linear_wgrad(ga["q"], gb["q"], y3)
    torch.cuda.synchronize()
    assert rel_fro(y3.cpu().numpy(), round_out(ref, torch.float32)) <= GEMM_TOL


def _coded_operand(rng, rows, cols, code_lo, code_hi, S, tile=False, scale_fmt=api.UE5M3):
    """Random payload codes and scale codes in [code_lo, code_hi), the same
    operand for the GPU and the oracle."""
    codes = rng.integers(0, 256, size=(rows, cols // 2), dtype=np.uint8)
    scales = rng.integers(code_lo, code_hi, size=(rows // 16 if tile else rows, cols // 16), dtype=np.uint8)
    g = api.QTensor(torch.from_numpy(codes).to(DEV), torch.from_numpy(scales).to(DEV), dev_scalar(S), rows,
                    cols, api.TILE16x16 if tile else api.ROW16, scale_fmt=scale_fmt)
    o = oracle.QTensor(codes, scales, np.float32(S), rows, cols, oracle.TILE16 if tile else oracle.ROW16,
                       scale_fmt=scale_fmt)
    return g, o


@pytest.mark.parametrize("case", [
    # (A codes, B codes, scale format): subnormal UE5M3 scales (down to
    # 2^-17) against mid-range ones; the largest codes (up to 61440) on both
    # sides; the whole UE5M3 range; the whole E4M3 range (2^-9 .. 448)
    ((0x01, 0x09), (0x70, 0x80), api.UE5M3),
    ((0xE8, 0xF8), (0xE8, 0xF8), api.UE5M3),
    ((0x01, 0xF8), (0x01, 0xF8), api.UE5M3),
    ((0x01, 0x7F), (0x01, 0x7F), api.E4M3),
])
@pytest.mark.parametrize("out", [torch.float32, torch.bfloat16])
def test_gemm_extreme_scale_codes(case, out):
    # every decoded value e2m1 * dec, from 2^-18 to 368640, enters the
    # contraction exactly: an operand decode that lost range or precision
    # anywhere would show against the exact fp64 contraction
    (alo, ahi), (blo, bhi), fmt = case
    rng = np.random.default_rng(alo * 31 + blo + fmt)
    M, N, K = 300, 272, 1088
    ga, oa = _coded_operand(rng, M, K, alo, ahi, 0.5, scale_fmt=fmt)
    gb, ob = _coded_operand(rng, N, K, blo, bhi, 3.0, tile=True, scale_fmt=fmt)
    y = torch.full((M, N), float("nan"), dtype=out, device=DEV)
    api.fp4q_linear_fwd(ga, gb, y)
    torch.cuda.synchronize()
    ref = oracle.gemm(oa, ob)
    yf = y.float().cpu().numpy()
    assert np.isfinite(yf).all()
    if fmt == api.UE5M3 and alo == 0x01 and ahi == 0x09:
        # scales with a narrow range: every output is a short exact-product
        # sum, so fp32 accumulation leaves only a tiny relative error
        assert rel_fro(yf, round_out(ref, out)) <= (2e-5 if out == torch.float32 else GEMM_TOL)
    _gemm_check(y, ref)


@pytest.mark.parametrize("out,N", [(torch.float32, (1 << 22) + 48), (torch.bfloat16, (1 << 23) + 48)])
def test_gemm_output_beyond_4gib(out, N):
    # An output of 5 GB: every 256-row tile band spans more than 2^32 bytes,
    # so interior tiles take the 64-bit-offset store path (K = 64 is one k
    # tile, so no tile is split into K halves here). Sampled columns (the first
    # and last tiles among them) match the oracle, and no output element is
    # left unwritten. With a held amax, ROW16 codes of a row depend on that
    # row alone, so the oracle quantizes only the sampled rows of B.
    M, K = 300, 64
    rng = np.random.default_rng(N)
    A = torch.from_numpy(inputs.activation(rng, M, K, inputs.outlier_columns(rng, K)))
    B = inputs.gaussian(rng, N, K, 0.02)
    aa, ab = float(oracle.amax(host_view(A))), float(np.abs(B).max())
    ga, oa = quant_both(A, aa, "row16")
    assert_quant_equal(ga, oa)
    qb = api.quantize(torch.from_numpy(B).to(DEV), dev_scalar(ab))[0]
    y = torch.full((M, N), float("nan"), dtype=out, device=DEV)
    api.fp4q_linear_fwd(ga["q"], qb, y)
    torch.cuda.synchronize()
    assert not torch.isnan(y).any().item()
    cols = np.unique(np.concatenate([np.arange(0, 300), np.arange(N - 300, N),
                                     rng.choice(N, 256, replace=False)]))
    ob = oracle.quantize(B[cols], ab, 448.0, oracle.ROW16, 0, 0, 0)
    idx = torch.from_numpy(cols).to(DEV)
    np.testing.assert_array_equal(qb.codes.index_select(0, idx).cpu().numpy(), ob.q.codes)
    np.testing.assert_array_equal(qb.scales.index_select(0, idx).cpu().numpy(), ob.q.scales)
    _gemm_check(y.index_select(1, idx), oracle.gemm(oa.q, ob.q))
