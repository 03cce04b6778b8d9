"""The K64 packing (the contraction cut into tiles of 64 elements, each tile
holding every row's codes and scales back to back) through the C ABI.

The packing changes only where bytes live, so every K64 result must equal
the row-major one exactly: quantize outputs unpacked by index permutation are
compared with the oracle bit for bit (every layout, rounding, input dtype,
block size and scale format), and the GEMMs, the probe-matched GEMM and the
dequantization on K64 operands must reproduce the row-major results bit for
bit, at shapes with ragged M and N tails and a split-tail wgrad."""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
from fp4_block_scaled_fp4q_amd import api, inputs
from parity_util import DEV, GEMM_TOL, assert_quant_equal, quant_both, rel_fro, round_out

pytestmark = pytest.mark.gpu
K64 = api.PACK_K64
FORMATS = [(16, api.UE5M3), (32, api.E4M3), (32, api.UE5M3), (16, api.E4M3)]


def data(shape, kind, dtype, seed):
    rng = np.random.default_rng(seed)
    R, C = shape
    x = (inputs.activation(rng, R, C, inputs.outlier_columns(rng, C)) if kind == "act"
         else inputs.loguniform_grad(rng, R, C))
    t = torch.from_numpy(x)
    return t.to(torch.bfloat16) if dtype == torch.bfloat16 else t


def held(x: torch.Tensor) -> float:
    return float(oracle.amax(inputs.bf16_bits(x) if x.dtype == torch.bfloat16 else x.numpy()))


@pytest.mark.parametrize("block,fmt", FORMATS)
@pytest.mark.parametrize("layout,transposed", [("row16", False), ("row16", True), ("col16", False),
                                               ("tile", False), ("tile", True)])
@pytest.mark.parametrize("rnd", [api.RNE, api.SR])
@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_quantize_k64_matches_oracle(block, fmt, layout, transposed, rnd, dtype):
    shape = (192, 320)  # several 64-wide tiles in both directions; ragged vs 256
    x = data(shape, "grad" if rnd == api.SR else "act", dtype, block + fmt + rnd)
    g, o = quant_both(x, held(x), layout, rnd, seed=5, subseq=2, transposed=transposed, block=block,
                      scale_fmt=fmt, pack=K64)
    assert_quant_equal(g, o, f"{layout} T={transposed} block {block} fmt {fmt}")
    assert g["q"].pack == K64 and g["q"].codes.dim() == 3


def _pair(x, A, layout, transposed=False, rnd=api.RNE, block=16, fmt=api.UE5M3):
    xd = x.to(DEV)
    a = torch.tensor([A], dtype=torch.float32, device=DEV)
    kw = dict(transposed=transposed, block=block, scale_fmt=fmt)
    rows = api.quantize(xd, a, 448.0, layout, rnd, 3, 1, pack=api.PACK_ROWS, **kw)
    k64 = api.quantize(xd, a, 448.0, layout, rnd, 3, 1, pack=K64, **kw)
    return rows, k64


@pytest.mark.parametrize("M,N,K", [(300, 224, 512), (256, 512, 1024), (64, 32, 64), (320, 192, 576)])
@pytest.mark.parametrize("block,fmt", [(16, api.UE5M3), (32, api.E4M3)])
def test_linear_k64_equals_rows(M, N, K, block, fmt):
    rng = np.random.default_rng(M + N + K + block)
    X = torch.from_numpy(inputs.activation(rng, M, K, inputs.outlier_columns(rng, K))).to(torch.bfloat16)
    W = torch.from_numpy(inputs.gaussian(rng, N, K, 0.02)).to(torch.bfloat16)
    dY = torch.from_numpy(inputs.loguniform_grad(rng, M, N)).to(torch.bfloat16)
    kw = dict(block=block, fmt=fmt)
    (xr, _, _), (xk, _, _) = _pair(X, held(X), api.ROW16, **kw)
    # the transposed weight copy (dgrad's operand) is blocked along N
    (wr, wrt, _), (wk, wkt, _) = _pair(W, held(W), api.TILE16x16, transposed=N % 64 == 0, **kw)
    dyr = dyk = None
    if N % 64 == 0:
        (dyr, _, _), (dyk, _, _) = _pair(dY, held(dY), api.ROW16, rnd=api.SR, **kw)
    # wgrad operands are blocked along tokens: M % 64 for K64
    wgrad = M % 64 == 0
    if wgrad:
        (dytr, _, _), (dytk, _, _) = _pair(dY, held(dY), api.COL16, rnd=api.SR, **kw)
        (xtr, _, _), (xtk, _, _) = _pair(X, held(X), api.COL16, **kw)
    for out in (torch.bfloat16, torch.float32):
        y = [torch.full((M, N), float("nan"), dtype=out, device=DEV) for _ in range(2)]
        api.fp4q_linear_fwd(xr, wr, y[0])
        api.fp4q_linear_fwd(xk, wk, y[1])
        torch.cuda.synchronize()
        assert torch.equal(y[0], y[1]), "fwd"
        if dyr is not None:
            dx = [torch.full((M, K), float("nan"), dtype=out, device=DEV) for _ in range(2)]
            api.fp4q_linear_dgrad(dyr, wrt, dx[0])
            api.fp4q_linear_dgrad(dyk, wkt, dx[1])
            torch.cuda.synchronize()
            assert torch.equal(dx[0], dx[1]), "dgrad"
        if wgrad:
            dw = [torch.full((N, K), float("nan"), dtype=out, device=DEV) for _ in range(2)]
            api.fp4q_linear_wgrad(dytr, xtr, dw[0])
            api.fp4q_linear_wgrad(dytk, xtk, dw[1])
            torch.cuda.synchronize()
            assert torch.equal(dw[0], dw[1]), "wgrad"
    # and the fwd result against the oracle's contraction
    ox = oracle.quantize(inputs.bf16_bits(X), held(X), 448.0, oracle.ROW16, block=block, scale_fmt=fmt).q
    ow = oracle.quantize(inputs.bf16_bits(W), held(W), 448.0, oracle.TILE16, block=block, scale_fmt=fmt).q
    assert rel_fro(y[1].float().cpu().numpy(), round_out(oracle.gemm(ox, ow), torch.float32)) <= GEMM_TOL


def test_split_tail_wgrad_k64():
    # 8 output tiles of 256 x 256 (fp32): the split-tail path on K64 operands
    M, N, K = 1024, 512, 1024
    rng = np.random.default_rng(9)
    a = torch.from_numpy(rng.standard_normal((K, M)).astype(np.float32))
    b = torch.from_numpy((0.02 * rng.standard_normal((N, M))).astype(np.float32))
    (ar, _, _), (ak, _, _) = _pair(a, float(np.abs(a.numpy()).max()), api.ROW16)
    (br, _, _), (bk, _, _) = _pair(b, float(np.abs(b.numpy()).max()), api.ROW16)
    y = [torch.full((K, N), float("nan"), dtype=torch.float32, device=DEV) for _ in range(2)]
    api.fp4q_linear_wgrad(ar, br, y[0])
    api.fp4q_linear_wgrad(ak, bk, y[1])
    torch.cuda.synchronize()
    assert torch.equal(y[0], y[1])


@pytest.mark.parametrize("snap", [0, 10])
def test_probe_k64_equals_rows(snap):
    rng = np.random.default_rng(snap)
    A = torch.from_numpy(rng.standard_normal((200, 256)).astype(np.float32))
    B = torch.from_numpy(rng.standard_normal((144, 256)).astype(np.float32))
    (ar, _, _), (ak, _, _) = _pair(A, float(np.abs(A.numpy()).max()), api.ROW16)
    (br, _, _), (bk, _, _) = _pair(B, float(np.abs(B.numpy()).max()), api.TILE16x16)
    y = [torch.empty((200, 144), dtype=torch.float32, device=DEV) for _ in range(2)]
    api.fp4q_linear_probe(ar, br, y[0], snap)
    api.fp4q_linear_probe(ak, bk, y[1], snap)
    torch.cuda.synchronize()
    assert torch.equal(y[0], y[1])


@pytest.mark.parametrize("block,fmt", FORMATS)
def test_dequant_k64_equals_rows(block, fmt):
    x = data((128, 192), "act", torch.float32, 77)
    for layout in (api.ROW16, api.TILE16x16):
        (qr, _, _), (qk, _, _) = _pair(x, held(x), layout, block=block, fmt=fmt)
        for dt in (torch.float32, torch.bfloat16):
            assert torch.equal(api.dequant(qr, dt), api.dequant(qk, dt))


def test_k64_empty_shapes():
    # no rows, or a contraction of length 0 (a multiple of 64): nothing is
    # written but the tensor scale, and a K = 0 GEMM writes zeros
    a = torch.tensor([3.0], dtype=torch.float32, device=DEV)
    for shape in ((0, 128), (64, 0)):
        x = torch.zeros(shape, dtype=torch.bfloat16, device=DEV)
        for layout in (api.ROW16, api.COL16, api.TILE16x16):
            if layout == api.COL16 and shape[0] % 64:
                continue
            q, _, _ = api.quantize(x, a, layout=layout, pack=K64)
            torch.cuda.synchronize()
            assert q.codes.numel() == 0 and q.scales.numel() == 0
            assert float(q.enc_scale.cpu()[0]) == np.float32(np.float32(6 * 448.0) / np.float32(3.0))
    xa = torch.zeros((32, 0), dtype=torch.bfloat16, device=DEV)
    xb = torch.zeros((48, 0), dtype=torch.bfloat16, device=DEV)
    qa, _, _ = api.quantize(xa, a, pack=K64)
    qb, _, _ = api.quantize(xb, a, layout=api.TILE16x16, pack=K64)
    y = torch.full((32, 48), float("nan"), dtype=torch.float32, device=DEV)
    api.fp4q_linear_fwd(qa, qb, y)
    torch.cuda.synchronize()
    assert torch.all(y == 0)
