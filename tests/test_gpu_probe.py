"""The probe-matched GEMM numerics (fp4q_linear_probe) against the oracle:
64-wide slice sums, round-toward-zero addition of the slices, the optional
1/1024 snap, then alpha ("UE5M3 FP4 Block Scaling for Stable Language Model
Pretraining", §6 and Appendix B).

The matrix core aligns each group of products to the largest and keeps 24
bits below its leading bit, so a slice sum is exact, and equal to the
oracle's, whenever the slice's products are multiples of a common 2^g whose
absolute sum stays below 2^(g+24). Outputs whose slices all meet that
condition must match the oracle bit for bit (this exercises the toward-zero
additions and the snap exactly); the rest may differ by a few units in the
last place."""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
from fp4_block_scaled_fp4q_amd import api, inputs
from parity_util import DEV, probe_exact_condition, quant_both, rel_fro

pytestmark = pytest.mark.gpu


def operand(codes: np.ndarray, scales: np.ndarray, S: float, layout: int):
    """The same operand for the GPU (api.QTensor) and the oracle."""
    rows, half = codes.shape
    cols = 2 * half
    g = api.QTensor(torch.from_numpy(codes).to(DEV), torch.from_numpy(scales).to(DEV),
                    torch.tensor([S], dtype=torch.float32, device=DEV), rows, cols, layout)
    o = oracle.QTensor(codes, scales, np.float32(S), rows, cols,
                       oracle.TILE16 if layout == api.TILE16x16 else oracle.ROW16)
    return g, o


def random_operand(rng, rows, cols, layout, code_lo, code_hi, S=1.0):
    codes = rng.integers(0, 256, size=(rows, cols // 2), dtype=np.uint8)
    srows = rows // 16 if layout == api.TILE16x16 else rows
    scales = rng.integers(code_lo, code_hi, size=(srows, cols // 16), dtype=np.uint8)
    return operand(codes, scales, S, layout)


def run_probe(a, b, dtype=torch.float32, snap=0):
    y = torch.empty((a.rows, b.rows), dtype=dtype, device=DEV)
    api.fp4q_linear_probe(a, b, y, snap)
    torch.cuda.synchronize()
    return y.float().cpu().numpy()


def test_toward_zero_slice_addition_hand_worked():
    K = 128
    ac = np.zeros((2, K // 2), np.uint8)
    asc = np.full((2, K // 16), 0x78, np.uint8)  # scale 1.0
    ac[0, 0] = 0x02                              # element 0: 1.0
    ac[0, 32] = 0x03                             # element 64: 1.5
    asc[0, 4] = 0x18                             # block of element 64: 2^-12
    ac[1] = np.where(ac[0] != 0, ac[0] | 0x08, 0)  # negated row
    asc[1] = asc[0]
    bc = np.zeros((1, K // 2), np.uint8)
    bsc = np.full((1, K // 16), 0x78, np.uint8)
    bc[0, 0] = 0x02
    bc[0, 32] = 0x02                             # element 64: 1.0
    bsc[0, 4] = 0x18                             # x 2^-12
    ga, oa = operand(ac, asc, 1.0, api.ROW16)
    gb, ob = operand(bc, bsc, 1.0, api.ROW16)
    y = run_probe(ga, gb)
    # slices: 1 and 1.5 * 2^-24 = 0.75 ulp(1); toward zero keeps +-1
    assert y[0, 0] == np.float32(1.0) and y[1, 0] == np.float32(-1.0)
    np.testing.assert_array_equal(y, oracle.gemm_probe(oa, ob))
    # the default accumulation rounds the same sum to nearest
    yd = torch.empty((2, 1), dtype=torch.float32, device=DEV)
    api.fp4q_linear_fwd(ga, gb, yd)
    torch.cuda.synchronize()
    assert yd.cpu().numpy()[0, 0] == np.float32(1.0 + 2.0 ** -23)


@pytest.mark.parametrize("M,N,K", [(200, 136, 1088), (128, 128, 64), (33, 300, 208), (256, 16, 4096)])
@pytest.mark.parametrize("snap", [0, 10])
@pytest.mark.parametrize("codes", [(0x70, 0x80), (0x20, 0x28)])
def test_bit_exact_when_slice_sums_are_representable(M, N, K, snap, codes):
    # scale codes over one or two binades: a slice's 64 products span a few
    # binades only, so every slice sum is exact in binary32 on both sides
    rng = np.random.default_rng(M * 7 + N + K + snap + codes[0])
    ga, oa = random_operand(rng, M, K, api.ROW16, *codes, S=2.0)
    gb, ob = random_operand(rng, N, K, api.TILE16x16 if N % 16 == 0 else api.ROW16, *codes, S=0.75)
    ref = oracle.gemm_probe(oa, ob, snap)
    np.testing.assert_array_equal(run_probe(ga, gb, torch.float32, snap), ref)
    ref_bf16 = torch.from_numpy(ref).to(torch.bfloat16).float().numpy()
    np.testing.assert_array_equal(run_probe(ga, gb, torch.bfloat16, snap), ref_bf16)
    if snap and codes[0] == 0x20:
        assert (ref == 0).mean() > 0.2  # the dead zone of the 1/1024 grid is exercised


@pytest.mark.parametrize("K", [512, 4096])
def test_toward_zero_every_slice_addition(K):
    # K / 64 slices: slice 0 sums to 1.0, every later slice to 0.75 ulp(1)
    # (1.5 times 2^-12 times 2^-12). Each addition onto the running 1.0 must
    # truncate, so the result is exactly 1.0 (rounding any one addition to
    # nearest would give 1 + ulp or more). The k loop runs two slices per
    # trip, so both slices of a trip are checked.
    n = K // 64
    ac = np.zeros((1, K // 2), np.uint8)
    asc = np.full((1, K // 16), 0x78, np.uint8)
    bc = np.zeros((1, K // 2), np.uint8)
    bsc = np.full((1, K // 16), 0x78, np.uint8)
    ac[0, 0] = 0x02
    bc[0, 0] = 0x02
    for sl in range(1, n):
        ac[0, 32 * sl] = 0x03
        asc[0, 4 * sl] = 0x18
        bc[0, 32 * sl] = 0x02
        bsc[0, 4 * sl] = 0x18
    ga, oa = operand(ac, asc, 1.0, api.ROW16)
    gb, ob = operand(bc, bsc, 1.0, api.ROW16)
    y = run_probe(ga, gb)
    assert y[0, 0] == np.float32(1.0)
    np.testing.assert_array_equal(y, oracle.gemm_probe(oa, ob))


@pytest.mark.parametrize("case", ["activations-weights", "gradients-weights"])
@pytest.mark.parametrize("snap", [0, 10])
def test_bit_exact_under_the_stated_condition(case, snap):
    # quantized operands of the 8192-token layer's distributions, K = 4096
    # (64 slices, so 63 toward-zero additions that round): every output whose
    # slices meet the exactness condition equals the oracle bit for bit; the
    # others (slices whose products span more than the matrix core's 24-bit
    # alignment window) stay within a few units in the last place
    M, N, K = 256, 512, 4096
    if case == "activations-weights":
        wl = inputs.make("linear_fwd", scale_rows=M)
        A = wl.tensors["X"].t[:, :K].contiguous()
        B = wl.tensors["W"].t[:N, :K].contiguous()
        ga, oa = quant_both(A, float(oracle.amax(inputs.bf16_bits(A))), "row16")
        gb, ob = quant_both(B, float(oracle.amax(inputs.bf16_bits(B))), "tile")
        qa, qb, oqa, oqb = ga["q"], gb["q"], oa.q, ob.q
    else:
        rng = np.random.default_rng(3)
        A = inputs.to_bf16(inputs.loguniform_grad(rng, M, K))
        Bt = inputs.to_bf16(inputs.gaussian(rng, K, N, 0.02))
        ga, oa = quant_both(A, float(oracle.amax(inputs.bf16_bits(A))), "row16", 1, seed=5)
        gb, ob = quant_both(Bt, float(oracle.amax(inputs.bf16_bits(Bt))), "tile", transposed=True)
        qa, qb, oqa, oqb = ga["q"], gb["qt"], oa.q, ob.qt
    ref = oracle.gemm_probe(oqa, oqb, snap)
    y = run_probe(qa, qb, torch.float32, snap)
    ok = probe_exact_condition(oracle.decode_f64(oqa), oracle.decode_f64(oqb))
    assert ok.mean() > 0.99
    eq = y.view(np.uint32) == ref.view(np.uint32)
    assert eq[ok].all(), f"{int((~eq[ok]).sum())} outputs meeting the condition differ"
    rest = ~ok & ~eq
    if rest.any():
        ulps = np.abs(y[rest].view(np.int32).astype(np.int64) - ref[rest].view(np.int32).astype(np.int64))
        assert ulps.max() <= 1024


@pytest.mark.parametrize("shape", [(192, 256, 512), (130, 96, 208)])
def test_quantized_linear_close_to_oracle(shape):
    M, N, K = shape
    wl = inputs.make("linear_fwd", scale_rows=M)
    X = wl.tensors["X"].t[:, :K].contiguous()
    W = wl.tensors["W"].t[:N, :K].contiguous()
    gx, ox = quant_both(X, float(oracle.amax(inputs.bf16_bits(X))), "row16")
    gw, ow = quant_both(W, float(oracle.amax(inputs.bf16_bits(W))), "tile" if N % 16 == 0 else "row16")
    ref = oracle.gemm_probe(ox.q, ow.q).astype(np.float64)
    y = run_probe(gx["q"], gw["q"]).astype(np.float64)
    assert rel_fro(y, ref) < 1e-6
    # and both are close to the exact contraction
    assert rel_fro(ref, oracle.gemm(ox.q, ow.q)) < 1e-5


def test_empty_and_zero_length_contraction():
    rng = np.random.default_rng(0)
    ga, _ = random_operand(rng, 16, 0, api.ROW16, 0x70, 0x80)
    gb, _ = random_operand(rng, 32, 0, api.ROW16, 0x70, 0x80)
    y = run_probe(ga, gb, torch.float32, 10)
    assert y.shape == (16, 32) and not y.any()
    ge, _ = random_operand(rng, 0, 64, api.ROW16, 0x70, 0x80)
    gf, _ = random_operand(rng, 32, 64, api.ROW16, 0x70, 0x80)
    assert run_probe(ge, gf).shape == (0, 32)
