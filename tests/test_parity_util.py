"""The parity helpers' own logic, on the CPU: chunked oracle quantization
equals one oracle call on the whole tensor, and the elementwise GEMM bound
admits an fp32-accumulated evaluation while rejecting a planted error."""
import numpy as np
import pytest
import torch

import oracle
from fp4_block_scaled_fp4q_amd import inputs
from parity_util import check_gemm_elementwise, gemm_ref_and_bound, oracle_quantize_par, sub_operand


@pytest.mark.parametrize("layout", [oracle.ROW16, oracle.COL16, oracle.TILE16])
@pytest.mark.parametrize("rnd", [oracle.RNE, oracle.SR])
def test_chunked_oracle_quantize_equals_single_call(layout, rnd):
    rng = np.random.default_rng(3)
    x = inputs.bf16_bits(inputs.to_bf16(inputs.loguniform_grad(rng, 96, 1040)))
    a = float(oracle.amax(x))
    one = oracle.quantize(x, a, 448.0, layout, rnd, 5, 7, transposed=(layout == oracle.TILE16))
    q, qt = oracle_quantize_par(x, a, layout, rnd, seed=5, subseq=7, transposed=(layout == oracle.TILE16),
                                chunk=32)
    np.testing.assert_array_equal(q.codes, one.q.codes)
    np.testing.assert_array_equal(q.scales, one.q.scales)
    assert (q.rows, q.cols, q.layout) == (one.q.rows, one.q.cols, one.q.layout)
    if layout == oracle.TILE16:
        np.testing.assert_array_equal(qt.codes, one.qt.codes)
        np.testing.assert_array_equal(qt.scales, one.qt.scales)


def test_elementwise_bound_admits_fp32_accumulation_and_rejects_a_planted_error():
    rng = np.random.default_rng(4)
    A = inputs.activation(rng, 64, 512, inputs.outlier_columns(rng, 512))
    B = inputs.gaussian(rng, 96, 512, 0.02)
    qa = oracle.quantize(A, float(oracle.amax(A))).q
    qb = oracle.quantize(B, float(oracle.amax(B)), layout=oracle.TILE16).q
    ref, bound = gemm_ref_and_bound(qa, qb, torch.float32)
    # an fp32 evaluation: sequential fp32 sums of the decoded products
    da = oracle.decode_f64(qa).astype(np.float32)
    db = oracle.decode_f64(qb).astype(np.float32)
    acc = np.zeros((64, 96), np.float32)
    for k in range(512):
        acc = (acc + np.outer(da[:, k], db[:, k]).astype(np.float32)).astype(np.float32)
    alpha = np.float32(1.0 / (np.float64(qa.S) * np.float64(qb.S)))
    y = torch.from_numpy((acc * alpha).astype(np.float32))
    check_gemm_elementwise(y, ref, bound, "fp32 sequential")
    bad = y.clone()
    bad[5, 7] *= 1.001
    with pytest.raises(AssertionError):
        check_gemm_elementwise(bad, ref, bound, "planted")
    # a row band of a TILE operand keeps its tile scales
    sub = sub_operand(qb, 32, 32)
    np.testing.assert_array_equal(oracle.decode_f64(sub), oracle.decode_f64(qb)[32:64])


def test_lsb_exp_and_probe_exact_condition():
    """The lowest-set-bit exponent on known values, and the probe mode's
    exactness condition on slices whose products do and do not fit 24 bits
    above their common lowest bit."""
    from parity_util import lsb_exp, probe_exact_condition
    x = np.array([1.0, 0.75, 6.0, -0.5, 2.0 ** -30 * 3, 0.0])
    assert list(lsb_exp(x)[:5]) == [0, -2, 1, -1, -30]
    assert lsb_exp(x)[5] > 1000
    K = 128
    A = np.zeros((3, K))
    B = np.zeros((1, K))
    A[0, :2] = [1.0, 1.0]                  # products 1, 1: exact
    A[1, :2] = [1.0, 2.0 ** -30]           # products 1 and 2^-30: 31 bits apart
    A[2, 0], A[2, 64] = 1.0, 2.0 ** -30    # the same two products in different slices: exact
    B[0, :] = 1.0
    assert probe_exact_condition(A, B)[:, 0].tolist() == [True, False, True]
    # the boundary: 1 + 2^-24 needs 25 bits above the lowest (not exact),
    # 0.5 + 2^-24 and 1 + 2^-23 need 24 (exact)
    A2 = np.zeros((1, 64))
    for pair, want in (([1.0, 2.0 ** -24], False), ([0.5, 2.0 ** -24], True), ([1.0, 2.0 ** -23], True)):
        A2[0, :2] = pair
        assert probe_exact_condition(A2, np.ones((1, 64)))[0, 0] == want, pair
