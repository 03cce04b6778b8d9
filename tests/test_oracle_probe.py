"""Pins of the oracle's probe-matched GEMM numerics ("UE5M3 FP4 Block Scaling
for Stable Language Model Pretraining", §6 and Appendix B/C): 64-wide slice
dot products rounded once to binary32, slice partials added with binary32
additions rounded toward zero, an optional snap of the accumulator to
multiples of 1/1024, then the tensor-scale product."""
from fractions import Fraction

import numpy as np
import pytest

import oracle


def lattice(rng, shape, lo_exp, hi_exp):
    """Random decoded-operand values: e2m1 magnitude times a power of two and
    a 4-bit significand (like e2m1 * UE5M3), random sign."""
    e2m1 = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])
    mag = e2m1[rng.integers(0, 8, size=shape)]
    sig = (8 + rng.integers(0, 8, size=shape)) / 8.0
    ex = rng.integers(lo_exp, hi_exp + 1, size=shape).astype(np.float64)
    sign = np.where(rng.integers(0, 2, size=shape) == 0, -1.0, 1.0)
    return sign * mag * sig * np.exp2(ex)


def test_rtz_cross_slice_addition_hand_worked():
    # slice 0 sums to 1, slice 1 to 3 * 2^-25 = 0.75 ulp(1): nearest would
    # give 1 + 2^-23, toward zero keeps 1 (and -1 for the negated operands)
    A = np.zeros((2, 128))
    B = np.zeros((1, 128))
    A[0, 0], B[0, 0] = 1.0, 1.0
    A[0, 64], B[0, 64] = 1.5 * 2.0 ** -12, 2.0 ** -12
    A[1] = -A[0]
    y = oracle.gemm_probe_decoded(A, B)
    assert y[0, 0] == np.float32(1.0)
    assert y[1, 0] == np.float32(-1.0)
    # the same two products inside one slice are summed exactly, then rounded
    # to nearest: 1 + 0.75 ulp -> 1 + ulp
    A2 = np.zeros((1, 64))
    B2 = np.zeros((1, 64))
    A2[0, 0], B2[0, 0] = 1.0, 1.0
    A2[0, 1], B2[0, 1] = 1.5 * 2.0 ** -12, 2.0 ** -12
    y2 = oracle.gemm_probe_decoded(A2, B2)
    assert y2[0, 0] == np.float32(1.0 + 2.0 ** -23)


def test_exact_when_all_sums_are_representable():
    # small dyadic values: every slice sum and every running sum is exact in
    # binary32, so the result is the exact contraction (times alpha = 1)
    rng = np.random.default_rng(3)
    A = lattice(rng, (7, 320), -2, 1)
    B = lattice(rng, (5, 320), -2, 1)
    y = oracle.gemm_probe_decoded(A, B)
    exact = A @ B.T  # exact in float64 for these magnitudes
    assert np.array_equal(y.astype(np.float64), exact)


def test_single_slice_is_the_nearest_binary32_of_the_exact_sum():
    # wide magnitude spread: the 64-term sum is not representable; the
    # oracle's value must be the binary32 nearest to the exact rational sum
    rng = np.random.default_rng(5)
    A = lattice(rng, (6, 64), -14, 14)
    B = lattice(rng, (4, 64), -14, 14)
    y = oracle.gemm_probe_decoded(A, B)
    for i in range(6):
        for j in range(4):
            exact = sum(Fraction(float(A[i, t])) * Fraction(float(B[j, t])) for t in range(64))
            f = np.float32(y[i, j])
            lo = np.nextafter(f, np.float32(-np.inf))
            hi = np.nextafter(f, np.float32(np.inf))
            d = abs(exact - Fraction(float(f)))
            assert d <= abs(exact - Fraction(float(lo))) and d <= abs(exact - Fraction(float(hi)))
            if d == abs(exact - Fraction(float(lo))) or d == abs(exact - Fraction(float(hi))):
                assert int(f.view(np.uint32)) % 2 == 0  # a tie goes to the even significand


def test_partials_added_toward_zero_in_order():
    # three slices with partials 1, 0.75 ulp(1), 0.75 ulp(1): toward zero
    # after each addition keeps 1 both times (nearest would reach 1 + 2 ulp)
    A = np.zeros((1, 192))
    B = np.zeros((1, 192))
    A[0, 0], B[0, 0] = 1.0, 1.0
    for g in (1, 2):
        A[0, 64 * g], B[0, 64 * g] = 1.5 * 2.0 ** -12, 2.0 ** -12
    assert oracle.gemm_probe_decoded(A, B)[0, 0] == np.float32(1.0)


def test_snap_dead_zone_and_ties():
    # the 1/1024 snap maps accumulators in [-1/2048, 1/2048] to zero and
    # rounds halfway cases to the even multiple
    def one(c):
        A = np.array([[c]], np.float64)
        B = np.array([[1.0]], np.float64)
        return float(oracle.gemm_probe_decoded(A, B, snap_log2=10)[0, 0])
    for c in (2.0 ** -11, -(2.0 ** -11), 2.0 ** -12, 1.5 * 2.0 ** -12):
        assert one(c) == 0.0
    assert one(3 * 2.0 ** -11) == 2.0 / 1024   # 1.5 -> 2
    assert one(5 * 2.0 ** -11) == 2.0 / 1024   # 2.5 -> 2
    assert one(7 * 2.0 ** -11) == 4.0 / 1024   # 3.5 -> 4
    assert one(1.25) == 1.25                   # already on the grid


def test_alpha_applied_after_the_accumulation():
    rng = np.random.default_rng(9)
    A = lattice(rng, (3, 128), -2, 1)
    B = lattice(rng, (2, 128), -2, 1)
    y1 = oracle.gemm_probe_decoded(A, B, 1.0, 1.0)
    y = oracle.gemm_probe_decoded(A, B, 4.0, 8.0)
    assert np.array_equal(y, (y1 * np.float32(1.0 / 32.0)).astype(np.float32))


def test_toward_zero_contracts_magnitudes():
    # Appendix C: toward-zero accumulation shrinks magnitudes slightly (on the
    # order of a part per million) without changing direction
    rng = np.random.default_rng(11)
    A = lattice(rng, (16, 4096), -8, -4)
    B = lattice(rng, (16, 4096), -8, -4)
    y = oracle.gemm_probe_decoded(A, B).astype(np.float64)
    exact = A @ B.T
    ratio = np.linalg.norm(y) / np.linalg.norm(exact)
    assert 1.0 - 1e-5 < ratio < 1.0
    cos = float(np.sum(y * exact) / (np.linalg.norm(y) * np.linalg.norm(exact)))
    assert cos > 1.0 - 1e-9


def test_quantized_operands_path_matches_decoded_path():
    rng = np.random.default_rng(13)
    x = rng.standard_normal((32, 192)).astype(np.float32)
    w = (0.02 * rng.standard_normal((48, 192))).astype(np.float32)
    xq = oracle.quantize(x, oracle.amax(x)).q
    wq = oracle.quantize(w, oracle.amax(w), layout=oracle.TILE16).q
    y = oracle.gemm_probe(xq, wq)
    y2 = oracle.gemm_probe_decoded(oracle.decode_f64(xq), oracle.decode_f64(wq), xq.S, wq.S)
    assert np.array_equal(y, y2)
    # close to the exact contraction
    ref = oracle.gemm(xq, wq)
    assert np.linalg.norm(y - ref) / np.linalg.norm(ref) < 1e-6
