"""Pins of the oracle's block-32 and E4M3-scale variants ("UE5M3 FP4 Block
Scaling for Stable Language Model Pretraining": NVFP4's E4M3 block scale, §3
and §4.1; the block-32 run, §7.3)."""
import numpy as np
import pytest
import torch

import oracle


def test_e4m3_decode_matches_torch_float8():
    # torch's float8_e4m3fn is an independent implementation of the format
    codes = np.arange(0x7F, dtype=np.uint8)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).float().numpy()
    got = np.array([oracle.e4m3_decode(int(c)) for c in codes], np.float64)
    np.testing.assert_array_equal(got, ref.astype(np.float64))
    assert np.isnan(oracle.e4m3_decode(0x7F))


def test_e4m3_page_constants():
    # largest finite 448 and smallest subnormal 2^-9; against UE5M3 the page
    # states a maximum about 137 times larger and a minimum 256 times smaller
    assert oracle.e4m3_decode(0x7E) == 448.0
    assert oracle.e4m3_decode(0x01) == 2.0 ** -9
    assert round(oracle.ue5m3_decode(0xF7) / oracle.e4m3_decode(0x7E)) == 137
    assert oracle.e4m3_decode(0x01) / oracle.ue5m3_decode(0x01) == 256.0


def test_e4m3_encode_matches_torch_rounding():
    # in range, the pre-repair nearest code is torch's round-to-nearest-even
    # conversion to float8_e4m3fn (for raw above 2^-10, where no repair acts)
    rng = np.random.default_rng(2)
    raw = np.concatenate([
        np.exp2(rng.uniform(-10, np.log2(464.0), 20000)),
        np.array([oracle.e4m3_decode(c) for c in range(1, 0x7F)]),
        # midpoints between neighbouring codes (ties)
        np.array([(oracle.e4m3_decode(c) + oracle.e4m3_decode(c + 1)) / 2 for c in range(1, 0x7E)]),
    ]).astype(np.float32)
    raw = raw[raw > 2.0 ** -10]
    ref = torch.from_numpy(raw).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    got = np.array([oracle.e4m3_encode(float(r))[0] for r in raw], np.uint8)
    np.testing.assert_array_equal(got, ref)


def test_e4m3_repair():
    assert oracle.e4m3_encode(464.0) == (0x7E, 0)            # tie to the even code 448
    nxt = float(np.nextafter(np.float32(464.0), np.float32(1e9)))
    assert oracle.e4m3_encode(nxt) == (0x7E, 2)              # would round to 480: saturated
    assert oracle.e4m3_encode(1e30) == (0x7E, 2)
    assert oracle.e4m3_encode(2.0 ** -10) == (0x01, 1)       # tie to 0: zero-rounded
    above = float(np.nextafter(np.float32(2.0 ** -10), np.float32(1.0)))
    assert oracle.e4m3_encode(above) == (0x01, 0)


def test_e4m3_hand_worked_block():
    # A = 6, T = 448: S = 448; a block with amax 6 gets raw = 448 -> code
    # 0x7E, dec = 448, r = 1: payloads are the RNE codes of x itself
    x = np.array([[6.0, -3.0, 0.75, 1.25] + [0.0] * 12], np.float32)
    q = oracle.quantize(x, 6.0, layout=oracle.ROW16, scale_fmt=oracle.E4M3).q
    assert q.S == np.float32(448.0)
    assert q.scales[0, 0] == 0x7E
    assert q.codes[0, 0] == (0x7 | (0xD << 4))   # 6 -> 0x7, -3 -> 0xD
    assert q.codes[0, 1] == (0x2 | (0x2 << 4))   # ties: 0.75 -> 1.0 and 1.25 -> 1.0 (even code 2)
    # the same block in UE5M3 gets code 0xBE (448) and the same payloads
    u = oracle.quantize(x, 6.0, layout=oracle.ROW16).q
    assert u.scales[0, 0] == 0xBE
    np.testing.assert_array_equal(u.codes, q.codes)


@pytest.mark.parametrize("fmt", [oracle.UE5M3, oracle.E4M3])
def test_block32_equals_block16_when_halves_share_the_maximum(fmt):
    # if both 16-halves of every 32-block have the same amax, the block-32
    # scales are every other block-16 scale and the payloads coincide
    rng = np.random.default_rng(4)
    x = rng.standard_normal((8, 128)).astype(np.float32)
    x[:, 0::16] = 7.5  # the same maximum in every 16-half
    A = 7.5
    q32 = oracle.quantize(x, A, layout=oracle.ROW16, block=32, scale_fmt=fmt).q
    q16 = oracle.quantize(x, A, layout=oracle.ROW16, block=16, scale_fmt=fmt).q
    np.testing.assert_array_equal(q32.codes, q16.codes)
    np.testing.assert_array_equal(q32.scales, q16.scales[:, 0::2])


@pytest.mark.parametrize("fmt", [oracle.UE5M3, oracle.E4M3])
def test_block32_layouts_commute_with_transpose(fmt):
    rng = np.random.default_rng(6)
    x = rng.standard_normal((64, 96)).astype(np.float32)
    A = float(np.abs(x).max())
    col = oracle.quantize(x, A, layout=oracle.COL16, block=32, scale_fmt=fmt).q
    row_t = oracle.quantize(np.ascontiguousarray(x.T), A, layout=oracle.ROW16, block=32, scale_fmt=fmt).q
    np.testing.assert_array_equal(col.codes, row_t.codes)
    np.testing.assert_array_equal(col.scales, row_t.scales)
    t = oracle.quantize(x, A, layout=oracle.TILE16, block=32, scale_fmt=fmt, transposed=True)
    tt = oracle.quantize(np.ascontiguousarray(x.T), A, layout=oracle.TILE16, block=32, scale_fmt=fmt).q
    np.testing.assert_array_equal(t.qt.codes, tt.codes)
    np.testing.assert_array_equal(t.qt.scales, tt.scales)
    assert t.q.scales.shape == (2, 3)


@pytest.mark.parametrize("fmt", [oracle.UE5M3, oracle.E4M3])
def test_block32_exact_round_trip(fmt):
    # values e2m1 * 2^k with each 32-block's maximum 6 * 2^k round-trip
    # exactly (the scale is a power of two times T / A)
    rng = np.random.default_rng(8)
    mags = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0], np.float32)
    x = mags[rng.integers(0, 8, (32, 64))] * np.where(rng.integers(0, 2, (32, 64)) == 0, -1, 1)
    x = x.astype(np.float32)
    x[:, 0::32] = 6.0
    k = np.exp2(rng.integers(-3, 3, (32, 2))).astype(np.float32)
    x = x * np.repeat(k, 32, axis=1)
    A = float(np.abs(x).max())
    q = oracle.quantize(x, A, layout=oracle.ROW16, block=32, scale_fmt=fmt).q
    np.testing.assert_array_equal(oracle.dequant_f32(q), x)
