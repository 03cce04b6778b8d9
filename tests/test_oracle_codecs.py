"""Pins of the oracle's E2M1 and UE5M3 codecs.

Sources: "UE5M3 FP4 Block Scaling for Stable Language Model Pretraining"
(§2, §3, §4.1, §5.2) and "Rounding in Preconditioner Space: Redesigning 4-bit
AdamW Optimizer-State Quantization" (App. A.1 codebook, App. A.2 RTN/SR).

What pins what:
* E2M1 decode: the printed normalised codebook (x6) pins the six normal
  magnitudes and the maximum; the subnormal 0.5 is a reading (NVFP4/MXFP4
  E2M1), checked here only for gradual underflow (even spacing near zero).
* UE5M3 decode: all 256 codes against numpy's float16 of the bit pattern
  code << 7 (a library routine), plus the page's printed constants.
* Encoders: hand-worked examples and brute-force nearest search over the
  float16-derived codebook (independent of the oracle's decoder).
"""
import math
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _golden_lines(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return [ln.split() for ln in f if ln.strip() and not ln.startswith("#")]


def _pow2(tok):
    if tok.startswith("2^"):
        return 2.0 ** int(tok[2:])
    return float(tok)


def ue5m3_codebook_f16():
    """Decoded UE5M3 codebook from the float16 bit pattern code << 7."""
    bits = (np.arange(256, dtype=np.uint16) << 7).astype(np.uint16)
    return bits.view(np.float16).astype(np.float64)


# ------------------------------------------------------------------ E2M1
def test_e2m1_normals_match_printed_codebook():
    vals = [Fraction(v[0]) for v in _golden_lines("e2m1_codebook.txt")]
    scaled = sorted(float(6 * v) for v in vals)            # {0, 1/8, 1, 1.5, 2, 3, 4, 6}
    mags = sorted(oracle.e2m1_decode(c) for c in range(8))  # {0, 0.5, 1, 1.5, 2, 3, 4, 6}
    # zero, the six normal magnitudes and the maximum agree with the page
    assert mags[0] == scaled[0] == 0.0
    assert mags[2:] == scaled[2:]
    assert max(mags) == 6.0
    # sign symmetry, and both zero codes decode to zero
    for c in range(8):
        assert oracle.e2m1_decode(c | 8) == -oracle.e2m1_decode(c)
    assert oracle.e2m1_decode(0) == 0.0 and oracle.e2m1_decode(8) == 0.0
    assert math.copysign(1.0, oracle.e2m1_decode(8)) == -1.0
    # codes are monotone in magnitude
    assert all(oracle.e2m1_decode(c) < oracle.e2m1_decode(c + 1) for c in range(7))


def test_e2m1_subnormal_is_gradual_underflow():
    # READING (NVFP4/MXFP4 E2M1): the exponent-0 binade continues the spacing
    # of the first normal binade, so 0, 0.5, 1 are evenly spaced.
    v = [oracle.e2m1_decode(c) for c in range(4)]
    assert v[1] - v[0] == v[2] - v[1] == v[3] - v[2] == 0.5


def test_e2m1_rne_hand_worked_ties_and_saturation():
    # ties go to the even code: 0.25 -> 0 (code 0), 0.75 -> 1 (code 2),
    # 1.25 -> 1 (code 2), 1.75 -> 2 (code 4), 2.5 -> 2 (code 4),
    # 3.5 -> 4 (code 6), 5 -> 4 (code 6)
    cases = {0.25: 0, 0.75: 2, 1.25: 2, 1.75: 4, 2.5: 4, 3.5: 6, 5.0: 6,
             0.0: 0, 0.2: 0, 0.3: 1, 0.5: 1, 0.74: 1, 0.76: 2, 2.4: 4, 2.6: 5,
             4.9: 6, 5.1: 7, 6.0: 7, 6.5: 7, 1e30: 7, float("inf"): 7}
    for v, code in cases.items():
        assert oracle.e2m1_encode_rne(v) == code, v
        assert oracle.e2m1_encode_rne(-v) == (code | 8), -v
    assert oracle.e2m1_encode_rne(-0.0) == 8
    assert oracle.e2m1_encode_rne(float("nan"), negative=False) == 0
    assert oracle.e2m1_encode_rne(float("nan"), negative=True) == 8


def test_e2m1_rne_brute_force_sweep():
    rng = np.random.default_rng(123)
    mags = np.array([0, 0.5, 1, 1.5, 2, 3, 4, 6], np.float64)
    mids = (mags[1:] + mags[:-1]) / 2
    xs = np.concatenate([
        rng.uniform(0, 7, 4000).astype(np.float32),
        mids.astype(np.float32),
        np.nextafter(mids.astype(np.float32), np.float32(0)),
        np.nextafter(mids.astype(np.float32), np.float32(10)),
    ])
    for x in xs:
        a = min(float(x), 6.0)
        d = np.abs(mags - a)
        best = np.flatnonzero(d == d.min())
        want = best[0] if len(best) == 1 else [b for b in best if b % 2 == 0][0]
        assert oracle.e2m1_encode_rne(float(x)) == want, x


# ------------------------------------------------------------------ UE5M3
def test_ue5m3_decode_all_codes_against_float16_top_byte():
    cb = ue5m3_codebook_f16()
    for c in range(256):
        v = oracle.ue5m3_decode(c)
        if np.isnan(cb[c]):
            assert math.isnan(v), c
        else:
            assert v == cb[c], (c, v, cb[c])
    finite = [c for c in range(256) if math.isfinite(oracle.ue5m3_decode(c))]
    assert finite == list(range(0xF8))


def test_ue5m3_page_constants():
    g = {k: v for k, v in _golden_lines("ue5m3_page_constants.txt")}
    dec = [oracle.ue5m3_decode(c) for c in range(0xF8)]
    pos = [d for d in dec if d > 0]
    assert min(pos) == _pow2(g["min_subnormal"]) == oracle.ue5m3_decode(0x01)
    # smallest normal: the first code with a non-zero exponent field
    assert oracle.ue5m3_decode(0x08) == _pow2(g["min_normal"])
    assert max(pos) == float(g["max_finite"]) == oracle.ue5m3_decode(0xF7)
    e4m3_max = float(g["e4m3_max"])
    assert e4m3_max == torch.finfo(torch.float8_e4m3fn).max
    assert round(max(pos) / e4m3_max) == int(g["growth_T448"])        # 61440/448 = 137.1
    assert max(pos) / 2048 == float(g["growth_T2048"])                # 61440/2048 = 30
    assert round(2048 / 448, 1) == float(g["underflow_margin_T2048"])  # 4.57
    # E4M3 enumerated by the library dtype
    e4 = torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).float().numpy()
    e4_pos = e4[np.isfinite(e4) & (e4 > 0)]
    assert e4_pos.min() / min(pos) == float(g["subnormal_ratio_vs_e4m3"])  # 2^-9 / 2^-17
    # useful non-negative codes: 247 positive finite UE5M3 vs 126 positive finite E4M3
    assert len(pos) == 247 and len(np.unique(e4_pos)) == 126
    assert round(len(pos) / len(np.unique(e4_pos))) == int(g["useful_code_ratio"])


def _brute_ue5m3(raw):
    """Nearest of the float16-derived finite codebook, extended by 2^16 (0xF8)."""
    cb = ue5m3_codebook_f16()[:0xF8].tolist() + [65536.0]
    d = np.abs(np.array(cb) - float(raw))
    best = np.flatnonzero(d == d.min())
    return int(best[0] if len(best) == 1 else [b for b in best if b % 2 == 0][0])


def test_ue5m3_nearest_hand_worked():
    assert oracle.ue5m3_nearest(46.0) == 0xA4        # 44 and 48 tie; 48 (0xA4) is even
    assert oracle.ue5m3_nearest(42.0) == 0xA2        # 40 and 44 tie; 40 (0xA2) is even
    assert oracle.ue5m3_nearest(0.9375 * 2 ** -14) == 0x08
    assert oracle.ue5m3_nearest(2.0 ** -18) == 0x00  # tie between 0 and 2^-17: even code 0
    assert oracle.ue5m3_nearest(3 * 2.0 ** -19) == 0x01
    assert oracle.ue5m3_nearest(448.0) == 0xBE       # the default target
    assert oracle.ue5m3_nearest(2048.0) == 0xD0
    assert oracle.ue5m3_nearest(62000.0) == 0xF7
    assert oracle.ue5m3_nearest(63487.0) == 0xF7
    assert oracle.ue5m3_nearest(63488.0) == 0xF8     # midpoint to 2^16: even side overflows
    # repair
    assert oracle.ue5m3_encode(2.0 ** -18) == (0x01, 1)
    assert oracle.ue5m3_encode(0.0) == (0x01, 1)
    assert oracle.ue5m3_encode(63488.0) == (0xF7, 2)
    assert oracle.ue5m3_encode(float("inf")) == (0xF7, 2)
    assert oracle.ue5m3_encode(448.0) == (0xBE, 0)


def test_ue5m3_nearest_brute_force():
    cb = ue5m3_codebook_f16()[:0xF8].astype(np.float32)
    mids = ((cb[1:].astype(np.float64) + cb[:-1]) / 2).astype(np.float32)
    rng = np.random.default_rng(7)
    xs = np.concatenate([
        mids, np.nextafter(mids, np.float32(0)), np.nextafter(mids, np.float32(1e9)),
        cb, (2.0 ** rng.uniform(-20, 16.5, 3000)).astype(np.float32),
        np.array([63487.0, 63488.0, 63489.0, 65536.0, 1e6], np.float32),
    ])
    for x in xs:
        assert oracle.ue5m3_nearest(float(x)) == _brute_ue5m3(x), float(x)
