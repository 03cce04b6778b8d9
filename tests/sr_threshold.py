"""Inputs that put stochastic rounding exactly on its decision boundaries.

For an element with Philox word w (the oracle's generator, keyed by the
element's row-major index) the rule rounds |v| up iff w < ceil(p 2^32), p
the position of |v| between its neighbours. threshold_tensor builds an fp32
tensor in which every element sits at the last value that rounds down or the
first that rounds up for its own word, in every interval of the E2M1 grid
(the subnormal interval [0, 0.5) included, where the threshold is taken with
a ceiling), with a 6.0 in every 16-element row block and 16-row column block
(held amax 6 and T = 448 then give r = 1, so the payload rule sees each value
itself). It returns the tensor and the magnitude code each element must get."""
from __future__ import annotations

import numpy as np

import oracle

# (lower level, gap, P granularity as a power of two) of each interval:
# P = p 2^32 moves in steps of ulp(|v|) 2^32 / gap
_INTERVALS = [(0.5, 0.5, 9), (1.0, 0.5, 10), (1.5, 0.5, 10), (2.0, 1.0, 10), (3.0, 1.0, 10), (4.0, 2.0, 10)]
_LEVELS = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]


def _rd24(w: int) -> int:
    s = max(w.bit_length() - 24, 0)
    return (w >> s) << s


def _ru24(w: int) -> int:
    s = max(w.bit_length() - 24, 0)
    t = ((w + (1 << s) - 1) >> s) << s
    return t if t.bit_length() <= 24 + s else _ru24(t)


def threshold_tensor(rows: int, cols: int, seed: int, subseq: int, rng_seed: int = 0):
    assert rows % 16 == 0 and cols % 16 == 0
    rng = np.random.default_rng(rng_seed)
    x = np.zeros((rows, cols), np.float32)
    want = np.zeros((rows, cols), np.int64)  # magnitude code (0..7)
    for r in range(rows):
        for c in range(cols):
            if c % 16 == r % 16:
                x[r, c] = 6.0
                want[r, c] = 7
                continue
            i = r * cols + c
            w = oracle.sr_word(seed, subseq, i)
            up = bool(rng.integers(2))
            kind = int(rng.integers(len(_INTERVALS) + 1))
            if kind == len(_INTERVALS):
                # [0, 0.5): P = ceil(a 2^33), a a 24-bit value times 2^-33
                if up:
                    t = _ru24(w + 1) if w + 1 < 2 ** 32 else None
                else:
                    t = _rd24(w)
                if t is None or t >= 2 ** 32:
                    t, up = _rd24(w), False
                a = np.float32(np.ldexp(float(t), -33))
                lo_code = 0
            else:
                lo, gap, g = _INTERVALS[kind]
                P = (w >> g) << g
                if up:
                    P += 1 << g
                if P >= 2 ** 32:
                    P, up = (w >> g) << g, False
                a = np.float32(lo + np.ldexp(float(P), -32) * gap)
                assert float(a) == lo + P * 2.0 ** -32 * gap  # exact
                lo_code = _LEVELS.index(lo)
            x[r, c] = -a if rng.integers(2) else a
            want[r, c] = lo_code + int(up)
    return x, want
