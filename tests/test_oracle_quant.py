"""Pins of the oracle's per-row quantiser (input preparation).

Checked with exact rational arithmetic (fractions.Fraction): the scale must be
the binary16 value nearest to max|row|/28 (ties to even), and each code the
e3m2 magnitude nearest to |W|/s (ties to the even code, saturating at 28),
with the sign bit copied from W.
"""

from fractions import Fraction

import numpy as np
import pytest

import oracle


_FP16_VALUES = []


def _fp16_values():
    # All finite non-negative binary16 values, ascending, as Fractions.
    if not _FP16_VALUES:
        bits = np.arange(0, 0x7C00, dtype=np.uint16)
        _FP16_VALUES.extend(Fraction(float(v)) for v in bits.view(np.float16).astype(np.float64))
    return _FP16_VALUES


def _exact_fp16_rne(x: Fraction) -> float:
    vals = _fp16_values()
    # binary search for neighbours
    lo, hi = 0, len(vals) - 1
    while hi - lo > 1:
        mid = (lo + hi) // 2
        if vals[mid] <= x:
            lo = mid
        else:
            hi = mid
    a, b = vals[lo], vals[hi]
    if x <= a:
        return float(a)
    if x - a < b - x:
        return float(a)
    if x - a > b - x:
        return float(b)
    return float(a) if lo % 2 == 0 else float(b)


def _exact_code(w: float, s: float) -> int:
    mags = [Fraction(m) for m in oracle.E3M2_VALUES[:32]]
    a = abs(Fraction(w)) / Fraction(s)
    d = [abs(a - m) for m in mags]
    best = min(d)
    c = [i for i, di in enumerate(d) if di == best]
    idx = c[0] if len(c) == 1 else [i for i in c if i % 2 == 0][0]
    return (32 if np.signbit(w) else 0) | idx


def test_quantize_matches_exact_rationals():
    rng = np.random.default_rng(21)
    W = rng.normal(0, 0.02, (6, 96)).astype(np.float32)
    W[1, 5] = -0.0
    W[2, :] *= 1e-3                      # tiny row: many subnormal codes
    codes, scales = oracle.quantize_rows(W)
    for n in range(W.shape[0]):
        amax = max(abs(Fraction(float(w))) for w in W[n])
        s = _exact_fp16_rne(amax / 28)
        assert float(scales[n]) == s
        for k in range(W.shape[1]):
            assert codes[n, k] == _exact_code(float(W[n, k]), s), (n, k)


def test_quantize_ties_go_to_even_code():
    # Build rows whose scale is exactly 2^-6 and put elements exactly on
    # e3m2 midpoints times the scale (exact in float32).
    s = 2.0 ** -6
    mids = [(a + b) / 2 for a, b in zip(oracle.E3M2_VALUES[:31], oracle.E3M2_VALUES[1:32])]
    row = np.array([28 * s] + [m * s for m in mids] + [-m * s for m in mids], dtype=np.float32)
    codes, scales = oracle.quantize_rows(row[None, :])
    assert float(scales[0]) == s
    got = codes[0, 1:32]
    # midpoint between index i and i+1 -> the even index
    want = [i if i % 2 == 0 else i + 1 for i in range(31)]
    assert got.tolist() == want
    assert codes[0, 32:].tolist() == [w | 32 for w in want]


def test_quantize_saturates_when_scale_rounds_down():
    # max|row| / 28 rounds down in fp16, so |W/s| slightly exceeds 28 -> code 31.
    amax = np.float32(28 * (1 + 2.0 ** -11) * 0.01)   # chosen so fp16(amax/28) < amax/28
    row = np.array([[amax, -amax, amax / 2]], dtype=np.float32)
    codes, scales = oracle.quantize_rows(row)
    assert float(amax) / float(scales[0]) > 28.0
    assert codes[0].tolist()[:2] == [31, 63]


def test_quantize_zero_row_and_signed_zero():
    W = np.zeros((2, 8), dtype=np.float32)
    W[1, 0] = 1.0
    W[1, 1] = -0.0
    W[1, 2] = -1e-6                     # rounds to -0
    codes, scales = oracle.quantize_rows(W)
    assert float(scales[0]) == 0.0 and codes[0].tolist() == [0] * 8
    assert codes[1, 0] == 31 and codes[1, 1] == 0x20 and codes[1, 2] == 0x20


def test_quantize_rejects_out_of_range_and_nonfinite():
    with pytest.raises(ValueError):
        oracle.quantize_rows(np.full((1, 4), 1000.0, dtype=np.float32))   # s >= 16
    with pytest.raises(ValueError):
        oracle.quantize_rows(np.array([[np.nan, 1.0]], dtype=np.float32))
    with pytest.raises(ValueError):
        oracle.quantize_rows(np.zeros((2, 2), dtype=np.float64))
