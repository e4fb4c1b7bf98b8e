"""Pins of the oracle's e3m2 decode table and round-to-nearest-even encoder.

Each check ties the oracle to something other than itself: IEEE binary16
decoding (numpy), torch's float8_e5m2 rounding (same 2-bit mantissa grid on
the normal range), numpy's rint (round-half-even) on a frexp decomposition,
exact rational arithmetic and brute force.
"""

import os
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
from oracle import fp6_oracle as fo

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _golden_format():
    vals = {}
    with open(os.path.join(GOLDEN, "e3m2_format.txt")) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            k, v = line.split()
            vals[k] = float(v)
    return vals


ALL = np.arange(64, dtype=np.uint8)


def test_table_matches_ieee_fp16_embedding():
    # e3m2 is binary16 with the exponent field narrowed: the fp16 pattern
    # (s << 15) | ((c & 31) << 8) encodes v(c) * 2^-12 exactly (normals and
    # subnormals alike).  numpy decodes the fp16 pattern independently.
    bits = ((ALL.astype(np.uint16) >> 5) << 15) | ((ALL.astype(np.uint16) & 31) << 8)
    h = bits.view(np.float16).astype(np.float64) * 4096.0
    v = oracle.decode(ALL)
    assert np.array_equal(h, v)
    assert np.array_equal(np.signbit(h), np.signbit(v))


def test_table_closed_forms_and_golden():
    g = _golden_format()
    v = oracle.decode(ALL)
    assert len(oracle.E3M2_VALUES) == int(g["n_codes"])
    assert v.max() == g["max_normal"] and v[31] == 28.0 and v[63] == -28.0
    assert v[1] == g["min_subnormal"] == 2.0 ** -4
    assert v[3] == g["max_subnormal"]
    assert v[4] == g["min_normal"] == 2.0 ** (1 - g["bias"])
    # subnormal spacing 2^-4 continues into the first binade
    assert np.all(np.diff(v[0:5]) == 2.0 ** -4)
    # spacing 2^(e-5) inside binade e = 1..7
    for e in range(1, 8):
        assert np.all(np.diff(v[4 * e: 4 * e + 4]) == 2.0 ** (e - 5))
    # odd symmetry and signed zero
    assert np.array_equal(v[32:], -v[:32])
    assert np.signbit(v[32]) and not np.signbit(v[0])
    # monotone magnitudes; 63 distinct values (+0 and -0 collide)
    assert np.all(np.diff(v[:32]) > 0)
    assert len(set(v.tolist())) == 63


def test_encode_round_trip_all_codes():
    v = oracle.decode(ALL)
    assert np.array_equal(oracle.encode_rne(v), ALL)


def test_encode_matches_torch_e5m2_on_normal_range():
    # On [0.25, 28) the e3m2 grid equals the float8_e5m2 grid (both keep two
    # mantissa bits, and e5m2's exponents cover 2^-2..2^4), so RNE onto either
    # grid must agree.  x is float32 so torch rounds once.
    rng = np.random.default_rng(11)
    a = rng.uniform(0.25, 28.0, 200_000).astype(np.float32)
    sgn = rng.choice([-1.0, 1.0], a.size).astype(np.float32)
    x = a * sgn
    # all midpoints of the normal range too (exact in float32)
    mids = ((fo._MAGS[4:-1] + fo._MAGS[5:]) / 2).astype(np.float32)
    x = np.concatenate([x, mids, -mids])
    ref = torch.from_numpy(x).to(torch.float8_e5m2).to(torch.float64).numpy()
    got = oracle.decode(oracle.encode_rne(x.astype(np.float64)))
    assert np.array_equal(got, ref)


def test_encode_matches_frexp_rint_definition():
    # Independent RNE definition with numpy's rint (round-half-even):
    # subnormal range |x| < 0.25: rint(|x| * 16) / 16; normal range:
    # |x| = f * 2^E with f in [0.5,1): rint(f * 8) / 8 * 2^E; saturate at 28.
    rng = np.random.default_rng(12)
    a = np.concatenate([
        rng.uniform(0, 0.25, 100_000),
        np.exp(rng.uniform(np.log(0.25), np.log(40.0), 200_000)),
        fo._MIDS,
        np.nextafter(fo._MIDS, 0), np.nextafter(fo._MIDS, 100),
    ])
    f, E = np.frexp(a)
    ref = np.where(a < 0.25, np.rint(a * 16) / 16, np.ldexp(np.rint(f * 8) / 8, E))
    ref = np.minimum(ref, 28.0)
    got = oracle.decode(oracle.encode_rne(a))
    assert np.array_equal(got, ref)


def test_encode_brute_force_argmin_even_tiebreak():
    rng = np.random.default_rng(13)
    x = np.concatenate([rng.normal(0, 6, 50_000), fo._MIDS, -fo._MIDS, [0.0, -0.0, 1e-300, -1e-300]])
    mags = np.array(oracle.E3M2_VALUES[:32])
    for xi, ci in zip(x[:5000].tolist() + x[-70:].tolist(),
                      oracle.encode_rne(np.concatenate([x[:5000], x[-70:]])).tolist()):
        a = abs(Fraction(xi))
        dists = [abs(a - Fraction(m)) for m in mags.tolist()]
        best = min(dists)
        cands = [i for i, d in enumerate(dists) if d == best]
        idx = cands[0] if len(cands) == 1 else [i for i in cands if i % 2 == 0][0]
        sign = 1 if np.signbit(xi) else 0
        assert ci == (sign << 5) | idx, (xi, ci)


def test_encode_saturation_and_specials():
    e = oracle.encode_rne
    assert e(np.array([28.0 * (1 + 2.0 ** -11)]))[0] == 31
    assert e(np.array([29.9, 30.0, 1e9, np.inf]))[0:4].tolist() == [31, 31, 31, 31]
    assert e(np.array([-1e9, -np.inf])).tolist() == [63, 63]
    assert e(np.array([-0.0]))[0] == 0x20
    assert e(np.array([-0.01]))[0] == 0x20          # rounds to -0
    assert e(np.array([0.03125]))[0] == 0            # tie 0 vs 1/16 -> even (0)
    assert e(np.array([0.09375]))[0] == 2            # tie 1/16 vs 2/16 -> even (2)
    assert e(np.array([26.0]))[0] == 30              # tie 24 vs 28 -> even code 30 (24)
    with pytest.raises(ValueError):
        e(np.array([np.nan]))


def test_fp16_rne_is_single_rounding():
    # Exact rational check of float64 -> float16 on neighbours of random halves.
    rng = np.random.default_rng(14)
    hs = rng.integers(0, 0x7BFF, 3000).astype(np.uint16)
    lo = hs.view(np.float16).astype(np.float64)
    hi = (hs + 1).astype(np.uint16).view(np.float16).astype(np.float64)
    mid = (lo + hi) / 2
    for l, h, m, b in zip(lo, hi, mid, hs):
        assert fo.fp16_rne(np.array([m]))[0] == (l if b % 2 == 0 else h)
        assert fo.fp16_rne(np.array([np.nextafter(m, 0)]))[0] == l
        assert fo.fp16_rne(np.array([np.nextafter(m, 1e9)]))[0] == h


@pytest.mark.parametrize("mutation", ["swap", "sign", "subnormal"])
def test_pins_catch_planted_table_mistakes(monkeypatch, mutation):
    # Plant a plausible mistake in the oracle's table and check that the
    # IEEE-embedding pin rejects it.
    t = fo.FORMATS["e3m2"].table.copy()
    if mutation == "swap":
        t[[9, 10]] = t[[10, 9]]
    elif mutation == "sign":
        t[40] = -t[40]
    else:
        t[2] = 0.0625 * 3
    monkeypatch.setattr(fo.FORMATS["e3m2"], "table", t)
    bits = ((ALL.astype(np.uint16) >> 5) << 15) | ((ALL.astype(np.uint16) & 31) << 8)
    h = bits.view(np.float16).astype(np.float64) * 4096.0
    assert not np.array_equal(h, fo.decode(ALL))
