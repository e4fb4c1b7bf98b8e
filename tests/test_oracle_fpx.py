"""Pins of the oracle's narrower formats: FP6 e2m3, FP5 e2m2, FP4 e2m1.

Each check ties the oracle to something other than itself: IEEE binary16
decoding (numpy) of the fp16 embedding of each code, the closed forms in
tests/golden/fpx_formats.txt, torch's float8 rounding where the grids agree,
numpy's rint (round-half-even) on a frexp decomposition, exact rational
arithmetic, brute force, and hand-derived packed-byte images in
tests/golden/packed_v3_onehot_fpx.txt.
"""

import os
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
from oracle import fp6_oracle as fo

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
NEW = ("e2m3", "e2m2", "e2m1")
# fp16 embedding: (s << 15) | (magnitude << SHIFT) encodes v * 2^-14 for these
# bias-1 formats (the 2-bit exponent lands in fp16's exponent bits 11..10).
SHIFT = {"e2m3": 7, "e2m2": 8, "e2m1": 9}


def _golden():
    rows = {}
    with open(os.path.join(GOLDEN, "fpx_formats.txt")) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            p = line.split()
            rows[p[0]] = dict(bits=int(p[1]), bias=int(p[2]), max_normal=float(p[3]),
                              min_normal=float(p[4]), max_subnormal=float(p[5]),
                              min_subnormal=float(p[6]), n_codes=int(p[7]))
    return rows


def _codes(fmt):
    return np.arange(1 << fo.FORMATS[fmt].bits, dtype=np.uint8)


@pytest.mark.parametrize("fmt", NEW)
def test_table_matches_ieee_fp16_embedding(fmt):
    c = _codes(fmt).astype(np.uint16)
    bits = fo.FORMATS[fmt].bits
    mag = c & ((1 << (bits - 1)) - 1)
    sgn = c >> (bits - 1)
    h = ((sgn << 15) | (mag << SHIFT[fmt])).view(np.float16).astype(np.float64) * 2.0 ** 14
    v = oracle.decode(_codes(fmt), fmt)
    assert np.array_equal(h, v)
    assert np.array_equal(np.signbit(h), np.signbit(v))


@pytest.mark.parametrize("fmt", NEW)
def test_table_closed_forms_and_golden(fmt):
    g = _golden()[fmt]
    f = fo.FORMATS[fmt]
    v = oracle.decode(_codes(fmt), fmt)
    half = f.nmag
    assert f.bits == g["bits"] and f.bias == g["bias"] and v.size == g["n_codes"]
    assert f.max == g["max_normal"] == v.max() == -v.min()
    assert v[1] == g["min_subnormal"] == 2.0 ** (1 - f.bias - f.mbits)
    msub = (1 << f.mbits) - 1
    assert v[msub] == g["max_subnormal"]
    assert v[msub + 1] == g["min_normal"] == 2.0 ** (1 - f.bias)
    # subnormal spacing continues into the first binade; spacing 2^(e-1-M) in binade e
    assert np.all(np.diff(v[0: msub + 2]) == g["min_subnormal"])
    for e in range(1, 1 << f.ebits):
        blk = v[e << f.mbits: (e + 1) << f.mbits]
        assert np.all(np.diff(blk) == 2.0 ** (e - f.bias - f.mbits))
    assert np.array_equal(v[half:], -v[:half])
    assert np.signbit(v[half]) and not np.signbit(v[0])
    assert np.all(np.diff(v[:half]) > 0)


@pytest.mark.parametrize("fmt", NEW)
def test_encode_round_trip_all_codes(fmt):
    v = oracle.decode(_codes(fmt), fmt)
    assert np.array_equal(oracle.encode_rne(v, fmt), _codes(fmt))


@pytest.mark.parametrize("fmt,tdtype,lo", [("e2m3", torch.float8_e4m3fn, 1.0),
                                           ("e2m2", torch.float8_e5m2, 1.0)])
def test_encode_matches_torch_float8_on_normal_range(fmt, tdtype, lo):
    # On [1, max] the e2m3 grid is the float8_e4m3fn grid (3 mantissa bits) and
    # the e2m2 grid is the float8_e5m2 grid (2 mantissa bits), so RNE onto
    # either must agree there.  x is float32 so torch rounds once.
    f = fo.FORMATS[fmt]
    rng = np.random.default_rng(41)
    a = rng.uniform(lo, f.max, 100_000).astype(np.float32)
    mags = f.mags[f.mags >= lo]
    mids = ((mags[:-1] + mags[1:]) / 2).astype(np.float32)
    x = np.concatenate([a, -a, mids, -mids])
    ref = torch.from_numpy(x).to(tdtype).to(torch.float64).numpy()
    got = oracle.decode(oracle.encode_rne(x.astype(np.float64), fmt), fmt)
    assert np.array_equal(got, ref)


@pytest.mark.parametrize("fmt", NEW)
def test_encode_matches_frexp_rint_definition(fmt):
    # Subnormal range |x| < 2^(1-bias): rint(|x| / q) * q with q the subnormal
    # step; normal range |x| = f * 2^E, f in [0.5, 1): rint(f * 2^(M+1)) /
    # 2^(M+1) * 2^E; saturate at the largest magnitude.
    f = fo.FORMATS[fmt]
    rng = np.random.default_rng(42)
    mn = 2.0 ** (1 - f.bias)
    q = 2.0 ** (1 - f.bias - f.mbits)
    a = np.concatenate([
        rng.uniform(0, mn, 50_000),
        np.exp(rng.uniform(np.log(mn), np.log(2 * f.max), 100_000)),
        f.mids, np.nextafter(f.mids, 0), np.nextafter(f.mids, 100),
    ])
    fr, E = np.frexp(a)
    ref = np.where(a < mn, np.rint(a / q) * q, np.ldexp(np.rint(fr * 2 ** (f.mbits + 1)) / 2 ** (f.mbits + 1), E))
    ref = np.minimum(ref, f.max)
    got = oracle.decode(oracle.encode_rne(a, fmt), fmt)
    assert np.array_equal(got, ref)


@pytest.mark.parametrize("fmt", NEW)
def test_encode_brute_force_argmin_even_tiebreak(fmt):
    f = fo.FORMATS[fmt]
    rng = np.random.default_rng(43)
    x = np.concatenate([rng.normal(0, 2, 3000), f.mids, -f.mids, [0.0, -0.0, 1e-300, -1e-300, 1e9]])
    mags = [Fraction(m) for m in f.mags.tolist()]
    for xi, ci in zip(x.tolist(), oracle.encode_rne(x, fmt).tolist()):
        a = abs(Fraction(xi))
        dists = [abs(a - m) for m in mags]
        best = min(dists)
        cands = [i for i, d in enumerate(dists) if d == best]
        idx = cands[0] if len(cands) == 1 else [i for i in cands if i % 2 == 0][0]
        sign = 1 if np.signbit(xi) else 0
        assert ci == (sign << (f.bits - 1)) | idx, (xi, ci)


@pytest.mark.parametrize("fmt", NEW)
def test_codes_out_of_range_rejected(fmt):
    bits = fo.FORMATS[fmt].bits
    with pytest.raises(ValueError):
        oracle.decode(np.array([1 << bits]), fmt)
    with pytest.raises(ValueError):
        oracle.pack_scalar(np.full((16, 256), 1 << bits, dtype=np.uint8), fmt)
    with pytest.raises(ValueError):
        oracle.decode(np.array([0]), "e9m9")


@pytest.mark.parametrize("fmt", NEW)
@pytest.mark.parametrize("mutation", ["swap", "sign", "subnormal"])
def test_pins_catch_planted_table_mistakes(monkeypatch, fmt, mutation):
    f = fo.FORMATS[fmt]
    t = f.table.copy()
    if mutation == "swap":
        t[[5, 6]] = t[[6, 5]]
    elif mutation == "sign":
        t[f.nmag + 3] = -t[f.nmag + 3]
    else:
        t[1] = t[1] * 1.5
    monkeypatch.setattr(f, "table", t)
    c = _codes(fmt).astype(np.uint16)
    mag = c & (f.nmag - 1)
    sgn = c >> (f.bits - 1)
    h = ((sgn << 15) | (mag << SHIFT[fmt])).view(np.float16).astype(np.float64) * 2.0 ** 14
    assert not np.array_equal(h, fo.decode(_codes(fmt), fmt))


# ---------------------------------------------------------------------------
# Quantiser, exact rationals.
# ---------------------------------------------------------------------------
def _exact_fp16_rne(x: Fraction) -> float:
    bits = np.arange(0, 0x7C00, dtype=np.uint16)
    vals = [Fraction(float(v)) for v in bits.view(np.float16).astype(np.float64)]
    lo, hi = 0, len(vals) - 1
    while hi - lo > 1:
        mid = (lo + hi) // 2
        if vals[mid] <= x:
            lo = mid
        else:
            hi = mid
    a, b = vals[lo], vals[hi]
    if x - a < b - x:
        return float(a)
    if x - a > b - x:
        return float(b)
    return float(a) if lo % 2 == 0 else float(b)


@pytest.mark.parametrize("fmt", NEW)
def test_quantize_matches_exact_rationals(fmt):
    f = fo.FORMATS[fmt]
    rng = np.random.default_rng(44)
    W = rng.normal(0, 0.02, (4, 64)).astype(np.float32)
    W[1, 5] = -0.0
    W[2, :] *= 1e-2
    codes, scales = oracle.quantize_rows(W, fmt)
    mags = [Fraction(m) for m in f.mags.tolist()]
    for n in range(W.shape[0]):
        amax = max(abs(Fraction(float(w))) for w in W[n])
        s = _exact_fp16_rne(amax / Fraction(f.max))
        assert float(scales[n]) == s
        for k in range(W.shape[1]):
            a = abs(Fraction(float(W[n, k]))) / Fraction(s)
            d = [abs(a - m) for m in mags]
            best = min(d)
            c = [i for i, di in enumerate(d) if di == best]
            idx = c[0] if len(c) == 1 else [i for i in c if i % 2 == 0][0]
            want = ((1 << (f.bits - 1)) if np.signbit(W[n, k]) else 0) | idx
            assert codes[n, k] == want, (n, k)


def test_quantize_scale_limits():
    # 4 for e2m3 / e2m2 (s * 2^14 must stay an exact fp16), none for e2m1.
    big = np.full((1, 4), 40.0, dtype=np.float32)     # s = 40/7.5 or 40/7 > 4
    for fmt in ("e2m3", "e2m2"):
        with pytest.raises(ValueError):
            oracle.quantize_rows(big, fmt)
    codes, scales = oracle.quantize_rows(big, "e2m1")
    assert float(scales[0]) == float(np.float16(40.0 / 6.0)) and codes[0].tolist() == [7] * 4


# ---------------------------------------------------------------------------
# Packed layout.
# ---------------------------------------------------------------------------
def _onehot_cases():
    cases = []
    with open(os.path.join(GOLDEN, "packed_v3_onehot_fpx.txt")) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            p = line.split()
            img = {int(o): int(v, 16) for o, v in (q.split(":") for q in p[4:])}
            cases.append((p[0], int(p[1]), int(p[2]), int(p[3]), img))
    return cases


@pytest.mark.parametrize("case", _onehot_cases(), ids=lambda c: f"{c[0]}-n{c[1]}k{c[2]}c{c[3]}")
def test_onehot_golden_images(case):
    fmt, n, k, code, img = case
    N, K = 32, 512
    buf = np.zeros(oracle.packed_bytes(N, K, fmt), dtype=np.uint8)
    for off, val in img.items():
        buf[off] = val
    codes = np.zeros((N, K), dtype=np.uint8)
    codes[n, k] = code
    assert np.array_equal(oracle.unpack_scalar(buf, N, K, fmt), codes)
    assert np.array_equal(oracle.unpack_tiles(buf, N, K, fmt), codes)
    assert np.array_equal(oracle.pack_scalar(codes, fmt), buf)


@pytest.mark.parametrize("fmt", ("e3m2",) + NEW)
def test_layout_is_a_bijection_on_one_tile(fmt):
    f = fo.FORMATS[fmt]
    seen = set()
    for n in range(16):
        for k in range(256):
            slots = fo._slots(f, 16, 256, n, k)
            assert sorted(c for _, _, c in slots) == list(range(f.bits))
            for off, bit, _ in slots:
                key = off * 8 + bit
                assert 0 <= bit < 32 and key not in seen
                seen.add(key)
    assert seen == set(range(oracle.tile_bytes(fmt) * 8))


@pytest.mark.parametrize("fmt", ("e3m2",) + NEW)
def test_round_trip_and_unpackers_agree(fmt):
    f = fo.FORMATS[fmt]
    rng = np.random.default_rng(45)
    N, K = 32, 512
    c = rng.integers(0, 1 << f.bits, (N, K)).astype(np.uint8)
    b = oracle.pack_scalar(c, fmt)
    assert b.size == N * K * f.bits // 8
    assert np.array_equal(oracle.unpack_scalar(b, N, K, fmt), c)
    assert np.array_equal(oracle.unpack_tiles(b, N, K, fmt), c)
    r = rng.integers(0, 256, b.size).astype(np.uint8)
    assert np.array_equal(oracle.unpack_scalar(r, N, K, fmt), oracle.unpack_tiles(r, N, K, fmt))
    if fmt == "e3m2":
        assert np.array_equal(oracle.unpack_np(r, N, K), oracle.unpack_tiles(r, N, K))


@pytest.mark.parametrize("fmt", NEW)
def test_dequant_ref_matches_torch_fp16_multiply(fmt):
    # torch CPU: float16(v) * float16(s) computed in float32 and rounded once
    # to fp16 equals fp16_RNE(v * s) (the product of a <= 4-bit and an 11-bit
    # significand is exact in float32).
    f = fo.FORMATS[fmt]
    rng = np.random.default_rng(46)
    c = rng.integers(0, 1 << f.bits, (8, 64)).astype(np.uint8)
    s = (rng.uniform(-3.9, 3.9, 8)).astype(np.float16)
    v = torch.from_numpy(oracle.decode(c, fmt).astype(np.float32))
    ref = (v * torch.from_numpy(s.astype(np.float32))[:, None]).to(torch.float16).numpy()
    got = oracle.dequant_ref(c, s, fmt)
    assert np.array_equal(got.view(np.uint16), ref.view(np.uint16))
