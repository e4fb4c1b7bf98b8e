"""Pins of the oracle's packed-layout-v3 unpackers (FP6 e3m2).

The hand-derived one-hot byte images in tests/golden/packed_v3_onehot.txt fix
the reading of the layout independently of the oracle's code; bijection and
cross-implementation checks cover every other position.
"""

import os

import numpy as np
import pytest

import oracle
from oracle import fp6_oracle as fo

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _onehot_cases():
    cases = []
    with open(os.path.join(GOLDEN, "packed_v3_onehot.txt")) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            parts = line.split()
            n, k, code = int(parts[0]), int(parts[1]), int(parts[2])
            img = {int(o): int(v, 16) for o, v in (p.split(":") for p in parts[3:])}
            cases.append((n, k, code, img))
    return cases


@pytest.mark.parametrize("case", _onehot_cases(), ids=lambda c: f"n{c[0]}k{c[1]}c{c[2]}")
def test_onehot_golden_images(case):
    n, k, code, img = case
    N, K = 32, 512
    buf = np.zeros(N * K * 3 // 4, dtype=np.uint8)
    for off, val in img.items():
        buf[off] = val
    codes = np.zeros((N, K), dtype=np.uint8)
    codes[n, k] = code
    assert np.array_equal(oracle.unpack_scalar(buf, N, K), codes)
    assert np.array_equal(oracle.unpack_np(buf, N, K), codes)
    assert np.array_equal(oracle.pack_scalar(codes), buf)


def test_layout_is_a_bijection_on_one_tile():
    # Every (row, k, code-bit) of a 16x256 tile maps to a distinct bit of the
    # 3072-byte tile, and together they cover all 24576 bits.
    seen = set()
    for n in range(16):
        for k in range(256):
            w2, b_e2, b_s, w4, nib = fo._locate(16, 256, n, k)
            pos = [(w2, b_e2), (w2, b_s)] + [(w4, nib + t) for t in range(4)]
            for off, bit in pos:
                key = off * 8 + bit
                assert key not in seen
                seen.add(key)
    assert seen == set(range(3072 * 8))


def test_round_trip_random_and_adversarial():
    rng = np.random.default_rng(31)
    N, K = 32, 512
    pats = [
        rng.integers(0, 64, (N, K)).astype(np.uint8),
        np.full((N, K), 63, dtype=np.uint8),
        (np.indices((N, K)).sum(axis=0) % 2 * 63).astype(np.uint8),
        (np.arange(N * K) % 64).reshape(N, K).astype(np.uint8),
    ]
    for c in pats:
        b = oracle.pack_scalar(c)
        assert b.size == N * K * 3 // 4
        assert np.array_equal(oracle.unpack_scalar(b, N, K), c)
        assert np.array_equal(oracle.unpack_np(b, N, K), c)


def test_unpackers_agree_on_random_bytes():
    rng = np.random.default_rng(32)
    for N, K in [(16, 256), (48, 768), (32, 512)]:
        b = rng.integers(0, 256, N * K * 3 // 4).astype(np.uint8)
        assert np.array_equal(oracle.unpack_scalar(b, N, K), oracle.unpack_np(b, N, K))


def test_shape_and_size_errors():
    with pytest.raises(ValueError):
        oracle.unpack_np(np.zeros(10, np.uint8), 16, 256)
    with pytest.raises(ValueError):
        oracle.unpack_np(np.zeros(16 * 100 * 3 // 4, np.uint8), 16, 100)
    with pytest.raises(ValueError):
        oracle.pack_scalar(np.zeros((8, 256), np.uint8))
