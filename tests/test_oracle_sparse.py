"""Pins of the 2:4-sparse oracle (oracle/sparse24.py).

* pruning: brute force over the 6 pairs of every group (the pair whose
  magnitudes, largest first, compare highest; then the lower indices), on
  small-integer magnitudes with many ties;
* compression / expansion: round trips and the dense route -- the dense FP6
  oracle (pinned on its own) applied to the pruned matrix must give exactly
  the sparse de-quantised weights;
* packed layout: hand-derived one-hot byte images (tests/golden/
  packed_24_onehot.txt), a bijection over every bit of a tile, round trips and
  agreement of the scalar and vectorised unpackers.
"""

import itertools
import os

import numpy as np
import pytest

import oracle
from oracle import sparse24 as sp

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def test_prune_matches_brute_force_pairs():
    rng = np.random.default_rng(51)
    W = (rng.integers(-3, 4, (40, 64)) * 0.5).astype(np.float32)   # many equal magnitudes
    W[0, :8] = 0.0
    mask = sp.prune_2of4(W)
    pairs = list(itertools.combinations(range(4), 2))               # lexicographic
    for n in range(W.shape[0]):
        for t in range(W.shape[1] // 4):
            a = np.abs(W[n, 4 * t: 4 * t + 4].astype(np.float64))
            # largest kept magnitudes: maximise the sorted magnitude pair
            # lexicographically (largest first), then prefer lower indices
            best = max(pairs, key=lambda p: (sorted([a[p[0]], a[p[1]]], reverse=True), [-p[0], -p[1]]))
            want = np.zeros(4, bool)
            want[list(best)] = True
            assert np.array_equal(mask[n, 4 * t: 4 * t + 4], want), (n, t, a)


def test_prune_properties():
    rng = np.random.default_rng(52)
    W = rng.normal(0, 1, (16, 256)).astype(np.float32)
    m = sp.prune_2of4(W).reshape(16, 64, 4)
    a = np.abs(W).reshape(16, 64, 4)
    assert (m.sum(axis=2) == 2).all()
    kept_min = np.where(m, a, np.inf).min(axis=2)
    drop_max = np.where(~m, a, -np.inf).max(axis=2)
    assert (kept_min >= drop_max).all()
    with pytest.raises(ValueError):
        sp.prune_2of4(np.zeros((2, 6), np.float32))


def test_compress_expand_round_trip():
    rng = np.random.default_rng(53)
    W = rng.normal(0, 1, (8, 128)).astype(np.float32)
    mask = sp.prune_2of4(W)
    vals, pos = sp.compress(W, mask)
    p2 = pos.reshape(8, 32, 2)
    assert (p2[:, :, 0] < p2[:, :, 1]).all() and pos.max() <= 3
    assert np.array_equal(sp.expand(vals, pos, 128), np.where(mask, W, 0.0))
    with pytest.raises(ValueError):
        sp.compress(W, np.ones_like(mask))


def test_sparse_dequant_equals_dense_route():
    # The dense FP6 oracle on the pruned matrix (pruned entries +0) must give
    # the sparse de-quantised weights bit for bit, scales included.
    rng = np.random.default_rng(54)
    W = rng.normal(0, 0.02, (32, 1024)).astype(np.float32)
    W[3] *= 1e-3
    W[4, :] = 0.0
    codes, pos, scales = sp.quantize_sparse(W)
    wdq = sp.dequant_ref(codes, pos, scales, 1024)
    pruned = np.where(sp.prune_2of4(W), W, np.float32(0.0)).astype(np.float32)
    dc, ds = oracle.quantize_rows(pruned)
    assert np.array_equal(ds.view(np.uint16), scales.view(np.uint16))
    ref = oracle.dequant_ref(dc, ds)
    assert np.array_equal(wdq.view(np.uint16), ref.view(np.uint16))
    # and the GEMM through the dense de-quantised matrix
    X = rng.normal(0, 1, (3, 1024)).astype(np.float16)
    assert np.array_equal(oracle.gemm_ref(X, wdq), oracle.gemm_ref(X, ref))


def _background(N, K):
    buf = np.zeros(sp.packed_bytes(N, K), np.uint8)
    for t in range((N // 16) * (K // 512)):
        buf[t * 4096 + 3072: (t + 1) * 4096] = 0x44
    return buf


def _cases():
    out = []
    with open(os.path.join(GOLDEN, "packed_24_onehot.txt")) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            p = line.split()
            img = {int(o): int(v, 16) for o, v in (q.split(":") for q in p[5:])}
            out.append((int(p[0]), int(p[1]), int(p[2]), int(p[3]), int(p[4]), img))
    return out


@pytest.mark.parametrize("case", _cases(), ids=lambda c: f"n{c[0]}t{c[1]}c{c[2]}")
def test_onehot_golden_images(case):
    n, t2, code, p0, p1, img = case
    N, K = 32, 1024
    codes = np.zeros((N, K // 2), np.uint8)
    pos = np.tile(np.array([0, 1], np.uint8), (N, K // 4))
    codes[n, t2] = code
    t = t2 // 2
    pos[n, 2 * t], pos[n, 2 * t + 1] = p0, p1
    buf = _background(N, K)
    for off, val in img.items():
        buf[off] = val
    assert np.array_equal(sp.pack_scalar(codes, pos, K), buf)
    c, p = sp.unpack_scalar(buf, N, K)
    assert np.array_equal(c, codes) and np.array_equal(p, pos)
    c, p = sp.unpack_tiles(buf, N, K)
    assert np.array_equal(c, codes) and np.array_equal(p, pos)


def test_layout_is_a_bijection_on_one_tile():
    seen = set()
    for r in range(16):
        for t2 in range(256):
            for off, bit, _ in sp._sparse_slots(16, 512, r, t2):
                key = off * 8 + bit
                assert 0 <= bit < 32 and key not in seen
                seen.add(key)
    assert seen == set(range(4096 * 8))


def test_element_map_matches_smfmac_operand_order():
    # Inverse check of the dense offset formula: every (step, lane group,
    # element) pair of a tile owns a distinct dense group, and both elements
    # of a pair (i, i+1 with i even) share it.
    seen = {}
    for j in range(8):
        for g in range(4):
            for i in range(8):
                off = 64 * j + 32 * (g % 2) + 16 * (i // 4) + 8 * (g // 2) + 4 * ((i % 4) // 2)
                jj, gg, ib = sp._element_of(off)
                assert (jj, gg, ib) == (j, g, i - i % 2)
                seen.setdefault(off, set()).add((g, i))
    assert len(seen) == 128 and all(len(v) == 2 for v in seen.values())


def test_round_trip_random_and_errors():
    rng = np.random.default_rng(55)
    N, K = 32, 1024
    codes = rng.integers(0, 64, (N, K // 2)).astype(np.uint8)
    W = rng.normal(0, 1, (N, K)).astype(np.float32)
    _, pos = sp.compress(W, sp.prune_2of4(W))
    b = sp.pack_scalar(codes, pos, K)
    assert b.size == N * K // 2
    c, p = sp.unpack_tiles(b, N, K)
    assert np.array_equal(c, codes) and np.array_equal(p, pos)
    r = rng.integers(0, 256, b.size).astype(np.uint8)
    assert all(np.array_equal(a, b_) for a, b_ in zip(sp.unpack_scalar(r, N, K), sp.unpack_tiles(r, N, K)))
    bad = pos.copy()
    bad[0, 0], bad[0, 1] = 2, 1
    with pytest.raises(ValueError):
        sp.pack_scalar(codes, bad, K)
    with pytest.raises(ValueError):
        sp.pack_scalar(codes[:, :256], pos[:, :256], 512 + 256)
