"""Pins of the oracle's dequantisation and float64 GEMM.

Dequantisation is checked against binary16 closed forms and against torch's
CPU float16 multiply (which forms the product in float32, exact for a 3-bit by
11-bit significand, then rounds once); the GEMM against a naive triple loop on
every shape up to 8x8x8, against math.fsum, and on one-hot inputs.
"""

import math

import numpy as np
import pytest
import torch

import oracle

ALL = np.arange(64, dtype=np.uint8)


def _bits(h):
    return np.asarray(h, dtype=np.float16).view(np.uint16)


def test_dequant_closed_forms_unit_scale():
    codes = ALL[None, :]
    wdq = oracle.dequant_ref(codes, np.array([1.0], np.float16))
    b = _bits(wdq)[0]
    assert b[1] == 0x2C00 and b[31] == 0x4F00 and b[0x20] == 0x8000 and b[0] == 0
    # s = 1 reproduces v exactly; the fp16 pattern is (s<<15)|((c&31)<<8) + 12 in exponent
    assert np.array_equal(wdq.astype(np.float64)[0], oracle.decode(ALL))


@pytest.mark.parametrize("j", list(range(-24, 4)))
def test_dequant_power_of_two_scales_vs_torch(j):
    s = np.float16(2.0 ** j)
    wdq = oracle.dequant_ref(ALL[None, :], np.array([s]))
    v16 = torch.tensor(oracle.decode(ALL), dtype=torch.float16)
    ref = (v16 * torch.tensor(float(s), dtype=torch.float16)).numpy()
    assert np.array_equal(_bits(wdq)[0], _bits(ref))


def test_dequant_random_scales_full_range_vs_torch():
    rng = np.random.default_rng(41)
    # every finite binary16 magnitude below 16 (subnormals included), random sign
    sb = rng.integers(1, 0x4C00, 512).astype(np.uint16)
    sb |= (rng.integers(0, 2, 512).astype(np.uint16) << 15)
    s = sb.view(np.float16)
    codes = rng.integers(0, 64, (512, 64)).astype(np.uint8)
    wdq = oracle.dequant_ref(codes, s)
    ref = (torch.tensor(oracle.decode(codes), dtype=torch.float16)
           * torch.from_numpy(s.copy())[:, None]).numpy()
    assert np.array_equal(_bits(wdq), _bits(ref))


def test_gemm_ref_vs_naive_all_small_shapes():
    rng = np.random.default_rng(42)
    for M in range(1, 9):
        for N in range(1, 9):
            for K in range(1, 9):
                X = rng.standard_normal((M, K)).astype(np.float16)
                W = rng.standard_normal((N, K)).astype(np.float16)
                a = oracle.gemm_ref(X, W)
                b = oracle.gemm_naive(X, W)
                assert a.shape == (M, N)
                assert np.allclose(a, b, rtol=1e-12, atol=1e-12), (M, N, K)


def test_gemm_ref_vs_exact_fsum():
    rng = np.random.default_rng(43)
    X = rng.standard_normal((3, 1024)).astype(np.float16)
    W = rng.standard_normal((5, 1024)).astype(np.float16)
    Y = oracle.gemm_ref(X, W)
    for m in range(3):
        for n in range(5):
            exact = math.fsum(float(x) * float(w) for x, w in zip(X[m], W[n]))
            assert abs(Y[m, n] - exact) <= 1e-12 * (1 + abs(exact))


def test_gemm_one_hot_and_zero():
    rng = np.random.default_rng(44)
    W = rng.standard_normal((24, 16)).astype(np.float16)
    X = np.eye(16, dtype=np.float16)[[3, 0, 15]]
    Y = oracle.gemm_ref(X, W)
    assert np.array_equal(Y, W[:, [3, 0, 15]].T.astype(np.float64))
    assert not np.any(oracle.gemm_ref(np.zeros((2, 16), np.float16), W))


def test_tolerance_report_accepts_rounding_and_rejects_mistakes():
    rng = np.random.default_rng(45)
    X = rng.standard_normal((16, 512)).astype(np.float16)
    codes = rng.integers(0, 64, (64, 512)).astype(np.uint8)
    s = np.full(64, 0.003, np.float16)
    wdq = oracle.dequant_ref(codes, s)
    R = oracle.gemm_ref(X, wdq)
    assert oracle.tolerance_report(R.astype(np.float16), R)["ok"]
    # dropped k-term
    bad = oracle.gemm_ref(X[:, 1:], wdq[:, 1:])
    assert not oracle.tolerance_report(bad, R)["ok"]
    # wrong sign on one weight row
    w2 = wdq.copy()
    w2[7] = -w2[7]
    assert not oracle.tolerance_report(oracle.gemm_ref(X, w2), R)["ok"]
    # transposed index (rows of Y permuted)
    assert not oracle.tolerance_report(R[::-1], R)["ok"]
    # NaN never passes
    Rn = R.copy()
    Rn[0, 0] = np.nan
    assert not oracle.tolerance_report(Rn, R)["ok"]
