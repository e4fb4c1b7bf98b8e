"""Host-side library tests (no GPU): exported symbols, quantiser and packer
parity with the oracle, and every argument error the C ABI can return before
touching the GPU."""

import ctypes
import os
import re

import numpy as np
import pytest

import oracle
import weight_only_fp6_amd as fp6
from weight_only_fp6_amd import synth

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared_functions():
    names = []
    for fn in os.listdir(os.path.join(ROOT, "include")):
        if fn.endswith(".h"):
            txt = open(os.path.join(ROOT, "include", fn)).read()
            txt = re.sub(r"/\*.*?\*/", "", txt, flags=re.S)
            names += re.findall(r"\b(fp(?:6s|6|x)_\w+)\s*\(", txt)
    return sorted(set(names))


def test_library_exports_every_declared_symbol():
    names = _declared_functions()
    assert len(names) >= 9
    for n in names:
        assert hasattr(fp6.lib, n), n
    assert set(names) == set(fp6.EXPORTED)


def test_version_sizes_and_status_strings():
    assert fp6.pack_version() == 3
    assert fp6.packed_bytes(16, 256) == 3072
    assert fp6.packed_bytes(28672, 8192) == 176_160_768
    for bad in [(0, 256), (16, 0), (8, 256), (16, 128), (16, 300), (2**25, 256), (2**24, 2**24)]:
        assert fp6.packed_bytes(*bad) == 0
    for s in range(10):
        assert fp6.lib.fp6_status_string(s)


@pytest.mark.parametrize("shape", [(5, 7), (16, 256), (37, 1000)])
def test_quantizer_matches_oracle_random(shape):
    W = synth.weights(*shape, seed=7 + shape[0])
    c_lib, s_lib = fp6.quantize_rows(W)
    c_ref, s_ref = oracle.quantize_rows(W)
    assert np.array_equal(s_lib.view(np.uint16), s_ref.view(np.uint16))
    assert np.array_equal(c_lib, c_ref)


def test_quantizer_matches_oracle_adversarial():
    rng = np.random.default_rng(5)
    rows = []
    # exact e3m2 midpoints times a power-of-two scale (ties), saturation, zeros
    s = 2.0 ** -6
    mids = [(a + b) / 2 for a, b in zip(oracle.E3M2_VALUES[:31], oracle.E3M2_VALUES[1:32])]
    rows.append(np.array([28 * s] + [m * s for m in mids] + [-m * s for m in mids] + [0.0] * 1, np.float32))
    rows.append(np.zeros(64, np.float32))
    r = np.zeros(64, np.float32)
    r[3] = -0.0
    r[4] = np.float32(28 * (1 + 2.0 ** -11) * 0.01)
    r[5] = -1e-9
    rows.append(r)
    rows.append((rng.standard_normal(64) * 1e-6).astype(np.float32))       # subnormal scales
    rows.append((rng.standard_normal(64) * 100).astype(np.float32))        # large scales
    width = max(len(x) for x in rows)
    W = np.zeros((len(rows), width), np.float32)
    for i, x in enumerate(rows):
        W[i, : len(x)] = x
    c_lib, s_lib = fp6.quantize_rows(W)
    c_ref, s_ref = oracle.quantize_rows(W)
    assert np.array_equal(s_lib.view(np.uint16), s_ref.view(np.uint16))
    assert np.array_equal(c_lib, c_ref)


def test_quantizer_errors():
    with pytest.raises(fp6.FP6Error) as e:
        fp6.quantize_rows(np.full((2, 4), 1000.0, np.float32))
    assert e.value.name == "FP6_E_SCALE"
    with pytest.raises(fp6.FP6Error) as e:
        fp6.quantize_rows(np.array([[1.0, np.inf]], np.float32))
    assert e.value.name == "FP6_E_VALUE"
    assert fp6.lib.fp6_quantize_rows(None, 1, 1, None, None) == 1


@pytest.mark.parametrize("shape", [(16, 256), (32, 512), (48, 768)])
def test_prepack_matches_oracle_packer_bytewise(shape):
    codes = synth.codes_uniform(*shape, seed=shape[1])
    scales = np.ones(shape[0], np.float16)
    got = fp6.prepack(codes, scales)
    assert got.size == shape[0] * shape[1] * 3 // 4
    assert np.array_equal(got, oracle.pack_scalar(codes))
    assert np.array_equal(oracle.unpack_scalar(got, *shape), codes)


def test_prepack_round_trip_llama_shape():
    # a full-size row block of the Llama-70B MLP (K = 8192) and a ragged-tile count
    for N, K in [(64, 8192), (32, 11008), (16, 7168)]:
        W = synth.weights(N, K, seed=N + K)
        codes, scales = fp6.quantize_rows(W)
        packed = fp6.prepack(codes, scales)
        assert np.array_equal(oracle.unpack_np(packed, N, K), codes)


def test_prepack_adversarial_patterns():
    N, K = 32, 512
    for c in [np.full((N, K), 63, np.uint8), np.zeros((N, K), np.uint8),
              (np.indices((N, K)).sum(axis=0) % 2 * 63).astype(np.uint8),
              np.tile(np.array([1 << b for b in range(6)], np.uint8), (N, K // 6 + 1))[:, :K]]:
        packed = fp6.prepack(c, np.ones(N, np.float16))
        assert np.array_equal(oracle.unpack_np(packed, N, K), c)


def test_prepack_errors():
    codes = np.zeros((16, 256), np.uint8)
    ones = np.ones(16, np.float16)
    bad = codes.copy()
    bad[3, 7] = 64
    with pytest.raises(fp6.FP6Error) as e:
        fp6.prepack(bad, ones)
    assert e.value.name == "FP6_E_CODE"
    for sv in [np.nan, np.inf, 16.0, -16.0, 60000.0]:
        s = ones.copy()
        s[5] = sv
        with pytest.raises(fp6.FP6Error) as e:
            fp6.prepack(codes, s)
        assert e.value.name == "FP6_E_SCALE"
    s = ones.copy()
    s[5] = np.float16(15.99)          # largest accepted magnitude region
    fp6.prepack(codes, s)
    with pytest.raises(fp6.FP6Error) as e:
        fp6.prepack(np.zeros((16, 100), np.uint8), ones)
    assert e.value.name == "FP6_E_SHAPE"
    out = np.zeros(3072, np.uint8)
    vp = ctypes.c_void_p
    p = lambda a: a.ctypes.data_as(vp)
    assert fp6.lib.fp6_prepack(p(codes), p(ones), 16, 256, p(out), 3071) == 6      # size
    assert fp6.lib.fp6_prepack(None, p(ones), 16, 256, p(out), 3072) == 1          # null
    assert fp6.lib.fp6_prepack(p(codes), p(ones), 16, 256, None, 3072) == 1


def test_linear_and_dequant_argument_errors_before_any_hip_call():
    L = fp6.lib
    A = 1 << 20  # a fake, 16-byte aligned "device" address: never dereferenced
    # shape errors
    assert L.fp6_linear(A, A, A, A, 4, 24, 256, None) == 2
    assert L.fp6_linear(A, A, A, A, 4, 16, 200, None) == 2
    assert L.fp6_linear(A, A, A, A, -1, 16, 256, None) == 2
    assert L.fp6_linear(A, A, A, A, 2**25, 16, 256, None) == 2
    # M == 0 is a no-op (no pointer needed)
    assert L.fp6_linear(None, None, None, None, 0, 16, 256, None) == 0
    # nulls
    assert L.fp6_linear(None, A, A, A, 4, 16, 256, None) == 1
    assert L.fp6_linear(A, A, None, A, 4, 16, 256, None) == 1
    # alignment
    assert L.fp6_linear(A + 8, A, A, A, 4, 16, 256, None) == 3
    assert L.fp6_linear(A, A + 4, A, A, 4, 16, 256, None) == 3
    assert L.fp6_linear(A, A, A + 1, A, 4, 16, 256, None) == 3
    assert L.fp6_linear(A, A, A, A + 2, 4, 16, 256, None) == 3
    # plan parameters
    assert L.fp6_linear_plan(A, A, A, A, 4, 16, 256, 99, 0, None) == 8
    assert L.fp6_linear_plan(A, A, A, A, 4, 16, 256, 0, 2, None) == 8   # 2 splits > 1 k-tile
    assert L.fp6_linear_plan(A, A, A, A, 4, 16, 256, 0, -1, None) == 8
    assert L.fp6_linear_plan(A, A, A, A, 17, 16, 256, 9, 0, None) == 8     # k-split: M <= 16
    assert L.fp6_linear_plan(A, A, A, A, 4, 16, 8448, 9, 0, None) == 8     # k-split: K <= 8192
    assert L.fp6_linear_plan(A, A, A, A, 4, 16, 65 * 256, 12, 2, None) == 8  # <= 8192 of K per split
    assert L.fp6_linear_plan(A, A, A, A, 17, 16, 256, 26, 0, None) == 8    # k-ring: M <= 16
    assert L.fp6_linear_plan(A, A, A, A, 4, 16, 8448, 26, 1, None) == 8    # k-ring: <= 8192 of K per split
    assert L.fp6_linear_plan(A, A, A, A, 4, 16, 256, 27, 0, None) == 8     # unknown variant
    # dequant
    assert L.fp6_dequant(A, A, A, 16, 100, None) == 2
    assert L.fp6_dequant(None, A, A, 16, 256, None) == 1
    assert L.fp6_dequant(A, A, A + 8, 16, 256, None) == 3


# ---------------------------------------------------------------------------
# Other weight formats (fpx_* entry points).
# ---------------------------------------------------------------------------
FPX = ("e2m3", "e2m2", "e2m1")


def test_fpx_sizes_and_bits():
    assert [fp6.bits(f) for f in ("e3m2",) + FPX] == [6, 6, 5, 4]
    assert fp6.lib.fpx_bits(4) == 0 and fp6.lib.fpx_bits(-1) == 0
    for f, tb in (("e3m2", 3072), ("e2m3", 3072), ("e2m2", 2560), ("e2m1", 2048)):
        assert fp6.packed_bytes(16, 256, f) == tb == oracle.tile_bytes(f)
        assert fp6.packed_bytes(28672, 8192, f) == oracle.packed_bytes(28672, 8192, f)
        assert fp6.packed_bytes(16, 100, f) == 0
    assert fp6.lib.fpx_packed_bytes(7, 16, 256) == 0
    with pytest.raises(ValueError):
        fp6.packed_bytes(16, 256, "e5m2")


def test_fpx_format0_is_fp6():
    W = synth.weights(48, 768, seed=3)
    c0, s0 = fp6.quantize_rows(W)
    codes = np.empty((48, 768), np.uint8)
    scales = np.empty(48, np.uint16)
    p = lambda a: a.ctypes.data_as(ctypes.c_void_p)
    assert fp6.lib.fpx_quantize_rows(0, p(W), 48, 768, p(codes), p(scales)) == 0
    assert np.array_equal(codes, c0) and np.array_equal(scales, s0.view(np.uint16))
    out = np.empty(fp6.packed_bytes(48, 768), np.uint8)
    assert fp6.lib.fpx_prepack(0, p(codes), p(scales), 48, 768, p(out), out.size) == 0
    assert np.array_equal(out, fp6.prepack(c0, s0))


@pytest.mark.parametrize("fmt", FPX)
@pytest.mark.parametrize("shape", [(5, 7), (16, 256), (37, 1000)])
def test_fpx_quantizer_matches_oracle_random(fmt, shape):
    W = synth.weights(*shape, seed=11 + shape[0])
    c_lib, s_lib = fp6.quantize_rows(W, fmt)
    c_ref, s_ref = oracle.quantize_rows(W, fmt)
    assert np.array_equal(s_lib.view(np.uint16), s_ref.view(np.uint16))
    assert np.array_equal(c_lib, c_ref)


@pytest.mark.parametrize("fmt", FPX)
def test_fpx_quantizer_matches_oracle_adversarial(fmt):
    f = oracle.FORMATS[fmt]
    s = 2.0 ** -6
    mags = f.mags.tolist()
    mids = [(a + b) / 2 for a, b in zip(mags[:-1], mags[1:])]
    rng = np.random.default_rng(6)
    rows = [
        np.array([f.max * s] + [m * s for m in mids] + [-m * s for m in mids], np.float32),
        np.zeros(40, np.float32),
        (rng.standard_normal(40) * 1e-6).astype(np.float32),
        (rng.standard_normal(40) * 5).astype(np.float32),
    ]
    r = np.zeros(40, np.float32)
    r[3] = -0.0
    r[4] = np.float32(f.max * (1 + 2.0 ** -11) * 0.01)
    r[5] = -1e-9
    rows.append(r)
    width = max(len(x) for x in rows)
    W = np.zeros((len(rows), width), np.float32)
    for i, x in enumerate(rows):
        W[i, : len(x)] = x
    c_lib, s_lib = fp6.quantize_rows(W, fmt)
    c_ref, s_ref = oracle.quantize_rows(W, fmt)
    assert np.array_equal(s_lib.view(np.uint16), s_ref.view(np.uint16))
    assert np.array_equal(c_lib, c_ref)


@pytest.mark.parametrize("fmt", FPX)
@pytest.mark.parametrize("shape", [(16, 256), (32, 512)])
def test_fpx_prepack_matches_oracle_packer_bytewise(fmt, shape):
    rng = np.random.default_rng(shape[1])
    codes = rng.integers(0, 1 << fp6.bits(fmt), shape).astype(np.uint8)
    got = fp6.prepack(codes, np.ones(shape[0], np.float16), fmt)
    assert np.array_equal(got, oracle.pack_scalar(codes, fmt))


@pytest.mark.parametrize("fmt", FPX)
def test_fpx_prepack_round_trip_llama_shape(fmt):
    for N, K in [(64, 8192), (32, 11008)]:
        W = synth.weights(N, K, seed=N + K + 1)
        codes, scales = fp6.quantize_rows(W, fmt)
        packed = fp6.prepack(codes, scales, fmt)
        assert np.array_equal(oracle.unpack_tiles(packed, N, K, fmt), codes)


@pytest.mark.parametrize("fmt", FPX)
def test_fpx_errors(fmt):
    b = fp6.bits(fmt)
    codes = np.zeros((16, 256), np.uint8)
    ones = np.ones(16, np.float16)
    bad = codes.copy()
    bad[2, 9] = 1 << b
    with pytest.raises(fp6.FP6Error) as e:
        fp6.prepack(bad, ones, fmt)
    assert e.value.name == "FP6_E_CODE"
    bad[2, 9] = (1 << b) - 1
    fp6.prepack(bad, ones, fmt)
    limit = oracle.FORMATS[fmt].scale_limit
    for sv in [np.nan, np.inf] + ([limit, -limit] if np.isfinite(limit) else []):
        s = ones.copy()
        s[5] = sv
        with pytest.raises(fp6.FP6Error) as e:
            fp6.prepack(codes, s, fmt)
        assert e.value.name == "FP6_E_SCALE"
    if not np.isfinite(limit):
        s = ones.copy()
        s[5] = 60000.0
        fp6.prepack(codes, s, fmt)   # FP4 accepts any finite scale
    with pytest.raises(fp6.FP6Error) as e:
        fp6.quantize_rows(np.full((1, 4), 1e6 if np.isfinite(limit) else 1e30, np.float32), fmt)
    assert e.value.name == "FP6_E_SCALE"
    L = fp6.lib
    p = lambda a: a.ctypes.data_as(ctypes.c_void_p)
    out = np.zeros(fp6.packed_bytes(16, 256, fmt), np.uint8)
    f = fp6.FORMATS[fmt]
    assert L.fpx_prepack(f, p(codes), p(ones), 16, 256, p(out), out.size + 1) == 6
    assert L.fpx_prepack(9, p(codes), p(ones), 16, 256, p(out), out.size) == 8
    assert L.fpx_quantize_rows(9, p(np.zeros((1, 4), np.float32)), 1, 4, p(codes), p(ones)) == 8
    A = 1 << 20
    assert L.fpx_linear(9, A, A, A, A, 4, 16, 256, None) == 8
    assert L.fpx_linear(f, A, A, A, A, 4, 16, 200, None) == 2
    assert L.fpx_linear(f, None, None, None, None, 0, 16, 256, None) == 0
    assert L.fpx_linear(f, A + 8, A, A, A, 4, 16, 256, None) == 3
    assert L.fpx_linear_plan(f, A, A, A, A, 4, 16, 256, 99, 0, None) == 8
    assert L.fpx_dequant(9, A, A, A, 16, 256, None) == 8
    assert L.fpx_dequant(f, A, A, A, 16, 100, None) == 2


# ---------------------------------------------------------------------------
# 2:4-sparse FP6 (fp6s_* entry points).
# ---------------------------------------------------------------------------
from oracle import sparse24  # noqa: E402


@pytest.mark.parametrize("shape", [(3, 8), (16, 512), (37, 1024)])
def test_sparse_prune_quantize_matches_oracle(shape):
    W = synth.weights(*shape, seed=21 + shape[0])
    c, p, s = fp6.prune_quantize(W)
    oc, op, osc = sparse24.quantize_sparse(W)
    assert np.array_equal(s.view(np.uint16), osc.view(np.uint16))
    assert np.array_equal(p, op) and np.array_equal(c, oc)


def test_sparse_prune_quantize_ties_and_zeros():
    rng = np.random.default_rng(8)
    W = (rng.integers(-2, 3, (16, 256)) * 0.25).astype(np.float32)   # many equal magnitudes and zeros
    W[3] = 0.0
    W[4, :4] = [-0.0, 0.0, -0.0, 0.0]
    c, p, s = fp6.prune_quantize(W)
    oc, op, osc = sparse24.quantize_sparse(W)
    assert np.array_equal(s.view(np.uint16), osc.view(np.uint16))
    assert np.array_equal(p, op) and np.array_equal(c, oc)


@pytest.mark.parametrize("shape", [(16, 512), (32, 1024)])
def test_sparse_prepack_matches_oracle_packer_bytewise(shape):
    N, K = shape
    W = synth.weights(N, K, seed=K + 3)
    c, p, s = fp6.prune_quantize(W)
    got = fp6.sparse_prepack(c, p, s, K)
    assert got.size == N * K // 2
    assert np.array_equal(got, sparse24.pack_scalar(c, p, K))


def test_sparse_prepack_round_trip_large():
    for N, K in [(64, 8192), (32, 7168)]:
        W = synth.weights(N, K, seed=N + K + 2)
        c, p, s = fp6.prune_quantize(W)
        cc, pp = sparse24.unpack_tiles(fp6.sparse_prepack(c, p, s, K), N, K)
        assert np.array_equal(cc, c) and np.array_equal(pp, p)


def test_sparse_errors():
    assert fp6.sparse_packed_bytes(16, 512) == 4096
    assert fp6.sparse_packed_bytes(16, 768) == 0 and fp6.sparse_packed_bytes(8, 512) == 0
    N, K = 16, 512
    c = np.zeros((N, K // 2), np.uint8)
    p = np.tile(np.array([0, 1], np.uint8), (N, K // 4))
    s = np.ones(N, np.float16)
    fp6.sparse_prepack(c, p, s, K)
    for bad_p in ([1, 1], [2, 1], [0, 4]):
        q = p.copy()
        q[5, 10:12] = bad_p
        with pytest.raises(fp6.FP6Error) as e:
            fp6.sparse_prepack(c, q, s, K)
        assert e.value.name == "FP6_E_VALUE"
    cb = c.copy()
    cb[0, 0] = 64
    with pytest.raises(fp6.FP6Error) as e:
        fp6.sparse_prepack(cb, p, s, K)
    assert e.value.name == "FP6_E_CODE"
    sb = s.copy()
    sb[2] = 16.0
    with pytest.raises(fp6.FP6Error) as e:
        fp6.sparse_prepack(c, p, sb, K)
    assert e.value.name == "FP6_E_SCALE"
    with pytest.raises(fp6.FP6Error) as e:
        fp6.prune_quantize(np.zeros((2, 6), np.float32))
    assert e.value.name == "FP6_E_SHAPE"
    with pytest.raises(fp6.FP6Error) as e:
        fp6.prune_quantize(np.array([[1.0, np.nan, 0.0, 0.0]], np.float32))
    assert e.value.name == "FP6_E_VALUE"
    L = fp6.lib
    A = 1 << 20
    assert L.fp6s_linear(A, A, A, A, 4, 16, 768, None) == 2          # K % 512
    assert L.fp6s_linear(None, None, None, None, 0, 16, 512, None) == 0
    assert L.fp6s_linear(A + 8, A, A, A, 4, 16, 512, None) == 3
    assert L.fp6s_linear_plan(A, A, A, A, 4, 16, 512, 10, 0, None) == 8
    assert L.fp6s_linear_plan(A, A, A, A, 17, 16, 512, 6, 0, None) == 8     # k-split: M <= 16
    assert L.fp6s_linear_plan(A, A, A, A, 4, 16, 9 * 512, 6, 1, None) == 8  # <= 8 tiles per split
    assert L.fp6s_linear_plan(A, A, A, A, 17, 16, 512, 1, 0, None) == 8    # k-slice: M <= 16
    assert L.fp6s_linear_plan(A, A, A, A, 4, 16, 512 * 17, 1, 0, None) == 8  # k-slice: K <= 8192
    assert L.fp6s_linear_plan(A, A, A, A, 4, 16, 512, 2, 2, None) == 8    # 2 splits > 1 tile
    assert L.fp6s_linear_plan(A, A, A, A, 17, 16, 512, 9, 0, None) == 8    # k-ring: M <= 16
    assert L.fp6s_linear_plan(A, A, A, A, 4, 16, 512 * 17, 9, 0, None) == 8  # k-ring: K <= 8192
    assert L.fp6s_linear_plan(A, A, A, A, 4, 16, 1024, 9, 2, None) == 8   # k-ring: no K-splits
    assert L.fp6s_dequant(A, A, A, 16, 768, None) == 2
    assert L.fp6s_dequant(None, A, A, 16, 512, None) == 1


def _binding_cases():
    """(call, expected message fragment) for every device-tensor check of the
    Python binding; each call has exactly one bad argument and fails before
    any library call (CPU tensors are rejected last, for being off the GPU)."""
    import torch
    N, K, M = 32, 512, 4
    f16, u8 = torch.float16, torch.uint8
    nb, snb = fp6.packed_bytes(N, K), fp6.sparse_packed_bytes(N, K)
    X = torch.zeros((M, K), dtype=f16)
    P, PS = torch.zeros(nb, dtype=u8), torch.zeros(snb, dtype=u8)
    S = torch.zeros(N, dtype=f16)
    Y = torch.zeros((M, N), dtype=f16)
    W16 = torch.zeros((N, K), dtype=f16)
    cases = [
        # dequant: packed size / dtype, scales dtype / count, out shape / dtype / layout
        (lambda: fp6.dequant(torch.zeros(nb - 1, dtype=u8), S, N, K), "packed"),
        (lambda: fp6.dequant(torch.zeros(nb, dtype=torch.int8), S, N, K), "packed"),
        (lambda: fp6.dequant(torch.zeros(fp6.packed_bytes(N, K, "e2m1") + 16, dtype=u8), S, N, K, fmt="e2m1"), "packed"),
        (lambda: fp6.dequant(P, torch.zeros(N, dtype=torch.float32), N, K), "scales"),
        (lambda: fp6.dequant(P, torch.zeros(N - 1, dtype=f16), N, K), "scales"),
        (lambda: fp6.dequant(P, S, N, K, out=torch.zeros((N, K - 1), dtype=f16)), "out"),
        (lambda: fp6.dequant(P, S, N, K, out=torch.zeros((N, K), dtype=torch.float32)), "out"),
        (lambda: fp6.dequant(P, S, N, K, out=torch.zeros((K, N), dtype=f16).t()), "out"),
        (lambda: fp6.dequant(P, S, N, K, out=W16), "GPU"),
        (lambda: fp6.dequant(P, S, N, K), "GPU"),
        # sparse_dequant
        (lambda: fp6.sparse_dequant(torch.zeros(snb + 1, dtype=u8), S, N, K), "packed"),
        (lambda: fp6.sparse_dequant(P, S, N, K), "packed"),           # dense-sized buffer
        (lambda: fp6.sparse_dequant(PS, torch.zeros(N, dtype=torch.bfloat16), N, K), "scales"),
        (lambda: fp6.sparse_dequant(PS, torch.zeros(2 * N, dtype=f16), N, K), "scales"),
        (lambda: fp6.sparse_dequant(PS, S, N, K, out=torch.zeros((N, K // 2), dtype=f16)), "out"),
        (lambda: fp6.sparse_dequant(PS, S, N, K, out=torch.zeros((N, K), dtype=u8)), "out"),
        (lambda: fp6.sparse_dequant(PS, S, N, K, out=W16), "GPU"),
        # linear / sparse_linear
        (lambda: fp6.linear(torch.zeros((M, K), dtype=torch.float32), P, S, N, K), "X"),
        (lambda: fp6.linear(torch.zeros((M, K + 1), dtype=f16), P, S, N, K), "X"),
        (lambda: fp6.linear(torch.zeros((K, M), dtype=f16).t(), P, S, N, K), "X"),
        (lambda: fp6.linear(X, P[:-1], S, N, K), "packed"),
        (lambda: fp6.linear(X, P, S[:-1], N, K), "scales"),
        (lambda: fp6.linear(X, P, S, N, K, out=torch.zeros((M, N + 1), dtype=f16)), "out"),
        (lambda: fp6.linear(X, P, S, N, K, out=Y), "GPU"),
        (lambda: fp6.sparse_linear(X, P, S, N, K), "packed"),
        (lambda: fp6.sparse_linear(X, PS, S.float(), N, K), "scales"),
        (lambda: fp6.sparse_linear(X, PS, S, N, K, out=Y), "GPU"),
    ]
    return cases


def test_binding_rejects_bad_device_tensors():
    cases = _binding_cases()
    for i, (call, frag) in enumerate(cases):
        with pytest.raises(ValueError, match=frag):
            call()
