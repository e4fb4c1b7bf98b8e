"""GPU parity of the other weight formats (FP6 e2m3, FP5 e2m2, FP4 e2m1)
against the CPU oracle, through the fpx_* entry points (needs an MI355X).

Same bars as the FP6 e3m2 tests: de-quantisation bit-exact, fused linear
within |Y - Y_ref| <= 2e-3 (|Y_ref| + rms) per element and relative Frobenius
<= 5e-4, one-hot activations reproducing Wdq exactly, for every kernel
configuration on small ragged shapes and for the automatic plan on every
output element of every workload layer at full size.
"""

import numpy as np
import pytest

import oracle
from weight_only_fp6_amd import synth

from _workloads import Prepared, dense_weight_set, prepare_shape, workload, y_ref

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():  # pragma: no cover - CPU container
    pytest.skip("no GPU", allow_module_level=True)

import weight_only_fp6_amd as fp6  # noqa: E402

DEV = torch.device("cuda:0")
FMTS = ("e2m3", "e2m2", "e2m1")
ALL_VARIANTS = (0, 1, 2, 3, 4, 5, 6, 7, 8, 10, 11, 14, 15, 16, 17, 18, 19, 20, 21, 22, 23, 24, 25)
SMALL_M_VARIANTS = (9, 12, 13, 26)


def _bits16(t):
    return t.detach().cpu().numpy().view(np.uint16)


def _assert_tol(y_dev, y_ref, what=""):
    rep = oracle.tolerance_report(y_dev.detach().cpu().numpy().astype(np.float64), y_ref)
    assert rep["ok"], (what, rep)


def _dequant_dev(codes, scales, fmt):
    N, K = codes.shape
    packed = torch.from_numpy(fp6.prepack(codes, scales, fmt)).to(DEV)
    s = torch.from_numpy(np.ascontiguousarray(scales, np.float16)).to(DEV)
    out = fp6.dequant(packed, s, N, K, fmt=fmt)
    torch.cuda.synchronize()
    return _bits16(out)


@pytest.mark.parametrize("fmt", FMTS)
def test_dequant_all_codes_unit_scale(fmt):
    N, K = 64, 512
    ncode = 1 << fp6.bits(fmt)
    codes = ((np.arange(N)[:, None] * 7 + np.arange(K)[None, :]) % ncode).astype(np.uint8)
    scales = np.ones(N, np.float16)
    assert np.array_equal(_dequant_dev(codes, scales, fmt), oracle.dequant_ref(codes, scales, fmt).view(np.uint16))


@pytest.mark.parametrize("fmt", FMTS)
def test_dequant_power_of_two_subnormal_and_random_scales(fmt):
    rng = np.random.default_rng(7)
    js = list(range(-24, 2))
    ncode = 1 << fp6.bits(fmt)
    N, K = 16 * len(js) + 512, 256
    codes = rng.integers(0, ncode, (N, K)).astype(np.uint8)
    lim = 0x4400 if fmt != "e2m1" else 0x7BFF          # |s| < 4, or any finite fp16
    sb = rng.integers(1, lim, 512).astype(np.uint16) | (rng.integers(0, 2, 512).astype(np.uint16) << 15)
    scales = np.concatenate([np.repeat(np.array([2.0 ** j for j in js], np.float16), 16), sb.view(np.float16)])
    ref = oracle.dequant_ref(codes, scales, fmt).view(np.uint16)
    assert np.array_equal(_dequant_dev(codes, scales, fmt), ref)
    assert (ref[:16 * 10] & 0x7C00 == 0).any()     # fp16 subnormal weights survive


def _first_of_weight_set(name):
    shp = synth.SHAPES[name]
    return next(n for n, q in synth.SHAPES.items() if (q.N, q.K, q.seed_w) == (shp.N, shp.K, shp.seed_w)) == name


@pytest.mark.parametrize("fmt, name", [(f, n) for f in FMTS for n in synth.SHAPES])
def test_linear_workloads(fmt, name):
    # Every workload layer at full size: every output element of the
    # automatic plan, and (once per weight set) the whole de-quantised weight
    # matrix bit for bit, with the library quantiser equal to the oracle's.
    shp = synth.SHAPES[name]
    ws, X, yref = workload(name, fmt)
    packed, s = ws.to_device()
    Y = fp6.linear(torch.from_numpy(X).to(DEV), packed, s, shp.N, shp.K, fmt=fmt)
    torch.cuda.synchronize()
    _assert_tol(Y, yref, what=(fmt, name))
    if _first_of_weight_set(name):
        assert ws.codes_match and ws.scales_match, (fmt, name)
        W16 = fp6.dequant(packed, s, shp.N, shp.K, fmt=fmt)
        torch.cuda.synchronize()
        assert np.array_equal(_bits16(W16), ws.wdq_ref.view(np.uint16)), (fmt, name)


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("M", [1, 3, 16, 17, 64, 100])
@pytest.mark.parametrize("NK", [(16, 256), (80, 2816)])
def test_linear_small_shapes_every_variant(fmt, M, NK):
    N, K = NK
    p = Prepared(M, N, K, seed_w=N * 5 + K, seed_x=M * 13 + 2, fmt=fmt)
    X, packed, s = p.to_device()
    for variant in ALL_VARIANTS + (SMALL_M_VARIANTS if M <= 16 else ()):
        Y = fp6.linear_plan(X, packed, s, N, K, variant=variant, fmt=fmt)
        torch.cuda.synchronize()
        _assert_tol(Y, p.y_ref, what=(fmt, M, N, K, variant))


@pytest.mark.parametrize("fmt", FMTS)
def test_linear_forced_splits(fmt):
    name = "llama7b_mlp_down_16x4096x11008"
    shp = synth.SHAPES[name]
    ws, X, yref = workload(name, fmt)
    packed, s = ws.to_device()
    Xd = torch.from_numpy(X).to(DEV)
    for variant, splits in [(1, 7), (3, 43), (5, 3), (10, 4), (11, 2), (14, 8), (15, 5), (16, 2), (17, 3), (18, 1), (18, 4), (23, 5), (24, 3)]:
        Y = fp6.linear_plan(Xd, packed, s, shp.N, shp.K, variant=variant, splits=splits, fmt=fmt)
        torch.cuda.synchronize()
        _assert_tol(Y, yref, what=(fmt, variant, splits))


@pytest.mark.parametrize("fmt, K", [(f, K) for f in FMTS for K in (512, 1280, 4096, 8192, 8448, 11008, 12288)])
def test_linear_k_coverage(fmt, K):
    # k-split (up to K = 8192) and k-slice (up to 12288: 1..3 tiles per wave)
    # kernels and the automatic plan at M = 1, 2, 4 and 16; every output.
    N = 16 * 300
    ws = dense_weight_set(N, K, K + 9, fmt)
    packed, s = ws.to_device()
    variants = (0,) + (SMALL_M_VARIANTS if K <= 8192 else (13,))
    for M in (1, 2, 4, 16):
        X = synth.activations(M, K, K + 10 + M)
        yref = y_ref(X, ws.wdq_ref)
        Xd = torch.from_numpy(X).to(DEV)
        for variant in variants:
            Y = fp6.linear_plan(Xd, packed, s, N, K, variant=variant, fmt=fmt)
            torch.cuda.synchronize()
            _assert_tol(Y, yref, what=(fmt, M, K, variant))


@pytest.mark.parametrize("fmt", FMTS)
def test_linear_auto_kring_narrow_layers(fmt):
    # Automatic plans on narrow layers (at most 3/4 of the CUs with a row
    # block) with 4096 < K <= 8192 at M = 5..16: the k-ring kernel with 2
    # K-splits, one row block per workgroup (2048 rows) and two (3072 rows,
    # 32 k-tiles).  Every output element, and the plan.
    if torch.cuda.get_device_properties(0).multi_processor_count != 256:
        pytest.skip("plan thresholds are stated for 256 CUs")
    for M, N, K in ((16, 2048, 6144), (8, 3072, 8192)):
        assert fp6.plan_query(M, N, K) == (26, 2)
        ws = dense_weight_set(N, K, N + K + 3, fmt)
        packed, s = ws.to_device()
        X = synth.activations(M, K, M + 41)
        yref = y_ref(X, ws.wdq_ref)
        Y = fp6.linear(torch.from_numpy(X).to(DEV), packed, s, N, K, fmt=fmt)
        torch.cuda.synchronize()
        _assert_tol(Y, yref, what=(fmt, M, N, K))


@pytest.mark.parametrize("fmt", FMTS)
def test_linear_one_hot_reproduces_wdq_exactly(fmt):
    N, K = 64, 1024
    p = Prepared(16, N, K, seed_w=97, seed_x=3, fmt=fmt)
    ks = np.array([0, 1, 7, 8, 255, 256, 300, 511, 512, 777, 1000, 1023, 31, 32, 33, 600])
    X = np.zeros((16, K), np.float16)
    X[np.arange(16), ks] = 1.0
    Xd = torch.from_numpy(X).to(DEV)
    _, packed, s = p.to_device()
    want = p.wdq_ref[:, ks].T.astype(np.float64)
    for variant, splits in [(0, 0), (1, 1), (1, 4), (2, 3), (5, 3), (6, 1), (8, 1), (9, 0), (12, 0),
                            (13, 0), (14, 1), (15, 2), (16, 1), (10, 1), (10, 3), (11, 2), (17, 1), (17, 3), (18, 1), (18, 3),
                            (19, 2), (20, 1), (21, 3), (22, 2), (23, 1), (23, 3), (24, 2), (25, 0), (26, 0)]:
        Y = fp6.linear_plan(Xd, packed, s, N, K, variant=variant, splits=splits, fmt=fmt)
        torch.cuda.synchronize()
        assert np.array_equal(Y.cpu().numpy().astype(np.float64), want), (fmt, variant, splits)


@pytest.mark.parametrize("fmt", FMTS)
def test_kring_one_hot_every_tile_slot(fmt):
    # One-hot activations through the k-ring kernel at K = 8192 (4 k-tiles
    # per wave) with 3 row blocks per workgroup and a short last one: every
    # output must equal a de-quantised weight exactly, for every tile slot.
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    N, K, M = 16 * (2 * cus + 9), 8192, 16
    ws = dense_weight_set(N, K, 4343, fmt)
    cols = []
    for m in range(M):
        w = (5 * m + 2) % 8
        cols.append((4 * w + m % 4) * 256 + (29 * m + 3) % 256)
    ks = np.array(cols)
    X = np.zeros((M, K), np.float16)
    X[np.arange(M), ks] = 1.0
    Xd = torch.from_numpy(X).to(DEV)
    packed, s = ws.to_device()
    want = ws.wdq_ref[:, ks].T.astype(np.float64)
    for m_used in (1, 16):
        Y = fp6.linear_plan(Xd[:m_used].contiguous(), packed, s, N, K, variant=26, fmt=fmt)
        torch.cuda.synchronize()
        assert np.array_equal(Y.cpu().numpy().astype(np.float64), want[:m_used]), (fmt, m_used)


def test_fpx_format0_matches_fp6_bitwise():
    shp = synth.SHAPES["llama7b_attn_1x4096x4096"]
    p = prepare_shape(shp)
    X, packed, s = p.to_device()
    a = fp6.linear(X, packed, s, shp.N, shp.K)
    b = torch.empty_like(a)
    st = fp6.lib.fpx_linear(0, X.data_ptr(), packed.data_ptr(), s.data_ptr(), b.data_ptr(),
                            shp.M, shp.N, shp.K, torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    assert st == 0
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))


def _adversarial_weights(N, K, seed, fmt):
    """As the e3m2 corner rows, per format: a zero row, a lone outlier over
    values that quantise to zero, negative values below half the smallest
    subnormal (codes -0) with one outlier, saturating +-max, exact ties
    between neighbouring magnitudes (power-of-two scale), a scale near the
    format's limit, then ordinary N(0, 0.02) rows."""
    f = oracle.FORMATS[fmt]
    rng = np.random.default_rng(seed)
    W = (rng.standard_normal((N, K)) * 0.02).astype(np.float32)
    W[0] = 0.0
    W[1] = 1e-6
    W[1, 5] = 1.0
    W[2] = -1e-9
    W[2, 7] = 0.5
    W[3] = np.where(np.arange(K) % 2 == 0, 1.0, -1.0)
    mags = np.array(f.mags, dtype=np.float64)
    mids = (mags[:-1] + mags[1:]) / 2
    row = np.resize(np.concatenate([mids, -mids]), K) * 2.0 ** -4
    row[0] = f.max * 2.0 ** -4                              # scale exactly 2^-4
    W[4] = row.astype(np.float32)
    limit = min(f.scale_limit, 16.0)
    W[5] = (rng.standard_normal(K) * 0.1).astype(np.float32)
    W[5, 3] = 0.9 * limit * f.max                           # scale 0.9 of the limit
    return W


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("M", [3, 17])
def test_linear_adversarial_rows(fmt, M):
    N, K = 96, 2816
    W = _adversarial_weights(N, K, 223 + M, fmt)
    X = synth.activations(M, K, 421 + M)
    X[:, ::5] = 0
    p = Prepared(M, N, K, seed_w=0, seed_x=0, W=W, X=X, fmt=fmt)
    assert np.array_equal(p.codes, p.ocodes)
    assert np.array_equal(p.scales.view(np.uint16), p.oscales.view(np.uint16))
    Xd, packed, s = p.to_device()
    assert np.array_equal(_bits16(fp6.dequant(packed, s, N, K, fmt=fmt)), p.wdq_ref.view(np.uint16))
    for variant, splits in [(0, 0), (1, 3), (15, 2), (18, 1), (10, 1), (17, 3), (19, 3), (22, 2), (23, 2), (24, 1), (25, 0)]:
        Y = fp6.linear_plan(Xd, packed, s, N, K, variant=variant, splits=splits, fmt=fmt)
        torch.cuda.synchronize()
        _assert_tol(Y, p.y_ref, what=(fmt, M, variant, splits))
        assert not Y[:, 0].cpu().numpy().astype(np.float64).any(), (fmt, M, variant, splits)
