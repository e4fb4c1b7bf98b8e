"""GPU parity of the HIP path against the CPU oracle (needs an MI355X).

* De-quantisation export: bit-exact against oracle.dequant_ref.
* Fused linear: |Y - Y_ref| <= 2e-3 (|Y_ref| + rms(Y_ref)) per element and
  relative Frobenius error <= 5e-4, on every workload shape at full size
  (sampled output columns for the two largest layers) and on small shapes that
  span several tiles with ragged M; one-hot inputs must reproduce Wdq exactly.
"""

import functools

import numpy as np
import pytest

import oracle
from weight_only_fp6_amd import synth

from _workloads import Prepared, prepare_shape  # noqa: F401

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():  # pragma: no cover - CPU container
    pytest.skip("no GPU", allow_module_level=True)

import weight_only_fp6_amd as fp6  # noqa: E402

DEV = torch.device("cuda:0")
# Kernel configurations of fp6_linear_plan: 0 = automatic, 1-4 and 7-8
# streaming, 5-6 and 10-11 tiled, 9 k-split persistent (M <= 16, K <= 8192).
ALL_VARIANTS = (0, 1, 2, 3, 4, 5, 6, 7, 8, 10, 11, 14, 15, 16, 17, 18, 19, 20, 21, 22)
KSPLIT = 9
KSPLIT16 = 12
KSLICE = 13


def _bits16(t):
    return t.detach().cpu().numpy().view(np.uint16)


def _assert_tol(y_dev, y_ref, rms=None, what=""):
    y = y_dev.detach().cpu().numpy().astype(np.float64)
    rep = oracle.tolerance_report(y, y_ref, rms=rms)
    assert rep["ok"], (what, rep)
    return rep


# ----------------------------------------------------------------------------
# De-quantisation (bit-exact)
# ----------------------------------------------------------------------------
def _dequant_dev(codes, scales):
    N, K = codes.shape
    packed = torch.from_numpy(fp6.prepack(codes, scales)).to(DEV)
    s = torch.from_numpy(np.ascontiguousarray(scales, np.float16)).to(DEV)
    out = fp6.dequant(packed, s, N, K)
    torch.cuda.synchronize()
    return _bits16(out)


def test_dequant_all_codes_unit_scale():
    N, K = 64, 512
    codes = ((np.arange(N)[:, None] * 7 + np.arange(K)[None, :]) % 64).astype(np.uint8)
    scales = np.ones(N, np.float16)
    got = _dequant_dev(codes, scales)
    ref = oracle.dequant_ref(codes, scales).view(np.uint16)
    assert np.array_equal(got, ref)


def test_dequant_power_of_two_and_subnormal_scales():
    js = list(range(-24, 4))
    N, K = 16 * len(js), 256
    codes = synth.codes_uniform(N, K, seed=3)
    scales = np.repeat(np.array([2.0 ** j for j in js], np.float16), 16)
    got = _dequant_dev(codes, scales)
    ref = oracle.dequant_ref(codes, scales).view(np.uint16)
    assert np.array_equal(got, ref)
    # the tiny scales produce fp16 subnormal weights: they must survive
    assert (ref[:16 * 10] & 0x7C00 == 0).any()


def test_dequant_random_scales_full_range():
    rng = np.random.default_rng(4)
    N, K = 1024, 512
    sb = rng.integers(1, 0x4C00, N).astype(np.uint16) | (rng.integers(0, 2, N).astype(np.uint16) << 15)
    scales = sb.view(np.float16)
    codes = synth.codes_uniform(N, K, seed=4)
    got = _dequant_dev(codes, scales)
    ref = oracle.dequant_ref(codes, scales).view(np.uint16)
    assert np.array_equal(got, ref)


@functools.lru_cache(maxsize=2)
def _prep(name, sample):
    return prepare_shape(synth.SHAPES[name], sample=sample)


_NK = {}
for _n, _s in synth.SHAPES.items():
    _NK.setdefault((_s.N, _s.K, _s.cfg), _n)


@pytest.mark.parametrize("name", sorted(_NK.values()))
def test_dequant_workload_weights(name):
    shp = synth.SHAPES[name]
    sample = None if shp.N * shp.K <= 16 * 2**20 else 256
    p = _prep(name, sample)
    packed = torch.from_numpy(p.packed).to(DEV)
    s = torch.from_numpy(p.scales.copy()).to(DEV)
    out = fp6.dequant(packed, s, shp.N, shp.K)
    got = _bits16(out[torch.from_numpy(p.rows).to(DEV)])
    assert np.array_equal(got, p.wdq_ref.view(np.uint16))


# ----------------------------------------------------------------------------
# Fused linear at the workload shapes (automatic plan = the benchmarked launch)
# ----------------------------------------------------------------------------
@pytest.mark.parametrize("name", list(synth.SHAPES))
def test_linear_workloads(name):
    shp = synth.SHAPES[name]
    sample = None if shp.N * shp.K <= 48 * 2**20 else 384
    p = _prep(name, sample)
    X, packed, s = p.to_device()
    Y = fp6.linear(X, packed, s, shp.N, shp.K)
    torch.cuda.synchronize()
    ycols = Y[:, torch.from_numpy(p.rows).to(DEV)]
    _assert_tol(ycols, p.y_ref, what=name)


# ----------------------------------------------------------------------------
# Small shapes spanning several tiles, ragged M, forced schedules
# ----------------------------------------------------------------------------
@pytest.mark.parametrize("M", [1, 2, 3, 5, 8, 15, 16, 17, 31, 33, 64, 100, 257])
@pytest.mark.parametrize("NK", [(16, 256), (64, 1024), (80, 2816)])
def test_linear_small_shapes_ragged_m(M, NK):
    N, K = NK
    p = Prepared(M, N, K, seed_w=N * 7 + K, seed_x=M * 11 + 1)
    X, packed, s = p.to_device()
    for variant in ALL_VARIANTS + ((KSPLIT, KSPLIT16, KSLICE) if M <= 16 else ()):
        Y = fp6.linear_plan(X, packed, s, N, K, variant=variant)
        torch.cuda.synchronize()
        _assert_tol(Y, p.y_ref, what=(M, N, K, variant))


@pytest.mark.parametrize("splits", [1, 2, 3, 4, 7, 8, 16, 43])
def test_linear_forced_splits_long_k(splits):
    # Llama-7B MLP down projection: K = 11008 = 43 tiles of 256 (43 is prime)
    shp = synth.SHAPES["llama7b_mlp_down_16x4096x11008"]
    p = _prep(shp.name, None)
    X, packed, s = p.to_device()
    for variant in (1, 3, 5, 6, 10, 11, 14, 16, 17, 18, 19, 20, 21, 22):
        Y = fp6.linear_plan(X, packed, s, shp.N, shp.K, variant=variant, splits=splits)
        torch.cuda.synchronize()
        _assert_tol(Y, p.y_ref, what=(splits, variant))


@pytest.mark.parametrize("K", [256, 512, 1280, 2048, 4096, 6144, 8192])
@pytest.mark.parametrize("M", [1, 4, 16])
def test_linear_ksplit_k_coverage(M, K):
    # the k-split and k-slice kernels at every per-wave tile count (1..4,
    # ragged ranges), with more row blocks than workgroups (N = 16*300 > 256)
    N = 16 * 300
    p = Prepared(M, N, K, seed_w=K + M, seed_x=K * 3 + M, sample=64)
    X, packed, s = p.to_device()
    for variant in (KSPLIT, KSPLIT16, KSLICE):
        Y = fp6.linear_plan(X, packed, s, N, K, variant=variant)
        torch.cuda.synchronize()
        _assert_tol(Y[:, torch.from_numpy(p.rows).to(DEV)], p.y_ref, what=(M, K, variant))


@pytest.mark.parametrize("K", [2048, 4096])
@pytest.mark.parametrize("per_wg", [2, 3, 4, 5, 7, 9])
@pytest.mark.parametrize("M", [1, 5, 16])
def test_linear_ksplit_row_blocks_per_workgroup(M, per_wg, K):
    # The k-split kernels run straight-line code for 2-8 row blocks per
    # workgroup (4 register stages; a workgroup with fewer than the form's
    # count repeats its last row block) and loop beyond.  N is sized from the CU count so that the first
    # workgroups get per_wg row blocks and the rest per_wg - 1; one row of
    # every row block is checked.  At K = 2048 half of the 16 waves have an
    # empty k-range.
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    nblocks = (per_wg - 1) * cus + max(cus // 3, 1)
    N = 16 * nblocks
    W = synth.weights(N, K, 900 + per_wg + K)
    X = synth.activations(M, K, 910 + M)
    codes, scales = fp6.quantize_rows(W)
    packed = fp6.prepack(codes, scales)
    rows = 16 * np.arange(nblocks) + (np.arange(nblocks) * 7) % 16
    oc, osc = oracle.quantize_rows(W[rows])
    y_ref = oracle.gemm_ref(X, oracle.dequant_ref(oc, osc))
    Xd = torch.from_numpy(X).to(DEV)
    Pd = torch.from_numpy(packed).to(DEV)
    Sd = torch.from_numpy(scales.copy()).to(DEV)
    cols = torch.from_numpy(rows).to(DEV)
    for variant in (KSPLIT, KSPLIT16):
        Y = fp6.linear_plan(Xd, Pd, Sd, N, K, variant=variant)
        torch.cuda.synchronize()
        _assert_tol(Y[:, cols], y_ref, what=(M, per_wg, K, variant))


@pytest.mark.parametrize("M", [1, 5, 16])
@pytest.mark.parametrize("NK", [(4096, 11008), (1024, 6400), (2048, 2304)])
def test_linear_ksplit_across_workgroups(M, NK):
    # The k-split kernels with K split across workgroups (fixed-order
    # fix-up): straight-line and looping forms, ragged split ranges, idle
    # waves; bitwise reproducible from run to run.
    N, K = NK
    p = Prepared(M, N, K, seed_w=N + K + 5, seed_x=M + 3, sample=192)
    X, packed, s = p.to_device()
    cols = torch.from_numpy(p.rows).to(DEV)
    ktiles = K // 256
    for variant, wk in ((KSPLIT, 8), (KSPLIT16, 16)):
        for splits in (2, 3, 4, 7):
            if splits > ktiles or -(-ktiles // splits) > 32:
                continue
            Y = fp6.linear_plan(X, packed, s, N, K, variant=variant, splits=splits).clone()
            Y2 = fp6.linear_plan(X, packed, s, N, K, variant=variant, splits=splits)
            torch.cuda.synchronize()
            _assert_tol(Y[:, cols], p.y_ref, what=(M, N, K, variant, splits))
            assert torch.equal(Y.view(torch.int16), Y2.view(torch.int16)), (M, N, K, variant, splits)


def test_linear_one_hot_reproduces_wdq_exactly():
    N, K = 64, 1024
    p = Prepared(16, N, K, seed_w=99, seed_x=1)
    ks = np.array([0, 1, 7, 8, 255, 256, 300, 511, 512, 777, 1000, 1023, 31, 32, 33, 600])
    X = np.zeros((16, K), np.float16)
    X[np.arange(16), ks] = 1.0
    Xd = torch.from_numpy(X).to(DEV)
    _, packed, s = p.to_device()
    for variant, splits in [(0, 0), (1, 1), (1, 4), (2, 1), (2, 3), (3, 2), (4, 1), (5, 1), (5, 3), (6, 1), (6, 2), (7, 2), (8, 1), (KSPLIT, 0), (KSPLIT16, 0), (KSLICE, 0), (14, 1), (15, 2), (16, 1), (10, 1), (10, 3), (11, 2), (17, 1), (17, 3), (18, 1), (18, 3), (19, 2), (20, 3), (21, 1), (22, 4)]:
        Y = fp6.linear_plan(Xd, packed, s, N, K, variant=variant, splits=splits)
        torch.cuda.synchronize()
        got = Y.cpu().numpy().astype(np.float64)
        want = p.wdq_ref[:, ks].T.astype(np.float64)
        assert np.array_equal(got, want), (variant, splits)


def test_linear_zero_activations_give_zero():
    N, K = 64, 1024
    p = Prepared(5, N, K, seed_w=98, seed_x=2)
    _, packed, s = p.to_device()
    X = torch.zeros((5, K), dtype=torch.float16, device=DEV)
    for splits in (1, 4):
        Y = fp6.linear_plan(X, packed, s, N, K, variant=1, splits=splits)
        torch.cuda.synchronize()
        assert not Y.cpu().numpy().astype(np.float64).any()


def test_linear_is_deterministic():
    shp = synth.SHAPES["llama7b_mlp_down_16x4096x11008"]
    p = _prep(shp.name, None)
    X, packed, s = p.to_device()
    a = fp6.linear(X, packed, s, shp.N, shp.K).clone()
    b = fp6.linear(X, packed, s, shp.N, shp.K).clone()
    c = fp6.linear_plan(X, packed, s, shp.N, shp.K, variant=1, splits=8).clone()
    d = fp6.linear_plan(X, packed, s, shp.N, shp.K, variant=1, splits=8).clone()
    torch.cuda.synchronize()
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))
    assert torch.equal(c.view(torch.int16), d.view(torch.int16))


def test_linear_very_long_k_and_minimum_shape():
    for (M, N, K) in [(4, 16, 2**18), (1, 16, 256)]:
        p = Prepared(M, N, K, seed_w=K + 5, seed_x=K + 6)
        X, packed, s = p.to_device()
        Y = fp6.linear(X, packed, s, N, K)
        torch.cuda.synchronize()
        _assert_tol(Y, p.y_ref, what=(M, N, K))


def test_linear_m_zero_is_noop():
    N, K = 16, 256
    packed = torch.zeros(fp6.packed_bytes(N, K), dtype=torch.uint8, device=DEV)
    s = torch.ones(N, dtype=torch.float16, device=DEV)
    X = torch.zeros((0, K), dtype=torch.float16, device=DEV)
    Y = fp6.linear(X, packed, s, N, K)
    torch.cuda.synchronize()
    assert Y.shape == (0, N)


def test_linear_on_side_stream_matches_default_stream():
    shp = synth.SHAPES["llama7b_attn_1x4096x4096"]
    p = _prep(shp.name, None)
    X, packed, s = p.to_device()
    a = fp6.linear(X, packed, s, shp.N, shp.K)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        b = fp6.linear(X, packed, s, shp.N, shp.K)
    torch.cuda.synchronize()
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))
    _assert_tol(b, p.y_ref)


def test_split_k_plans_run_concurrently_on_several_streams():
    # Each stream has its own split-K workspace: split plans queued on four
    # streams without synchronisation in between (dense k-split, streaming
    # and tiled fix-ups, sparse k-split) must each equal their one-stream
    # result bit for bit.
    cases = [(16, 8192, 8192, 0, 0, False), (5, 2048, 11008, 15, 3, False),
             (128, 2048, 7168, 10, 3, False), (16, 8192, 8192, 0, 0, True)]
    streams = [torch.cuda.Stream() for _ in range(4)]
    prepared = []
    for i, (M, N, K, v, sp, sparse) in enumerate(cases):
        W = synth.weights(N, K, 820 + i)
        X = torch.from_numpy(synth.activations(M, K, 830 + i)).to(DEV)
        if sparse:
            c, pos, sc = fp6.prune_quantize(W)
            P = torch.from_numpy(fp6.sparse_prepack(c, pos, sc, K)).to(DEV)
            run = fp6.sparse_linear_plan
        else:
            c, sc = fp6.quantize_rows(W)
            P = torch.from_numpy(fp6.prepack(c, sc)).to(DEV)
            run = fp6.linear_plan
        S = torch.from_numpy(sc.copy()).to(DEV)
        want = run(X, P, S, N, K, variant=v, splits=sp).clone()
        prepared.append((run, X, P, S, N, K, v, sp, want))
    torch.cuda.synchronize()
    outs = [[] for _ in cases]
    for st in streams:
        st.wait_stream(torch.cuda.current_stream())
    for rep in range(6):
        for i, (run, X, P, S, N, K, v, sp, want) in enumerate(prepared):
            st = streams[(i + rep) % len(streams)]
            with torch.cuda.stream(st):
                outs[i].append(run(X, P, S, N, K, variant=v, splits=sp, stream=st))
    torch.cuda.synchronize()
    for i, (run, X, P, S, N, K, v, sp, want) in enumerate(prepared):
        for rep, y in enumerate(outs[i]):
            assert torch.equal(y.view(torch.int16), want.view(torch.int16)), (cases[i], rep)


def test_release_then_reuse_and_grow_workspace():
    # The split-K workspace is allocated on first need, grown on demand and
    # freed by release(); a later split call must allocate it again and give
    # the same bits.
    p = Prepared(16, 256, 4096, seed_w=77, seed_x=78)
    X, packed, s = p.to_device()
    a = fp6.linear_plan(X, packed, s, p.N, p.K, variant=15, splits=2).clone()
    fp6.release()
    b = fp6.linear_plan(X, packed, s, p.N, p.K, variant=15, splits=2).clone()
    c = fp6.linear_plan(X, packed, s, p.N, p.K, variant=10, splits=16).clone()  # larger workspace
    fp6.release()
    fp6.release()  # nothing left to free
    torch.cuda.synchronize()
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))
    _assert_tol(a, p.y_ref, what="split 2")
    _assert_tol(c, p.y_ref, what="split 16")


def _adversarial_weights(N, K, seed):
    """Rows that exercise the corners of quantisation and de-quantisation:
    a zero row (scale 0), a lone outlier over values that quantise to zero or
    subnormals, a row of negative values below half the smallest subnormal
    (codes -0) plus one outlier, saturating +-max, exact ties between e3m2
    magnitudes (scale 2^-4 exactly), a large scale (|s| close to 16), then
    ordinary N(0, 0.02) rows."""
    rng = np.random.default_rng(seed)
    W = (rng.standard_normal((N, K)) * 0.02).astype(np.float32)
    W[0] = 0.0
    W[1] = 1e-6
    W[1, 5] = 1.0
    W[2] = -1e-9
    W[2, 7] = 0.5
    W[3] = np.where(np.arange(K) % 2 == 0, 1.0, -1.0)
    mags = np.array(oracle.E3M2_VALUES[:32], dtype=np.float64)
    mids = (mags[:-1] + mags[1:]) / 2                      # ties between neighbours
    row = np.resize(np.concatenate([mids, -mids]), K) * 2.0 ** -4
    row[0] = 28 * 2.0 ** -4                                 # max |W| -> scale exactly 2^-4
    W[4] = row.astype(np.float32)
    W[5] = (rng.standard_normal(K) * 100).astype(np.float32)
    W[5, 3] = 400.0                                         # scale 400/28 ~ 14.3
    return W


@pytest.mark.parametrize("M", [3, 17])
def test_linear_adversarial_rows(M):
    N, K = 96, 2816
    W = _adversarial_weights(N, K, seed=123 + M)
    X = synth.activations(M, K, 321 + M)
    X[:, ::7] = 0
    p = Prepared(M, N, K, seed_w=0, seed_x=0, W=W, X=X)
    assert np.array_equal(p.codes, p.ocodes) and np.array_equal(p.scales.view(np.uint16), p.oscales.view(np.uint16))
    Xd, packed, s = p.to_device()
    assert np.array_equal(_bits16(fp6.dequant(packed, s, N, K)), p.wdq_ref.view(np.uint16))
    for variant, splits in [(0, 0), (1, 3), (15, 2), (18, 1), (10, 1), (17, 3), (19, 3), (22, 2)]:
        Y = fp6.linear_plan(Xd, packed, s, N, K, variant=variant, splits=splits)
        torch.cuda.synchronize()
        _assert_tol(Y, p.y_ref, what=(M, variant, splits))
        # the zero row gives exactly zero outputs
        assert not Y[:, 0].cpu().numpy().astype(np.float64).any(), (M, variant, splits)


@pytest.mark.parametrize("M, N, K", [(1, 1 << 20, 256), (40, 1 << 20, 256), (2, 16, 1 << 22)])
def test_linear_large_n_or_k(M, N, K):
    # Far beyond the workloads in one dimension: a million output rows (at
    # M=1 the persistent k-split kernel walks 256 row blocks per workgroup; at
    # M=40 the whole-tile tiled kernel launches 4096 workgroups), or K = 4M
    # with a single row block (the plan splits K 64 ways through the fix-up).
    # Sampled output columns.
    p = Prepared(M, N, K, seed_w=N + K + 1, seed_x=M + 2, sample=256)
    X, packed, s = p.to_device()
    Y = fp6.linear(X, packed, s, N, K)
    torch.cuda.synchronize()
    _assert_tol(Y[:, torch.from_numpy(p.rows).to(DEV)], p.y_ref, what=(M, N, K))


# ----------------------------------------------------------------------------
# Automatic plans (schedule rules) on a 256-CU MI355X
# ----------------------------------------------------------------------------
DENSE_PLANS = [
    ((1, 4096, 4096), (KSLICE, 1)),      # one row block per CU: k-slice
    ((16, 4096, 2048), (KSLICE, 1)),
    ((16, 8192, 2048), (KSPLIT, 1)),     # K <= 2048: 8-wave k-split
    ((16, 11008, 4096), (KSPLIT16, 1)),  # 3 row blocks per workgroup in flight
    ((16, 8192, 8192), (KSPLIT16, 2)),   # K split across workgroups
    ((16, 5120, 5120), (KSPLIT, 3)),     # 8 waves: fewer idle waves on 10-tile splits
    ((16, 4096, 11008), (KSPLIT16, 3)),
    ((1, 4096, 11008), (KSLICE, 1)),     # M <= 4, one row block per CU: k-slice up to K = 12288
    ((16, 28672, 8192), (18, 1)),        # streaming, 8 waves, one round of workgroups
    ((16, 57344, 8192), (16, 1)),        # 2 row blocks per wave: one round instead of 1.75
    ((16, 8192, 28672), (14, 4)),        # 2 row blocks per wave, split while a whole round fits
    ((32, 21504, 7168), (19, 3)),        # 32 columns per workgroup
    ((64, 4096, 4096), (22, 4)),         # 64 columns, 1 row block per wave
    ((64, 21504, 7168), (20, 3)),
    ((128, 21504, 7168), (10, 3)),       # tiled
    ((128, 8192, 8192), (22, 2)),        # two 64-column passes on a narrower layer
    ((72, 4096, 11008), (22, 4)),
    ((256, 4096, 4096), (22, 2)),
    ((256, 8192, 8192), (10, 4)),        # as many workgroups as CUs: tiled
]
SPARSE_PLANS = [
    ((1, 4096, 4096), (1, 1)),
    ((16, 11008, 4096), (6, 1)),
    ((16, 4096, 4096), (6, 1)),          # one row block per CU, M >= 12: k-split
    ((8, 4096, 4096), (1, 1)),           # M <= 11: k-slice
    ((16, 13824, 5120), (2, 1)),         # 7 row blocks per workgroup: streaming
    ((16, 8192, 8192), (6, 2)),
    ((16, 28672, 8192), (2, 1)),
    ((16, 8192, 28672), (3, 4)),
    ((32, 21504, 7168), (8, 3)),
    ((64, 21504, 7168), (4, 3)),
    ((128, 4096, 4096), (7, 2)),         # 32-column passes on a narrow layer
    ((48, 11008, 4096), (7, 1)),
]


def test_automatic_plans_on_256_cus():
    # The schedule rules picked from the measurements; the rules depend on
    # the CU count, so they are pinned for the 256-CU part only.
    if torch.cuda.get_device_properties(0).multi_processor_count != 256:
        pytest.skip("plans pinned for 256 CUs")
    for (M, N, K), want in DENSE_PLANS:
        assert fp6.plan_query(M, N, K) == want, (M, N, K)
    for (M, N, K), want in SPARSE_PLANS:
        assert fp6.sparse_plan_query(M, N, K) == want, (M, N, K)
