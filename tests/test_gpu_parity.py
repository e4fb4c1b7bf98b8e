"""GPU parity of the HIP path against the CPU oracle (needs an MI355X).

* De-quantisation export: bit-exact against oracle.dequant_ref.
* Fused linear: |Y - Y_ref| <= 2e-3 (|Y_ref| + rms(Y_ref)) per element and
  relative Frobenius error <= 5e-4, with rms over the whole output, on every
  output element of every workload shape at full size and of small shapes
  that span several tiles with ragged M; one-hot inputs must reproduce Wdq
  exactly.
"""

import numpy as np
import pytest

import oracle
from weight_only_fp6_amd import synth

from _workloads import Prepared, dense_weight_set, workload, y_ref

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():  # pragma: no cover - CPU container
    pytest.skip("no GPU", allow_module_level=True)

import weight_only_fp6_amd as fp6  # noqa: E402

DEV = torch.device("cuda:0")
# Kernel configurations of fp6_linear_plan: 0 = automatic, 1-4 and 7-8
# streaming, 5-6 and 10-11 tiled, 9 k-split persistent (M <= 16, K <= 8192).
ALL_VARIANTS = (0, 1, 2, 3, 4, 5, 6, 7, 8, 10, 11, 14, 15, 16, 17, 18, 19, 20, 21, 22, 23, 24, 25)
KSPLIT = 9
KSPLIT16 = 12
KSLICE = 13
KRING = 26
SMALL_M = (KSPLIT, KSPLIT16, KSLICE, KRING)   # M <= 16 only


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


def _weight_set_names():
    """The first synth.SHAPES entry of every distinct weight set, in order."""
    seen = {}
    for name, shp in synth.SHAPES.items():
        seen.setdefault((shp.N, shp.K, shp.seed_w), name)
    return list(seen.values())


@pytest.mark.parametrize("name", _weight_set_names())
def test_dequant_workload_weights(name):
    # The whole de-quantised weight matrix of every workload layer (up to
    # 28672 x 8192), bit for bit; the library quantiser's codes and scales
    # equal the oracle's on every row.
    shp = synth.SHAPES[name]
    ws = dense_weight_set(shp.N, shp.K, shp.seed_w)
    assert ws.codes_match and ws.scales_match, name
    packed, s = ws.to_device()
    out = fp6.dequant(packed, s, shp.N, shp.K)
    torch.cuda.synchronize()
    assert np.array_equal(_bits16(out), ws.wdq_ref.view(np.uint16)), name


# ----------------------------------------------------------------------------
# Fused linear at the workload shapes (automatic plan = the benchmarked launch),
# every output element against Y_ref of the whole layer
# ----------------------------------------------------------------------------
class _full:
    """A whole workload layer on the device with Y_ref of every output."""

    def __init__(self, name):
        self.ws, self.X, self.y_ref = workload(name)

    def to_device(self):
        packed, s = self.ws.to_device()
        return torch.from_numpy(self.X).to(DEV), packed, s


@pytest.mark.parametrize("name", list(synth.SHAPES))
def test_linear_workloads(name):
    shp = synth.SHAPES[name]
    ws, X, yref = workload(name)
    packed, s = ws.to_device()
    Y = fp6.linear(torch.from_numpy(X).to(DEV), packed, s, shp.N, shp.K)
    torch.cuda.synchronize()
    _assert_tol(Y, yref, what=(name, fp6.plan_query(shp.M, shp.N, shp.K)))


# ----------------------------------------------------------------------------
# Small shapes spanning several tiles, ragged M, forced schedules
# ----------------------------------------------------------------------------
@pytest.mark.parametrize("M", [1, 2, 3, 5, 8, 15, 16, 17, 31, 33, 64, 100, 257])
@pytest.mark.parametrize("NK", [(16, 256), (64, 1024), (80, 2816)])
def test_linear_small_shapes_ragged_m(M, NK):
    N, K = NK
    p = Prepared(M, N, K, seed_w=N * 7 + K, seed_x=M * 11 + 1)
    X, packed, s = p.to_device()
    for variant in ALL_VARIANTS + (SMALL_M if M <= 16 else ()):
        Y = fp6.linear_plan(X, packed, s, N, K, variant=variant)
        torch.cuda.synchronize()
        _assert_tol(Y, p.y_ref, what=(M, N, K, variant))


@pytest.mark.parametrize("splits", [1, 2, 3, 4, 7, 8, 16, 43])
def test_linear_forced_splits_long_k(splits):
    # Llama-7B MLP down projection: K = 11008 = 43 tiles of 256 (43 is prime)
    shp = synth.SHAPES["llama7b_mlp_down_16x4096x11008"]
    p = _full(shp.name)
    X, packed, s = p.to_device()
    for variant in (1, 3, 5, 6, 10, 11, 14, 16, 17, 18, 19, 20, 21, 22, 23, 24):
        Y = fp6.linear_plan(X, packed, s, shp.N, shp.K, variant=variant, splits=splits)
        torch.cuda.synchronize()
        _assert_tol(Y, p.y_ref, what=(splits, variant))


KCOV_K = (256, 512, 1280, 2048, 4096, 6144, 8192, 8448, 11008, 12288)


@pytest.mark.parametrize("K, M", [(K, M) for K in KCOV_K for M in (1, 2, 4, 16)])
def test_linear_ksplit_k_coverage(K, M):
    # The k-split and k-slice kernels at every per-wave tile count: k-split
    # 1..4 tiles per wave up to K = 8192; k-slice 1..3 (K = 8448 and 11008
    # leave ragged 2-or-3-tile ranges, 12288 is 3 tiles in every wave), with
    # more row blocks than workgroups (N = 16*300 > 256); and the automatic
    # plan.  Every output element.
    N = 16 * 300
    ws = dense_weight_set(N, K, K + 7)
    X = synth.activations(M, K, K * 3 + M)
    yref = y_ref(X, ws.wdq_ref)
    Xd = torch.from_numpy(X).to(DEV)
    packed, s = ws.to_device()
    variants = (0,) + SMALL_M if K <= 8192 else (0, KSLICE)
    for variant in variants:
        Y = fp6.linear_plan(Xd, packed, s, N, K, variant=variant)
        torch.cuda.synchronize()
        _assert_tol(Y, yref, what=(M, K, variant))


@pytest.mark.parametrize("K", [8448, 11008, 12288])
def test_kslice_one_hot_third_tile_slot(K):
    # One-hot activations through the k-slice kernel with 3 tiles per wave:
    # columns land in each of a wave's three tile slots (and in the k-steps,
    # lane groups and elements inside a tile), so every output must equal a
    # de-quantised weight exactly.
    N, M = 64, 16
    ws = dense_weight_set(N, K, K + 11)
    kt = K // 256
    cols, slots = [], []
    for m in range(M):
        w = (5 * m + 3) % 16                        # wave w owns tiles [k0, k1)
        k0, k1 = w * kt // 16, (w + 1) * kt // 16
        slot = k1 - k0 - 1 if m % 2 == 0 else (m // 2) % (k1 - k0)
        slots.append(slot)
        cols.append((k0 + slot) * 256 + (37 * m + 11) % 256)
    assert 2 in slots
    ks = np.array(cols)
    X = np.zeros((M, K), np.float16)
    X[np.arange(M), ks] = 1.0
    Xd = torch.from_numpy(X).to(DEV)
    packed, s = ws.to_device()
    want = ws.wdq_ref[:, ks].T.astype(np.float64)
    for m_used in (1, 2, 4, 16):
        Y = fp6.linear_plan(Xd[:m_used].contiguous(), packed, s, N, K, variant=KSLICE)
        torch.cuda.synchronize()
        assert np.array_equal(Y.cpu().numpy().astype(np.float64), want[:m_used]), (K, m_used)


@pytest.mark.parametrize("K, per_wg, M", [(K, w, M) for K in (2048, 4096) for w in (2, 3, 4, 5, 7, 9)
                                          for M in (1, 5, 16)])
def test_linear_ksplit_row_blocks_per_workgroup(K, per_wg, M):
    # The k-split kernels run straight-line code for 2-8 row blocks per
    # workgroup (4 register stages; a workgroup with fewer than the form's
    # count repeats its last row block) and loop beyond.  N is sized from the
    # CU count so that the first workgroups get per_wg row blocks and the rest
    # per_wg - 1.  At K = 2048 half of the 16 waves have an empty k-range.
    # Every output element.
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    nblocks = (per_wg - 1) * cus + max(cus // 3, 1)
    N = 16 * nblocks
    ws = dense_weight_set(N, K, 900 + per_wg + K)
    X = synth.activations(M, K, 910 + M)
    yref = y_ref(X, ws.wdq_ref)
    Xd = torch.from_numpy(X).to(DEV)
    Pd, Sd = ws.to_device()
    for variant in (KSPLIT, KSPLIT16):
        Y = fp6.linear_plan(Xd, Pd, Sd, N, K, variant=variant)
        torch.cuda.synchronize()
        _assert_tol(Y, yref, what=(M, per_wg, K, variant))


@pytest.mark.parametrize("NK, M", [(NK, M) for NK in ((4096, 11008), (1024, 6400), (2048, 2304))
                                   for M in (1, 5, 16)])
def test_linear_ksplit_across_workgroups(NK, M):
    # The k-split kernels with K split across workgroups (fixed-order
    # fix-up): straight-line and looping forms, ragged split ranges, idle
    # waves; bitwise reproducible from run to run.  Every output element.
    N, K = NK
    ws = dense_weight_set(N, K, N + K + 5)
    X = synth.activations(M, K, M + 3)
    yref = y_ref(X, ws.wdq_ref)
    Xd = torch.from_numpy(X).to(DEV)
    packed, s = ws.to_device()
    ktiles = K // 256
    for variant, wk in ((KSPLIT, 8), (KSPLIT16, 16)):
        for splits in (2, 3, 4, 7):
            if splits > ktiles or -(-ktiles // splits) > 32:
                continue
            Y = fp6.linear_plan(Xd, packed, s, N, K, variant=variant, splits=splits).clone()
            Y2 = fp6.linear_plan(Xd, packed, s, N, K, variant=variant, splits=splits)
            torch.cuda.synchronize()
            _assert_tol(Y, yref, what=(M, N, K, variant, splits))
            assert torch.equal(Y.view(torch.int16), Y2.view(torch.int16)), (M, N, K, variant, splits)


@pytest.mark.parametrize("K, per_wg, M", [(K, w, M) for K, ws in ((256, (1, 3)), (2048, (1, 2, 3, 8)),
                                                                    (2816, (1, 2, 3, 5, 8)),
                                                                    (5120, (2, 3, 4)), (7168, (3,)), (8192, (2,)))
                                          for w in ws for M in (1, 5, 16)])
def test_linear_kring_row_blocks_per_workgroup(K, per_wg, M):
    # The k-ring kernel: each of 8 waves holds a fixed K slice of X (K/256 = 1
    # leaves 7 waves with an empty slice and stand-in tiles, 11, 20 and 28
    # k-tiles give ragged 1/2, 2/3 and 3/4-tile slices) and walks per_wg
    # row blocks (the last workgroup fewer); with one k-tile per wave (K <=
    # 2048) two row blocks are in flight, odd and even counts.  Every output
    # element.
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    nblocks = (per_wg - 1) * cus + max(cus // 3, 1) if per_wg > 1 else cus - 5
    N = 16 * nblocks
    ws = dense_weight_set(N, K, 700 + per_wg + K)
    X = synth.activations(M, K, 710 + M)
    yref = y_ref(X, ws.wdq_ref)
    Xd = torch.from_numpy(X).to(DEV)
    Pd, Sd = ws.to_device()
    Y = fp6.linear_plan(Xd, Pd, Sd, N, K, variant=KRING).clone()
    Y2 = fp6.linear_plan(Xd, Pd, Sd, N, K, variant=KRING)
    torch.cuda.synchronize()
    _assert_tol(Y, yref, what=(M, per_wg, K))
    assert torch.equal(Y.view(torch.int16), Y2.view(torch.int16)), (M, per_wg, K)


@pytest.mark.parametrize("name", ["llama70b_mlp_1x28672x8192", "llama70b_mlp_16x28672x8192",
                                  "llama7b_mlp_up_16x11008x4096"])
def test_linear_kring_workload_layers(name):
    # The k-ring kernel forced on whole workload layers: the Llama-70B MLP
    # (1792 row blocks = 7 per CU at 256 CUs, K = 8192: 4 k-tiles per wave)
    # and the Llama-7B MLP up projection.  Every output element.
    shp = synth.SHAPES[name]
    p = _full(name)
    X, packed, s = p.to_device()
    Y = fp6.linear_plan(X, packed, s, shp.N, shp.K, variant=KRING)
    torch.cuda.synchronize()
    _assert_tol(Y, p.y_ref, what=name)


@pytest.mark.parametrize("NK, M, splits", [(NK, M, sp) for NK in ((4096, 11008), (1024, 8448), (2048, 12288))
                                            for M in (1, 5, 16) for sp in (0, 2, 3)])
def test_linear_kring_k_splits(NK, M, splits):
    # The k-ring kernel with K split across workgroups (automatic: the fewest
    # splits that leave at most 4 k-tiles per wave) and the fixed-order
    # fix-up: ragged split and wave ranges, bitwise reproducible.  Every
    # output element.
    N, K = NK
    ws = dense_weight_set(N, K, N + K + 13)
    X = synth.activations(M, K, M + 17)
    yref = y_ref(X, ws.wdq_ref)
    Xd = torch.from_numpy(X).to(DEV)
    packed, s = ws.to_device()
    Y = fp6.linear_plan(Xd, packed, s, N, K, variant=KRING, splits=splits).clone()
    Y2 = fp6.linear_plan(Xd, packed, s, N, K, variant=KRING, splits=splits)
    torch.cuda.synchronize()
    _assert_tol(Y, yref, what=(M, N, K, splits))
    assert torch.equal(Y.view(torch.int16), Y2.view(torch.int16)), (M, N, K, splits)


@pytest.mark.parametrize("M, N, K", [(1, 6144, 11008), (4, 5120, 12288), (1, 2048, 11008), (8, 4096, 9216),
                                     (5, 2048, 5120), (16, 2560, 7168)])
def test_linear_auto_kring_k_split_layers(M, N, K):
    # Automatic plans that take the k-ring kernel with 2 K-splits: for
    # 8192 < K <= 12288, 3 row blocks per workgroup at M = 1 (X loaded
    # directly) and M = 4, one per workgroup on half of the CUs, and 2 per
    # workgroup at M = 8 (ragged wave ranges of 2-3 k-tiles); for narrow
    # layers with K <= 8192, 1-2 k-tiles per wave with one row block per
    # workgroup, and 2 row blocks per workgroup.  Every output element, and
    # the plan that produced it.
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    if cus != 256:
        pytest.skip("plan thresholds are stated for 256 CUs")
    assert fp6.plan_query(M, N, K) == (KRING, 2)
    ws = dense_weight_set(N, K, N + K + 29)
    X = synth.activations(M, K, M + 31)
    yref = y_ref(X, ws.wdq_ref)
    Xd = torch.from_numpy(X).to(DEV)
    packed, s = ws.to_device()
    Y = fp6.linear(Xd, packed, s, N, K)
    torch.cuda.synchronize()
    _assert_tol(Y, yref, what=(M, N, K))


def test_kring_one_hot_every_tile_slot():
    # One-hot activations through the k-ring kernel at K = 7168 (28 k-tiles:
    # waves own 3 or 4), 3 row blocks per workgroup with a short last
    # workgroup: columns land in every tile slot of several waves, so every
    # output must equal a de-quantised weight exactly.
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    N, K, M = 16 * (2 * cus + 7), 7168, 16
    ws = dense_weight_set(N, K, 4242)
    kt = K // 256
    cols = []
    for m in range(M):
        w = (3 * m + 1) % 8
        k0, k1 = w * kt // 8, (w + 1) * kt // 8
        slot = m % (k1 - k0)
        cols.append((k0 + slot) * 256 + (41 * m + 5) % 256)
    ks = np.array(cols)
    X = np.zeros((M, K), np.float16)
    X[np.arange(M), ks] = 1.0
    Xd = torch.from_numpy(X).to(DEV)
    packed, s = ws.to_device()
    want = ws.wdq_ref[:, ks].T.astype(np.float64)
    for m_used in (1, 5, 16):
        Y = fp6.linear_plan(Xd[:m_used].contiguous(), packed, s, N, K, variant=KRING)
        torch.cuda.synchronize()
        assert np.array_equal(Y.cpu().numpy().astype(np.float64), want[:m_used]), m_used


def test_kring_rejects_what_it_does_not_cover():
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    p = Prepared(16, 64, 512, seed_w=15, seed_x=16)
    X, packed, s = p.to_device()
    X17 = torch.zeros((17, 512), dtype=torch.float16, device=DEV)
    with pytest.raises(fp6.FP6Error):      # M <= 16
        fp6.linear_plan(X17, packed, s, 64, 512, variant=KRING)
    N = 16 * (8 * cus + 1)                 # 9 row blocks per CU
    big = torch.zeros(fp6.packed_bytes(N, 256), dtype=torch.uint8, device=DEV)
    sc = torch.zeros(N, dtype=torch.float16, device=DEV)
    X1 = torch.zeros((1, 256), dtype=torch.float16, device=DEV)
    with pytest.raises(fp6.FP6Error):
        fp6.linear_plan(X1, big, sc, N, 256, variant=KRING)
    Xk = torch.zeros((1, 8448), dtype=torch.float16, device=DEV)
    wk = torch.zeros(fp6.packed_bytes(64, 8448), dtype=torch.uint8, device=DEV)
    with pytest.raises(fp6.FP6Error):      # at most 32 k-tiles (4 per wave) per K-split
        fp6.linear_plan(Xk, wk, s, 64, 8448, variant=KRING, splits=1)
    N2 = 16 * (4 * cus + 1)                # 2 K-splits x 4+ row blocks: 9 units per CU
    big2 = torch.zeros(fp6.packed_bytes(N2, 8448), dtype=torch.uint8, device=DEV)
    sc2 = torch.zeros(N2, dtype=torch.float16, device=DEV)
    with pytest.raises(fp6.FP6Error):
        fp6.linear_plan(Xk, big2, sc2, N2, 8448, variant=KRING)


STREAM_K = 25


@pytest.mark.parametrize("M, N, K", [
    (128, 21504, 7168),   # OPT-30B QKV: 84 tiles x 56 half-tiles over one workgroup per CU
    (256, 21504, 7168),   # two column groups, 168 tiles
    (200, 4096, 4096),    # ragged M: the second column group is part empty
    (64, 1024, 11008),    # 4 tiles of 86 half-tiles: dozens of pieces per tile
    (1, 16, 256),         # one tile of 2 half-tiles: most workgroups idle
    (768, 25600, 256),    # 600 tiles of 2 half-tiles: a workgroup runs tails, whole tiles and heads
])
def test_linear_stream_k(M, N, K):
    # The stream-K tiled kernel: every output element against Y_ref, and
    # bitwise reproducible from run to run (fixed piece order).
    # The OPT-30B layer shares the workload tests' weight set (cached).
    seed = synth.SHAPES["opt30b_qkv_128x21504x7168"].seed_w if (N, K) == (21504, 7168) else 7 * N + K
    ws = dense_weight_set(N, K, seed)
    X = synth.activations(M, K, M + 29)
    yref = y_ref(X, ws.wdq_ref)
    Xd = torch.from_numpy(X).to(DEV)
    packed, s = ws.to_device()
    Y = fp6.linear_plan(Xd, packed, s, N, K, variant=STREAM_K).clone()
    Y2 = fp6.linear_plan(Xd, packed, s, N, K, variant=STREAM_K)
    torch.cuda.synchronize()
    _assert_tol(Y, yref, what=(M, N, K))
    assert torch.equal(Y.view(torch.int16), Y2.view(torch.int16)), (M, N, K)


def test_linear_stream_k_rejects_splits():
    p = Prepared(128, 64, 512, seed_w=5, seed_x=6)
    X, packed, s = p.to_device()
    with pytest.raises(fp6.FP6Error):
        fp6.linear_plan(X, packed, s, 64, 512, variant=STREAM_K, splits=2)


def test_linear_one_hot_reproduces_wdq_exactly():
    N, K = 64, 1024
    p = Prepared(16, N, K, seed_w=99, seed_x=1)
    ks = np.array([0, 1, 7, 8, 255, 256, 300, 511, 512, 777, 1000, 1023, 31, 32, 33, 600])
    X = np.zeros((16, K), np.float16)
    X[np.arange(16), ks] = 1.0
    Xd = torch.from_numpy(X).to(DEV)
    _, packed, s = p.to_device()
    for variant, splits in [(0, 0), (1, 1), (1, 4), (2, 1), (2, 3), (3, 2), (4, 1), (5, 1), (5, 3), (6, 1), (6, 2), (7, 2), (8, 1), (KSPLIT, 0), (KSPLIT16, 0), (KSLICE, 0), (14, 1), (15, 2), (16, 1), (10, 1), (10, 3), (11, 2), (17, 1), (17, 3), (18, 1), (18, 3), (19, 2), (20, 3), (21, 1), (22, 4), (23, 1), (23, 3), (24, 2), (25, 0), (KRING, 0)]:
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
    p = _full(shp.name)
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
    p = _full(shp.name)
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
    for variant, splits in [(0, 0), (1, 3), (15, 2), (18, 1), (10, 1), (17, 3), (19, 3), (22, 2), (23, 2), (24, 1), (25, 0)]:
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
    # Every output element.
    ws = dense_weight_set(N, K, N + K + 1)
    X = synth.activations(M, K, M + 2)
    yref = y_ref(X, ws.wdq_ref)
    packed, s = ws.to_device()
    Y = fp6.linear(torch.from_numpy(X).to(DEV), packed, s, N, K)
    torch.cuda.synchronize()
    _assert_tol(Y, yref, what=(M, N, K))


# ----------------------------------------------------------------------------
# Automatic plans (schedule rules) on a 256-CU MI355X
# ----------------------------------------------------------------------------
DENSE_PLANS = [
    ((1, 4096, 4096), (KSLICE, 1)),      # one row block per CU: k-slice
    ((4, 4096, 8192), (KSLICE, 1)),      # M <= 4, one row block per CU: k-slice
    ((16, 4096, 2048), (KRING, 1)),      # M > 4, every CU a row block: k-ring
    ((16, 8192, 2048), (KRING, 1)),      # K <= 4096: k-ring up to 8 row blocks per CU
    ((16, 28672, 4096), (KRING, 1)),
    ((16, 11008, 4096), (KRING, 1)),
    ((16, 8192, 8192), (KRING, 1)),      # longer K: k-ring up to 3 row blocks per CU
    ((1, 10240, 8192), (KRING, 1)),
    ((16, 5120, 5120), (KRING, 1)),
    ((16, 13824, 5120), (15, 1)),        # 4 row blocks per CU at K > 4096: streaming
    ((16, 18432, 8192), (KRING, 1)),     # 4-wave streaming workgroups would take 1.1 rounds
    ((4, 25600, 8192), (KRING, 1)),
    ((16, 2048, 8192), (KRING, 2)),      # half the CUs with a row block: k-ring, 2 K-splits
    ((8, 2048, 6144), (KRING, 2)),
    ((16, 3072, 6144), (KSPLIT, 3)),     # 3/4 of them, < 28 k-tiles: k-split kernel, K split
    ((16, 4096, 11008), (KRING, 2)),     # 8192 < K <= 12288, <= 3 row blocks per CU: k-ring, 2 K-splits
    ((16, 8192, 10240), (15, 2)),        # 4 per CU: streaming
    ((16, 3072, 8192), (KRING, 2)),      # 2 row blocks per workgroup at 32 k-tiles
    ((1, 4096, 11008), (KSLICE, 1)),     # M <= 4, one row block per CU: k-slice up to K = 12288
    ((3, 3072, 12288), (KSLICE, 1)),     # ... while more than half of the CUs have a row block
    ((1, 2048, 11008), (KRING, 2)),      # half of them: k-ring, 2 K-splits
    ((1, 6144, 11008), (KRING, 2)),      # more row blocks than CUs, <= 3 per CU after the split
    ((4, 5120, 12288), (KRING, 2)),
    ((16, 28672, 8192), (18, 1)),        # streaming, 8 waves, one round of workgroups
    ((16, 57344, 8192), (16, 1)),        # 2 row blocks per wave: one round instead of 1.75
    ((16, 8192, 28672), (15, 2)),        # split while a whole round of 4-wave workgroups fits
    ((32, 21504, 7168), (19, 3)),        # 32 columns per workgroup
    ((64, 4096, 4096), (22, 4)),         # 64 columns, 1 row block per wave
    ((64, 21504, 7168), (20, 3)),
    ((128, 21504, 7168), (10, 3)),       # tiled
    ((128, 8192, 8192), (22, 2)),        # two 64-column passes on a narrower layer
    ((72, 4096, 11008), (22, 4)),
    ((256, 4096, 4096), (22, 2)),
    ((256, 8192, 8192), (10, 4)),        # as many workgroups as CUs: tiled
    ((256, 21504, 7168), (25, 256)),     # 168 tiles: stream-K, one workgroup per CU
    ((512, 21504, 7168), (10, 1)),       # 336 tiles, more than CUs: split-K rounds
]
SPARSE_PLANS = [
    ((1, 4096, 4096), (1, 1)),
    ((16, 11008, 4096), (9, 1)),         # 3 row blocks per CU, K = 4096: k-ring
    ((16, 4096, 4096), (6, 1)),          # one row block per CU, M >= 12: k-split
    ((8, 4096, 4096), (1, 1)),           # M <= 11: k-slice
    ((16, 13824, 5120), (2, 1)),         # K/512 = 10 sparse tiles, ragged over 8 waves: streaming
    ((16, 8192, 8192), (9, 1)),
    ((16, 28672, 8192), (9, 1)),         # 7 row blocks per CU: k-ring
    ((1, 28672, 8192), (9, 1)),
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
