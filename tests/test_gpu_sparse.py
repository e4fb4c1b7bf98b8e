"""GPU parity of the 2:4-sparse FP6 path (fp6s_*) against the CPU oracle
(oracle/sparse24.py), needs an MI355X.

* De-quantisation export: dense Wdq (zeros at pruned positions) bit-exact.
* Fused sparse linear: |Y - Y_ref| <= 2e-3 (|Y_ref| + rms) per element and
  relative Frobenius <= 5e-4, every kernel configuration on small ragged
  shapes, the automatic plan on every output element of the workload layers
  whose K is a multiple of 512, at full size; one-hot activations reproduce
  Wdq exactly.
"""

import numpy as np
import pytest

import oracle
from oracle import sparse24
from weight_only_fp6_amd import synth

from _workloads import sparse_weight_set, workload, y_ref

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():  # pragma: no cover - CPU container
    pytest.skip("no GPU", allow_module_level=True)

import weight_only_fp6_amd as fp6  # noqa: E402

DEV = torch.device("cuda:0")
VARIANTS = (0, 2, 3, 4, 5, 7, 8)     # any M; 1 (k-slice) and 6 (k-split) only for M <= 16
KSLICE = 1
KSPLIT = 6
KRING = 9


class SpPrepared:
    """A 2:4-sparse layer (synthetic weights pruned and quantised by the
    library and by the oracle) with Y_ref of every output element."""

    def __init__(self, M, N, K, seed_w, seed_x):
        self.M, self.N, self.K = M, N, K
        self.ws = sparse_weight_set(N, K, seed_w)
        self.X = synth.activations(M, K, seed_x)
        self.scales, self.packed, self.wdq_ref = self.ws.scales, self.ws.packed, self.ws.wdq_ref
        self.y_ref = y_ref(self.X, self.wdq_ref)

    def to_device(self):
        return (torch.from_numpy(self.X).to(DEV), torch.from_numpy(self.packed).to(DEV),
                torch.from_numpy(self.scales.copy()).to(DEV))


def _assert_tol(y_dev, y_ref, what=""):
    rep = oracle.tolerance_report(y_dev.detach().cpu().numpy().astype(np.float64), y_ref)
    assert rep["ok"], (what, rep)


def test_dequant_all_codes_and_position_pairs():
    N, K = 48, 1024
    rng = np.random.default_rng(61)
    codes = rng.integers(0, 64, (N, K // 2)).astype(np.uint8)
    pairs = np.array([(a, b) for a in range(4) for b in range(a + 1, 4)], np.uint8)   # all 6
    pos = pairs[rng.integers(0, 6, (N, K // 4))].reshape(N, K // 2)
    sb = rng.integers(1, 0x4C00, N).astype(np.uint16) | (rng.integers(0, 2, N).astype(np.uint16) << 15)
    scales = sb.view(np.float16)
    scales[:16] = np.array([2.0 ** j for j in range(-24, -8)], np.float16)     # subnormal weights
    packed = torch.from_numpy(fp6.sparse_prepack(codes, pos, scales, K)).to(DEV)
    s = torch.from_numpy(scales.copy()).to(DEV)
    out = fp6.sparse_dequant(packed, s, N, K)
    torch.cuda.synchronize()
    ref = sparse24.dequant_ref(codes, pos, scales, K)
    assert np.array_equal(out.cpu().numpy().view(np.uint16), ref.view(np.uint16))


@pytest.mark.parametrize("M", [1, 3, 16, 17, 64, 100, 257])
@pytest.mark.parametrize("NK", [(16, 512), (80, 1536), (48, 4608)])
def test_linear_small_shapes_every_variant(M, NK):
    N, K = NK
    p = SpPrepared(M, N, K, seed_w=N * 3 + K, seed_x=M * 7 + 5)
    X, packed, s = p.to_device()
    for variant in VARIANTS + ((KSLICE, KSPLIT, KRING) if M <= 16 else ()):
        Y = fp6.sparse_linear_plan(X, packed, s, N, K, variant=variant)
        torch.cuda.synchronize()
        _assert_tol(Y, p.y_ref, what=(M, N, K, variant))


def test_linear_forced_splits():
    p = SpPrepared(16, 4096, 8192, seed_w=71, seed_x=72)
    X, packed, s = p.to_device()
    for variant in (2, 3, 4, 5, 7, 8):
        for splits in (1, 2, 3, 5, 16):
            Y = fp6.sparse_linear_plan(X, packed, s, p.N, p.K, variant=variant, splits=splits)
            torch.cuda.synchronize()
            _assert_tol(Y, p.y_ref, what=(variant, splits))
    for splits in (2, 3, 5):    # k-split: <= 8 tiles per split, <= 8 row blocks per workgroup
        Y = fp6.sparse_linear_plan(X, packed, s, p.N, p.K, variant=KSPLIT, splits=splits)
        torch.cuda.synchronize()
        _assert_tol(Y, p.y_ref, what=(KSPLIT, splits))


SPARSE_SHAPES = [n for n, q in synth.SHAPES.items() if q.K % 512 == 0]


@pytest.mark.parametrize("name", SPARSE_SHAPES)
def test_linear_workloads(name):
    # Every workload layer whose K is a multiple of 512, at full size: every
    # output element of the automatic plan, and (once per weight set) the
    # whole dense de-quantised matrix bit for bit, with the library's pruning
    # and quantisation equal to the oracle's.
    shp = synth.SHAPES[name]
    ws, X, yref = workload(name, sparse=True)
    packed, s = ws.to_device()
    Y = fp6.sparse_linear(torch.from_numpy(X).to(DEV), packed, s, shp.N, shp.K)
    torch.cuda.synchronize()
    _assert_tol(Y, yref, what=(name, fp6.sparse_plan_query(shp.M, shp.N, shp.K)))
    first = next(n for n in SPARSE_SHAPES if (synth.SHAPES[n].N, synth.SHAPES[n].K, synth.SHAPES[n].seed_w)
                 == (shp.N, shp.K, shp.seed_w))
    if first == name:
        assert ws.codes_match, name
        W16 = fp6.sparse_dequant(packed, s, shp.N, shp.K)
        torch.cuda.synchronize()
        assert np.array_equal(W16.cpu().numpy().view(np.uint16), ws.wdq_ref.view(np.uint16)), name


def test_linear_one_hot_reproduces_wdq_exactly():
    N, K = 64, 2048
    p = SpPrepared(16, N, K, seed_w=81, seed_x=82)
    ks = np.array([0, 1, 2, 3, 4, 63, 64, 100, 511, 512, 700, 1023, 1024, 1500, 2000, 2047])
    X = np.zeros((16, K), np.float16)
    X[np.arange(16), ks] = 1.0
    Xd = torch.from_numpy(X).to(DEV)
    _, packed, s = p.to_device()
    want = p.wdq_ref[:, ks].T.astype(np.float64)
    for variant, splits in [(0, 0), (1, 0), (2, 1), (2, 3), (3, 1), (3, 2), (4, 1), (4, 2), (5, 1), (5, 4),
                            (6, 0), (6, 2), (6, 4), (7, 1), (7, 3), (8, 2), (KRING, 0)]:
        Y = fp6.sparse_linear_plan(Xd, packed, s, N, K, variant=variant, splits=splits)
        torch.cuda.synchronize()
        assert np.array_equal(Y.cpu().numpy().astype(np.float64), want), (variant, splits)


def test_linear_is_deterministic_and_m_zero():
    p = SpPrepared(16, 4096, 4096, seed_w=91, seed_x=92)
    X, packed, s = p.to_device()
    for variant, splits in ((2, 4), (KSPLIT, 4)):
        a = fp6.sparse_linear_plan(X, packed, s, p.N, p.K, variant=variant, splits=splits).clone()
        b = fp6.sparse_linear_plan(X, packed, s, p.N, p.K, variant=variant, splits=splits).clone()
        torch.cuda.synchronize()
        assert torch.equal(a.view(torch.int16), b.view(torch.int16)), (variant, splits)
    Y = fp6.sparse_linear(torch.zeros((0, p.K), dtype=torch.float16, device=DEV), packed, s, p.N, p.K)
    torch.cuda.synchronize()
    assert Y.shape == (0, p.N)


@pytest.mark.parametrize("M", [3, 17])
def test_sparse_linear_adversarial_rows(M):
    # Corner rows for pruning and quantisation: a zero row, a lone outlier,
    # groups with equal magnitudes (ties broken by the lower index), -0
    # codes, saturation and a scale near 16, over ordinary N(0, 0.02) rows.
    N, K = 96, 2560
    rng = np.random.default_rng(500 + M)
    W = (rng.standard_normal((N, K)) * 0.02).astype(np.float32)
    W[0] = 0.0
    W[1] = 1e-6
    W[1, 5] = 1.0
    W[2] = -1e-9
    W[2, 7] = 0.5
    W[3] = np.where(np.arange(K) % 2 == 0, 1.0, -1.0)
    W[4] = np.resize(np.array([0.25, -0.25, 0.25, -0.25, 0.5, 0.5, 0.5, 0.5], np.float32), K)  # all ties
    W[5] = (rng.standard_normal(K) * 10).astype(np.float32)
    W[5, 3] = 400.0
    X = synth.activations(M, K, 600 + M)
    X[:, ::3] = 0
    c, p, s = fp6.prune_quantize(W)
    oc, op, osc = sparse24.quantize_sparse(W)
    assert np.array_equal(c, oc) and np.array_equal(p, op)
    assert np.array_equal(s.view(np.uint16), osc.view(np.uint16))
    wdq = sparse24.dequant_ref(oc, op, osc, K)
    y_ref = oracle.gemm_ref(X, wdq)
    packed = torch.from_numpy(fp6.sparse_prepack(c, p, s, K)).to(DEV)
    sd = torch.from_numpy(s.copy()).to(DEV)
    Xd = torch.from_numpy(X).to(DEV)
    out = fp6.sparse_dequant(packed, sd, N, K)
    torch.cuda.synchronize()
    assert np.array_equal(out.cpu().numpy().view(np.uint16), wdq.view(np.uint16))
    for variant, splits in [(0, 0), (2, 2), (3, 1), (4, 2), (5, 1), (7, 2), (8, 1)] + ([(KSLICE, 0), (KSPLIT, 0), (KSPLIT, 3), (KRING, 0)] if M <= 16 else []):
        Y = fp6.sparse_linear_plan(Xd, packed, sd, N, K, variant=variant, splits=splits)
        torch.cuda.synchronize()
        _assert_tol(Y, y_ref, what=(M, variant, splits))
        assert not Y[:, 0].cpu().numpy().astype(np.float64).any(), (M, variant, splits)


@pytest.mark.parametrize("K, per_wg, M", [(K, w, M) for K in (2048, 4096, 6144) for w in (1, 2, 3, 4, 5, 7, 8)
                                          for M in (1, 5, 16)])
def test_sparse_ksplit_row_blocks_per_workgroup(K, per_wg, M):
    # The sparse k-split kernel with 1-8 row blocks per workgroup (a
    # workgroup with fewer than its form's count repeats its last row
    # block), K split when it exceeds 8 tiles; N is sized from the CU count.
    # Every output element.
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    splits = -(-(K // 512) // 8)
    per_split = cus // splits
    nblocks = (per_wg - 1) * per_split + max(per_split // 3, 1)
    N = 16 * nblocks
    ws = sparse_weight_set(N, K, 950 + per_wg + K)
    X = synth.activations(M, K, 960 + M)
    packed, sd = ws.to_device()
    Y = fp6.sparse_linear_plan(torch.from_numpy(X).to(DEV), packed, sd, N, K, variant=KSPLIT)
    torch.cuda.synchronize()
    _assert_tol(Y, y_ref(X, ws.wdq_ref), what=(M, per_wg, K))


@pytest.mark.parametrize("K, per_wg, M", [(K, w, M) for K, ws in ((512, (1, 3)), (2560, (2,)), (4096, (1, 2, 5, 8)),
                                                                    (8192, (2, 7))) for w in ws for M in (1, 5, 16)])
def test_sparse_kring_row_blocks_per_workgroup(K, per_wg, M):
    # The sparse k-ring kernel: each of 8 waves holds a fixed slice of the
    # sparse tiles with its X resident (K = 512 leaves 7 waves with stand-in
    # tiles, 2560 gives ragged 0/1-tile slices, 8192 two tiles per wave),
    # walks per_wg row blocks (the last workgroup fewer; one tile per wave
    # keeps two row blocks in flight).  Every output element, bitwise
    # reproducible.
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    nblocks = (per_wg - 1) * cus + max(cus // 3, 1) if per_wg > 1 else cus - 5
    N = 16 * nblocks
    ws = sparse_weight_set(N, K, 970 + per_wg + K)
    X = synth.activations(M, K, 980 + M)
    packed, sd = ws.to_device()
    Xd = torch.from_numpy(X).to(DEV)
    Y = fp6.sparse_linear_plan(Xd, packed, sd, N, K, variant=KRING).clone()
    Y2 = fp6.sparse_linear_plan(Xd, packed, sd, N, K, variant=KRING)
    torch.cuda.synchronize()
    _assert_tol(Y, y_ref(X, ws.wdq_ref), what=(M, per_wg, K))
    assert torch.equal(Y.view(torch.int16), Y2.view(torch.int16)), (M, per_wg, K)


def test_sparse_kring_rejects_what_it_does_not_cover():
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    p = SpPrepared(16, 64, 1024, seed_w=25, seed_x=26)
    X, packed, s = p.to_device()
    with pytest.raises(fp6.FP6Error):      # no K-splits
        fp6.sparse_linear_plan(X, packed, s, 64, 1024, variant=KRING, splits=2)
    X17 = torch.zeros((17, 1024), dtype=torch.float16, device=DEV)
    with pytest.raises(fp6.FP6Error):      # M <= 16
        fp6.sparse_linear_plan(X17, packed, s, 64, 1024, variant=KRING)
    Xk = torch.zeros((1, 8704), dtype=torch.float16, device=DEV)
    wk = torch.zeros(fp6.sparse_packed_bytes(64, 8704), dtype=torch.uint8, device=DEV)
    with pytest.raises(fp6.FP6Error):      # K <= 8192
        fp6.sparse_linear_plan(Xk, wk, s, 64, 8704, variant=KRING)
    N = 16 * (8 * cus + 1)                 # 9 row blocks per CU
    big = torch.zeros(fp6.sparse_packed_bytes(N, 512), dtype=torch.uint8, device=DEV)
    sc = torch.zeros(N, dtype=torch.float16, device=DEV)
    X1 = torch.zeros((1, 512), dtype=torch.float16, device=DEV)
    with pytest.raises(fp6.FP6Error):
        fp6.sparse_linear_plan(X1, big, sc, N, 512, variant=KRING)


def test_sparse_kring_one_hot_every_tile_slot():
    # One-hot activations through the sparse k-ring kernel at K = 8192 (two
    # 512-k sparse tiles per wave) with 3 row blocks per workgroup and a
    # short last one: columns in both tile slots of every wave, kept or
    # pruned positions alike, so every output equals a de-quantised weight
    # exactly (zero where the weight was pruned).
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    N, K, M = 16 * (2 * cus + 9), 8192, 16
    ws = sparse_weight_set(N, K, 4444)
    cols = []
    for m in range(M):
        w = (3 * m + 1) % 8
        cols.append((2 * w + m % 2) * 512 + (37 * m + 7) % 512)
    ks = np.array(cols)
    X = np.zeros((M, K), np.float16)
    X[np.arange(M), ks] = 1.0
    Xd = torch.from_numpy(X).to(DEV)
    packed, sd = ws.to_device()
    want = ws.wdq_ref[:, ks].T.astype(np.float64)
    for m_used in (1, 16):
        Y = fp6.sparse_linear_plan(Xd[:m_used].contiguous(), packed, sd, N, K, variant=KRING)
        torch.cuda.synchronize()
        assert np.array_equal(Y.cpu().numpy().astype(np.float64), want[:m_used]), m_used
