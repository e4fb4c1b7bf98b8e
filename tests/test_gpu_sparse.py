"""GPU parity of the 2:4-sparse FP6 path (fp6s_*) against the CPU oracle
(oracle/sparse24.py), needs an MI355X.

* De-quantisation export: dense Wdq (zeros at pruned positions) bit-exact.
* Fused sparse linear: |Y - Y_ref| <= 2e-3 (|Y_ref| + rms) per element and
  relative Frobenius <= 5e-4, every kernel configuration on small ragged
  shapes, the automatic plan at the workload shapes whose K is a multiple of
  512 (sampled output columns for the large layers); one-hot activations
  reproduce Wdq exactly.
"""

import functools

import numpy as np
import pytest

import oracle
from oracle import sparse24
from weight_only_fp6_amd import synth

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():  # pragma: no cover - CPU container
    pytest.skip("no GPU", allow_module_level=True)

import weight_only_fp6_amd as fp6  # noqa: E402

DEV = torch.device("cuda:0")
VARIANTS = (0, 2, 3, 4, 5, 7, 8)     # any M; 1 (k-slice) and 6 (k-split) only for M <= 16
KSLICE = 1
KSPLIT = 6


class SpPrepared:
    def __init__(self, M, N, K, seed_w, seed_x, sample=None):
        self.M, self.N, self.K = M, N, K
        W = synth.weights(N, K, seed_w)
        self.X = synth.activations(M, K, seed_x)
        c, p, s = fp6.prune_quantize(W)
        self.scales = s
        self.packed = fp6.sparse_prepack(c, p, s, K)
        self.rows = np.arange(N) if sample is None else synth.sample_rows(N, sample, seed_w + 17)
        oc, op, osc = sparse24.quantize_sparse(W[self.rows])
        self.wdq_ref = sparse24.dequant_ref(oc, op, osc, K)
        self.y_ref = oracle.gemm_ref(self.X, self.wdq_ref)

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
    for variant in VARIANTS + ((KSLICE, KSPLIT) if M <= 16 else ()):
        Y = fp6.sparse_linear_plan(X, packed, s, N, K, variant=variant)
        torch.cuda.synchronize()
        _assert_tol(Y, p.y_ref, what=(M, N, K, variant))


def test_linear_forced_splits():
    p = SpPrepared(16, 4096, 8192, seed_w=71, seed_x=72, sample=256)
    X, packed, s = p.to_device()
    cols = torch.from_numpy(p.rows).to(DEV)
    for variant in (2, 3, 4, 5, 7, 8):
        for splits in (1, 2, 3, 5, 16):
            Y = fp6.sparse_linear_plan(X, packed, s, p.N, p.K, variant=variant, splits=splits)
            torch.cuda.synchronize()
            _assert_tol(Y[:, cols], p.y_ref, what=(variant, splits))
    for splits in (2, 3, 5):    # k-split: <= 8 tiles per split, <= 8 row blocks per workgroup
        Y = fp6.sparse_linear_plan(X, packed, s, p.N, p.K, variant=KSPLIT, splits=splits)
        torch.cuda.synchronize()
        _assert_tol(Y[:, cols], p.y_ref, what=(KSPLIT, splits))


@functools.lru_cache(maxsize=1)
def _prep(name, sample):
    shp = synth.SHAPES[name]
    return SpPrepared(shp.M, shp.N, shp.K, shp.seed_w, shp.seed_x, sample=sample)


@pytest.mark.parametrize("name", ["llama7b_attn_1x4096x4096", "llama7b_mlp_up_16x11008x4096",
                                  "llama70b_mlp_1x28672x8192", "llama70b_mlp_16x28672x8192",
                                  "opt30b_qkv_64x21504x7168", "opt30b_qkv_128x21504x7168",
                                  "opt30b_qkv_256x21504x7168"])
def test_linear_workloads(name):
    shp = synth.SHAPES[name]
    sample = None if shp.N * shp.K <= 48 * 2**20 else 384
    p = _prep(name, sample)
    X, packed, s = p.to_device()
    Y = fp6.sparse_linear(X, packed, s, shp.N, shp.K)
    torch.cuda.synchronize()
    _assert_tol(Y[:, torch.from_numpy(p.rows).to(DEV)], p.y_ref, what=name)


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
                            (6, 0), (6, 2), (6, 4), (7, 1), (7, 3), (8, 2)]:
        Y = fp6.sparse_linear_plan(Xd, packed, s, N, K, variant=variant, splits=splits)
        torch.cuda.synchronize()
        assert np.array_equal(Y.cpu().numpy().astype(np.float64), want), (variant, splits)


def test_linear_is_deterministic_and_m_zero():
    p = SpPrepared(16, 4096, 4096, seed_w=91, seed_x=92, sample=32)
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
    for variant, splits in [(0, 0), (2, 2), (3, 1), (4, 2), (5, 1), (7, 2), (8, 1)] + ([(KSLICE, 0), (KSPLIT, 0), (KSPLIT, 3)] if M <= 16 else []):
        Y = fp6.sparse_linear_plan(Xd, packed, sd, N, K, variant=variant, splits=splits)
        torch.cuda.synchronize()
        _assert_tol(Y, y_ref, what=(M, variant, splits))
        assert not Y[:, 0].cpu().numpy().astype(np.float64).any(), (M, variant, splits)


@pytest.mark.parametrize("K", [2048, 4096, 6144])
@pytest.mark.parametrize("per_wg", [1, 2, 3, 4, 5, 7, 8])
@pytest.mark.parametrize("M", [1, 5, 16])
def test_sparse_ksplit_row_blocks_per_workgroup(M, per_wg, K):
    # The sparse k-split kernel with 1-8 row blocks per workgroup (a
    # workgroup with fewer than its form's count repeats its last row
    # block), K split when it exceeds 8 tiles; N is sized from the CU count
    # and one row of every row block is checked.
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    splits = -(-(K // 512) // 8)
    per_split = cus // splits
    nblocks = (per_wg - 1) * per_split + max(per_split // 3, 1)
    N = 16 * nblocks
    W = synth.weights(N, K, 950 + per_wg + K)
    X = synth.activations(M, K, 960 + M)
    c, pos, sc = fp6.prune_quantize(W)
    packed = torch.from_numpy(fp6.sparse_prepack(c, pos, sc, K)).to(DEV)
    rows = 16 * np.arange(nblocks) + (np.arange(nblocks) * 5) % 16
    oc, op, osc = sparse24.quantize_sparse(W[rows])
    y_ref = oracle.gemm_ref(X, sparse24.dequant_ref(oc, op, osc, K))
    Y = fp6.sparse_linear_plan(torch.from_numpy(X).to(DEV), packed, torch.from_numpy(sc.copy()).to(DEV),
                               N, K, variant=KSPLIT)
    torch.cuda.synchronize()
    _assert_tol(Y[:, torch.from_numpy(rows).to(DEV)], y_ref, what=(M, per_wg, K))
