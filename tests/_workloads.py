"""Shared preparation of seeded workloads for the GPU parity tests.

The HIP path and the oracle start from the same synthetic float32 weights and
fp16 activations (weight_only_fp6_amd.synth) and then go separate ways: the
library quantises and packs with its own C++ code, the oracle with NumPy.

Full-size layers (up to 57344 x 8192 weights) are compared element by
element.  To keep that affordable the unchanged oracle functions are called on
row chunks from a thread pool (quantisation, pruning and de-quantisation are
defined row by row, and NumPy releases the GIL inside them), and the results
of one weight set are cached so that the M values of a layer share them.
"""

from __future__ import annotations

import functools
import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np

import oracle
from oracle import sparse24
import weight_only_fp6_amd as fp6
from weight_only_fp6_amd import synth

# Worker threads: the cores this process may use, at most 16.
THREADS = max(1, min(16, len(os.sched_getaffinity(0))))
ROW_CHUNK = 1024


def _row_chunks(N: int, chunk: int = ROW_CHUNK):
    return [(r0, min(N, r0 + chunk)) for r0 in range(0, N, chunk)]


def run_rows(N: int, fn) -> None:
    """fn(r0, r1) over row chunks of [0, N) on the thread pool."""
    chunks = _row_chunks(N)
    if len(chunks) == 1:
        fn(*chunks[0])
        return
    with ThreadPoolExecutor(THREADS) as ex:
        for _ in ex.map(lambda c: fn(*c), chunks):
            pass


@functools.lru_cache(maxsize=1)
def synth_weights(N: int, K: int, seed: int) -> np.ndarray:
    W = synth.weights(N, K, seed)
    W.setflags(write=False)
    return W


# ---------------------------------------------------------------------------
# Library side (host C++ through the binding) and oracle side, by row chunks.
# ---------------------------------------------------------------------------
def lib_quantize(W: np.ndarray, fmt: str):
    N, K = W.shape
    codes = np.empty((N, K), np.uint8)
    scales = np.empty(N, np.float16)

    def work(r0, r1):
        c, s = fp6.quantize_rows(W[r0:r1], fmt)
        codes[r0:r1] = c
        scales[r0:r1] = s

    run_rows(N, work)
    return codes, scales


def oracle_quantize_dequant(W: np.ndarray, fmt: str):
    """Oracle codes, scales and Wdq of every row (oracle.quantize_rows and
    oracle.dequant_ref applied to row chunks)."""
    N, K = W.shape
    codes = np.empty((N, K), np.uint8)
    scales = np.empty(N, np.float16)
    wdq = np.empty((N, K), np.float16)

    def work(r0, r1):
        c, s = oracle.quantize_rows(W[r0:r1], fmt)
        codes[r0:r1] = c
        scales[r0:r1] = s
        wdq[r0:r1] = oracle.dequant_ref(c, s, fmt)

    run_rows(N, work)
    return codes, scales, wdq


def oracle_dequant(codes: np.ndarray, scales: np.ndarray, fmt: str) -> np.ndarray:
    N, K = codes.shape
    wdq = np.empty((N, K), np.float16)

    def work(r0, r1):
        wdq[r0:r1] = oracle.dequant_ref(codes[r0:r1], scales[r0:r1], fmt)

    run_rows(N, work)
    return wdq


def oracle_sparse_dequant(codes, pos, scales, K: int) -> np.ndarray:
    N = codes.shape[0]
    wdq = np.empty((N, K), np.float16)

    def work(r0, r1):
        wdq[r0:r1] = sparse24.dequant_ref(codes[r0:r1], pos[r0:r1], scales[r0:r1], K)

    run_rows(N, work)
    return wdq


def y_ref(X: np.ndarray, wdq: np.ndarray, chunk: int = 4096) -> np.ndarray:
    """oracle.gemm_ref over column chunks of Y (bounded float64 temporaries)."""
    M, N = X.shape[0], wdq.shape[0]
    out = np.empty((M, N), np.float64)
    for c0 in range(0, N, chunk):
        c1 = min(N, c0 + chunk)
        out[:, c0:c1] = oracle.gemm_ref(X, wdq[c0:c1])
    return out


# ---------------------------------------------------------------------------
# Whole weight sets, cached (the M values of one layer share them).
# ---------------------------------------------------------------------------
class WeightSet:
    """Library-packed weights and the oracle's de-quantised weights of one
    layer.  ``codes_match`` / ``scales_match``: the library quantiser agrees
    with the oracle bit for bit on every row."""

    def __init__(self, N, K, packed, scales, wdq_ref, codes_match=True, scales_match=True, fmt="e3m2",
                 sparse=False):
        self.N, self.K, self.fmt, self.sparse = N, K, fmt, sparse
        self.packed, self.scales, self.wdq_ref = packed, scales, wdq_ref
        self.codes_match, self.scales_match = codes_match, scales_match

    def to_device(self):
        import torch
        dev = torch.device("cuda:0")
        return torch.from_numpy(self.packed).to(dev), torch.from_numpy(self.scales.copy()).to(dev)


def dense_weight_set(N: int, K: int, seed_w: int, fmt: str = "e3m2") -> WeightSet:
    """Synthetic N(0, 0.02) weights quantised by the library and by the oracle."""
    return _dense_weight_set(int(N), int(K), int(seed_w), fmt)


@functools.lru_cache(maxsize=8)
def _dense_weight_set(N, K, seed_w, fmt):
    W = synth_weights(N, K, seed_w)
    codes, scales = lib_quantize(W, fmt)
    packed = fp6.prepack(codes, scales, fmt)
    ocodes, oscales, wdq = oracle_quantize_dequant(W, fmt)
    return WeightSet(N, K, packed, scales, wdq, np.array_equal(codes, ocodes),
                     np.array_equal(scales.view(np.uint16), oscales.view(np.uint16)), fmt)


def sparse_weight_set(N: int, K: int, seed_w: int) -> WeightSet:
    """Synthetic weights 2:4-pruned and quantised by the library and by the oracle."""
    return _sparse_weight_set(int(N), int(K), int(seed_w))


@functools.lru_cache(maxsize=4)
def _sparse_weight_set(N, K, seed_w):
    W = synth_weights(N, K, seed_w)
    codes = np.empty((N, K // 2), np.uint8)
    pos = np.empty((N, K // 2), np.uint8)
    scales = np.empty(N, np.float16)
    wdq = np.empty((N, K), np.float16)
    match = np.ones(len(_row_chunks(N)), bool)

    def work(r0, r1):
        c, p, s = fp6.prune_quantize(W[r0:r1])
        codes[r0:r1], pos[r0:r1], scales[r0:r1] = c, p, s
        oc, op, osc = sparse24.quantize_sparse(W[r0:r1])
        wdq[r0:r1] = sparse24.dequant_ref(oc, op, osc, K)
        match[r0 // ROW_CHUNK] = (np.array_equal(c, oc) and np.array_equal(p, op)
                                  and np.array_equal(s.view(np.uint16), osc.view(np.uint16)))

    run_rows(N, work)
    packed = fp6.sparse_prepack(codes, pos, scales, K)
    return WeightSet(N, K, packed, scales, wdq, bool(match.all()), bool(match.all()), "e3m2", sparse=True)


def uniform_code_weight_set(N: int, K: int, seed: int, fmt: str = "e3m2", sparse: bool = False) -> WeightSet:
    """Every code equally likely and random row scales (no quantiser): the
    oracle de-quantises the same codes the library packs."""
    return _uniform_code_weight_set(int(N), int(K), int(seed), fmt, bool(sparse))


@functools.lru_cache(maxsize=1)
def _uniform_code_weight_set(N, K, seed, fmt, sparse):
    scales = synth.row_scales(N, seed + 1)
    if sparse:
        codes = synth.codes_uniform(N, K // 2, seed, bits=6)
        pos = synth.positions_2of4(N, K, seed + 2)
        packed = fp6.sparse_prepack(codes, pos, scales, K)
        wdq = oracle_sparse_dequant(codes, pos, scales, K)
    else:
        codes = synth.codes_uniform(N, K, seed, bits=fp6.bits(fmt))
        packed = fp6.prepack(codes, scales, fmt)
        wdq = oracle_dequant(codes, scales, fmt)
    return WeightSet(N, K, packed, scales, wdq, fmt=fmt, sparse=sparse)


def workload(name: str, fmt: str = "e3m2", sparse: bool = False):
    """(weight set, X, Y_ref over the whole output) of a synth.SHAPES entry."""
    shp = synth.SHAPES[name]
    if sparse:
        ws = sparse_weight_set(shp.N, shp.K, shp.seed_w)
    else:
        ws = dense_weight_set(shp.N, shp.K, shp.seed_w, fmt)
    X = synth.activations(shp.M, shp.K, shp.seed_x)
    return ws, X, y_ref(X, ws.wdq_ref)


# ---------------------------------------------------------------------------
# Small layers prepared in one go (optionally on a sample of output rows).
# ---------------------------------------------------------------------------
class Prepared:
    def __init__(self, M, N, K, seed_w, seed_x, sample=None, W=None, X=None, fmt="e3m2"):
        self.M, self.N, self.K, self.fmt = M, N, K, fmt
        self.W = synth.weights(N, K, seed_w) if W is None else W
        self.X = synth.activations(M, K, seed_x) if X is None else X
        # library (device path) inputs
        self.codes, self.scales = lib_quantize(self.W, fmt)
        self.packed = fp6.prepack(self.codes, self.scales, fmt)
        # oracle on all rows or on a sample of rows
        self.rows = np.arange(N) if sample is None else synth.sample_rows(N, sample, seed_w + 17)
        Wr = self.W if sample is None else np.ascontiguousarray(self.W[self.rows])
        self.ocodes, self.oscales, self.wdq_ref = oracle_quantize_dequant(Wr, fmt)
        self.y_ref = y_ref(self.X, self.wdq_ref)                # [M, len(rows)] f64

    def to_device(self):
        import torch
        dev = torch.device("cuda:0")
        return (torch.from_numpy(self.X).to(dev),
                torch.from_numpy(self.packed).to(dev),
                torch.from_numpy(self.scales.copy()).to(dev))


def prepare_shape(shape: synth.Shape, sample=None, fmt="e3m2") -> Prepared:
    return Prepared(shape.M, shape.N, shape.K, shape.seed_w, shape.seed_x, sample=sample, fmt=fmt)
