"""Shared preparation of seeded workloads for the GPU parity tests.

The HIP path and the oracle start from the same synthetic float32 weights and
fp16 activations (weight_only_fp6_amd.synth) and then go separate ways: the
library quantises and packs with its own C++ code, the oracle with NumPy.
"""

from __future__ import annotations

import numpy as np

import oracle
import weight_only_fp6_amd as fp6
from weight_only_fp6_amd import synth


class Prepared:
    def __init__(self, M, N, K, seed_w, seed_x, sample=None, W=None, X=None, fmt="e3m2"):
        self.M, self.N, self.K, self.fmt = M, N, K, fmt
        self.W = synth.weights(N, K, seed_w) if W is None else W
        self.X = synth.activations(M, K, seed_x) if X is None else X
        # library (device path) inputs
        self.codes, self.scales = fp6.quantize_rows(self.W, fmt)
        self.packed = fp6.prepack(self.codes, self.scales, fmt)
        # oracle on all rows or on a sample of rows
        self.rows = np.arange(N) if sample is None else synth.sample_rows(N, sample, seed_w + 17)
        oc, osc = oracle.quantize_rows(self.W[self.rows], fmt)
        self.ocodes, self.oscales = oc, osc
        self.wdq_ref = oracle.dequant_ref(oc, osc, fmt)         # [len(rows), K] fp16
        self.y_ref = oracle.gemm_ref(self.X, self.wdq_ref)      # [M, len(rows)] f64

    def to_device(self):
        import torch
        dev = torch.device("cuda:0")
        return (torch.from_numpy(self.X).to(dev),
                torch.from_numpy(self.packed).to(dev),
                torch.from_numpy(self.scales.copy()).to(dev))


def prepare_shape(shape: synth.Shape, sample=None, fmt="e3m2") -> Prepared:
    return Prepared(shape.M, shape.N, shape.K, shape.seed_w, shape.seed_x, sample=sample, fmt=fmt)
