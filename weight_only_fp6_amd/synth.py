"""Seeded synthetic inputs shared by the tests and the benchmark.

Only random numbers and shapes live here -- none of the FP6 arithmetic -- so
both the HIP path and the CPU oracle can draw identical inputs from it.

Workloads stand in for the linear layers of Llama and OPT models (FP6-LLM
pages: kernel benchmarks on linear layers of Llama and OPT models of various
sizes); no trained weights are used.  Weights are N(0, 0.02) float32, the
activations N(0, 1) fp16; quantisation to e3m2 codes with one fp16 scale per
row happens downstream (library quantiser on the GPU path, oracle quantiser on
the reference path).
"""

from __future__ import annotations

from dataclasses import dataclass

import numpy as np


@dataclass(frozen=True)
class Shape:
    name: str
    M: int
    N: int
    K: int
    cfg: int  # workload index used for seeding

    @property
    def seed_w(self) -> int:
        return 1000 * self.cfg + 1

    @property
    def seed_x(self) -> int:
        return 1000 * self.cfg + 2 + self.M


# The five workload families (M, N, K): the smallest layer, a Llama-7B
# attention projection (decode GEMV), a Llama-7B MLP up/down pair, a Llama-70B
# MLP layer with one GPU's full weights, and an OPT-30B QKV projection.
SHAPES = {
    "small_8x1024x1024": Shape("small_8x1024x1024", 8, 1024, 1024, 1),
    "llama7b_attn_1x4096x4096": Shape("llama7b_attn_1x4096x4096", 1, 4096, 4096, 2),
    "llama7b_mlp_up_16x11008x4096": Shape("llama7b_mlp_up_16x11008x4096", 16, 11008, 4096, 3),
    "llama7b_mlp_down_16x4096x11008": Shape("llama7b_mlp_down_16x4096x11008", 16, 4096, 11008, 31),
    "llama70b_mlp_1x28672x8192": Shape("llama70b_mlp_1x28672x8192", 1, 28672, 8192, 4),
    "llama70b_mlp_4x28672x8192": Shape("llama70b_mlp_4x28672x8192", 4, 28672, 8192, 4),
    "llama70b_mlp_16x28672x8192": Shape("llama70b_mlp_16x28672x8192", 16, 28672, 8192, 4),
    "opt30b_qkv_64x21504x7168": Shape("opt30b_qkv_64x21504x7168", 64, 21504, 7168, 5),
    "opt30b_qkv_128x21504x7168": Shape("opt30b_qkv_128x21504x7168", 128, 21504, 7168, 5),
    "opt30b_qkv_256x21504x7168": Shape("opt30b_qkv_256x21504x7168", 256, 21504, 7168, 5),
}


def weights(N: int, K: int, seed: int, chunk_rows: int = 4096) -> np.ndarray:
    """float32 [N,K] ~ N(0, 0.02), generated in row chunks (bounded memory)."""
    rng = np.random.Generator(np.random.PCG64(seed))
    out = np.empty((N, K), dtype=np.float32)
    for r0 in range(0, N, chunk_rows):
        r1 = min(N, r0 + chunk_rows)
        rng.standard_normal((r1 - r0, K), dtype=np.float32, out=out[r0:r1])
    out *= np.float32(0.02)
    return out


def activations(M: int, K: int, seed: int) -> np.ndarray:
    """fp16 [M,K] ~ N(0, 1)."""
    rng = np.random.Generator(np.random.PCG64(seed))
    return rng.standard_normal((M, K), dtype=np.float32).astype(np.float16)


def codes_uniform(N: int, K: int, seed: int, bits: int = 6) -> np.ndarray:
    """uint8 [N,K] uniform over all 2^bits codes (adversarial coverage)."""
    rng = np.random.Generator(np.random.PCG64(seed))
    return rng.integers(0, 1 << bits, (N, K), dtype=np.uint8)


def row_scales(N: int, seed: int, lo: float = 0.002, hi: float = 0.004) -> np.ndarray:
    """fp16 [N] drawn uniformly from [lo, hi) (the range that max|row|/28
    takes for N(0, 0.02) rows of a few thousand weights)."""
    rng = np.random.Generator(np.random.PCG64(seed))
    return rng.uniform(lo, hi, N).astype(np.float16)


def positions_2of4(N: int, K: int, seed: int) -> np.ndarray:
    """uint8 [N, K/2]: for every group of 4 along k, two distinct positions
    (0..3) in ascending order, each of the 6 pairs equally likely."""
    pairs = np.array([(a, b) for a in range(4) for b in range(a + 1, 4)], np.uint8)
    rng = np.random.Generator(np.random.PCG64(seed))
    return pairs[rng.integers(0, 6, (N, K // 4))].reshape(N, K // 2)


def sample_rows(N: int, count: int, seed: int) -> np.ndarray:
    """Sorted distinct row indices, always including the first and last row."""
    rng = np.random.Generator(np.random.PCG64(seed))
    count = min(count, N)
    rows = set(rng.choice(N, size=max(count - 2, 0), replace=False).tolist())
    rows.update({0, N - 1})
    return np.array(sorted(rows), dtype=np.int64)
