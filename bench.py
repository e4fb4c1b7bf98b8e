#!/usr/bin/env python3
"""Benchmark of the fused FP6 (e3m2) weight-only linear layer on one MI355X.

One step = one fused ``fp6_linear`` call (de-quantise + fp16 MFMA GEMM) over
one batch of synthetic activations, with the packed weights already resident
in HBM.  Weight copies are rotated so every call streams from HBM rather than
the 256 MB Infinity Cache.  The timed steps are replayed from a HIP graph
(captured from plain library launches on torch's current stream), bracketed
by torch.cuda.synchronize(); HIP events on the same stream give the average
launch duration.

Default workload: the Llama-7B attention projection, M=1 (decode GEMV),
N=4096, K=4096.  ``--workload`` selects another shape of
weight_only_fp6_amd.synth.SHAPES.

Prints ONE JSON line.  The CPU baseline is the plain oracle (NumPy), timed on
this host on a bounded sample of the same workload.
"""

from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

import numpy as np

METRIC = "W6A16 GEMM TFLOP/s + weight HBM GB/s (% of peak), Llama-shaped layers M=1..128"
DEFAULT_WORKLOAD = "llama7b_attn_1x4096x4096"
HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, vendor figure
FP16_MFMA_PEAK_TFLOPS = 2500.0  # MI355X dense fp16 MFMA, vendor figure
ROT_BYTES = 1 << 30            # >= 1 GiB of rotated weight copies (> 256 MB MALL)


def _parse():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=2000)
    ap.add_argument("--warmup", type=int, default=50)
    ap.add_argument("--workload", default=DEFAULT_WORKLOAD)
    ap.add_argument("--no-graph", action="store_true", help="time direct launches instead of a graph replay")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--variant", type=int, default=0, help="force kernel variant (0 = auto)")
    ap.add_argument("--splits", type=int, default=0, help="force K-splits (0 = auto)")
    return ap.parse_args()


def algorithmic_bytes(M, N, K):
    """Bytes one call must move at least: packed weights, scales, X, Y."""
    return N * K * 3 // 4 + 2 * N + 2 * M * K + 2 * M * N


def cpu_baseline(shape, packed, scales, X, budget_s=20.0):
    """Time the oracle (unpack + dequant + fp64 GEMM) on a bounded row sample."""
    import oracle
    from threadpoolctl import threadpool_limits
    with threadpool_limits(limits=1):
        return _cpu_baseline(oracle, shape, packed, scales, X, budget_s)


def _cpu_baseline(oracle, shape, packed, scales, X, budget_s):
    M, N, K = shape.M, shape.N, shape.K
    # rows in multiples of 16 (one packed row block = 16 rows x K)
    row_bytes = 16 * K * 3 // 4
    rows16 = max(1, min(N // 16, (16 * 2**20) // row_bytes))   # start with <= ~16 MB
    def run(nblk):
        nrows = 16 * nblk
        part = packed[: nblk * row_bytes]
        t0 = time.perf_counter()
        codes = oracle.unpack_np(part, nrows, K)
        wdq = oracle.dequant_ref(codes, scales[:nrows])
        oracle.gemm_ref(X, wdq)
        return time.perf_counter() - t0
    t = run(rows16)
    # grow or shrink the sample to about budget_s / 3 per run, then median of 3
    target = budget_s / 3
    scale = target / max(t, 1e-3)
    rows16 = int(max(1, min(N // 16, rows16 * scale)))
    ts = sorted(run(rows16) for _ in range(3))
    tmed = ts[1]
    nrows = 16 * rows16
    wbytes = nrows * K * 3 // 4
    return {
        "value": round(wbytes / tmed / 1e9, 4),
        "unit": "GB/s",
        "cores": 1,
        "kind": "oracle",
        "sample": f"{nrows} of {N} weight rows x K={K}, M={M}: unpack_np + dequant_ref + gemm_ref, "
                  f"median of 3 runs ({tmed:.2f} s each), BLAS limited to 1 thread",
        "tflops": round(2.0 * M * nrows * K / tmed / 1e12, 6),
    }


def main():
    args = _parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (this build has no multi-GPU path); got --gpus {args.gpus}",
              file=sys.stderr)
        sys.exit(2)
    import torch
    import weight_only_fp6_amd as fp6
    from weight_only_fp6_amd import synth

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(3)
    if args.workload not in synth.SHAPES:
        print(f"unknown workload {args.workload}; choose from {sorted(synth.SHAPES)}", file=sys.stderr)
        sys.exit(2)
    shape = synth.SHAPES[args.workload]
    M, N, K = shape.M, shape.N, shape.K
    dev = torch.device("cuda:0")

    # ---- inputs (host quantise + prepack, then upload R rotated copies) ----
    W = synth.weights(N, K, shape.seed_w)
    codes, scales = fp6.quantize_rows(W)
    del W
    packed = fp6.prepack(codes, scales)
    del codes
    X = synth.activations(M, K, shape.seed_x)
    R = int(min(64, max(2, math.ceil(ROT_BYTES / packed.nbytes))))
    pk_d = [torch.from_numpy(packed).to(dev) for _ in range(R)]
    sc_d = [torch.from_numpy(scales.copy()).to(dev) for _ in range(R)]
    x_d = [torch.from_numpy(X).to(dev) for _ in range(R)]
    y_d = [torch.empty((M, N), dtype=torch.float16, device=dev) for _ in range(R)]
    ptrs = [(x_d[i].data_ptr(), pk_d[i].data_ptr(), sc_d[i].data_ptr(), y_d[i].data_ptr()) for i in range(R)]
    L = fp6.lib
    # All work runs on one side stream (graph capture needs a non-default one).
    stream = torch.cuda.Stream()
    stream.wait_stream(torch.cuda.current_stream())
    torch.cuda.set_stream(stream)
    sh = stream.cuda_stream

    def launch(i):
        x, w, s, y = ptrs[i % R]
        st = L.fp6_linear_plan(x, w, s, y, M, N, K, args.variant, args.splits, sh)
        if st != 0:
            raise fp6.FP6Error("fp6_linear_plan", st)

    launch(0)                       # allocates the split-K workspace if the plan needs one
    torch.cuda.synchronize()

    def make_graph(n, offset):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=stream):
            for i in range(n):
                launch(offset + i)
        return g

    if args.no_graph:
        for i in range(args.warmup):
            launch(i)
    else:
        if args.warmup > 0:
            gw = make_graph(args.warmup, 0)
        gt = make_graph(args.steps, args.warmup)
        if args.warmup > 0:
            gw.replay()
    torch.cuda.synchronize()

    ev0 = torch.cuda.Event(enable_timing=True)
    ev1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    ev0.record(stream)
    if args.no_graph:
        for i in range(args.steps):
            launch(args.warmup + i)
    else:
        gt.replay()
    ev1.record(stream)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    wall_s = t1 - t0
    ev_ms = ev0.elapsed_time(ev1)
    per_launch_s = ev_ms / 1e3 / args.steps

    wbytes = N * K * 3 // 4
    abytes = algorithmic_bytes(M, N, K)
    flops = 2.0 * M * N * K
    weight_gbs = wbytes * args.steps / wall_s / 1e9
    tflops = flops * args.steps / wall_s / 1e12
    # Ridge: 2500 TFLOP/s / 8 TB/s = 312.5 flop/byte; per packed weight byte the
    # layer does 2*M*N*K / (0.75*N*K) = 2.67*M flop, so M < 117 is HBM-bound.
    hbm_bound = M < 117
    if hbm_bound:
        achieved = abytes / per_launch_s / 1e9
        roofline = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                    "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": None}
        value, unit = round(weight_gbs, 1), "GB/s"
    else:
        achieved = flops / per_launch_s / 1e12
        roofline = {"bound": "mfma", "achieved": round(achieved, 1), "peak": FP16_MFMA_PEAK_TFLOPS,
                    "unit": "TFLOP/s", "frac": round(achieved / FP16_MFMA_PEAK_TFLOPS, 4), "traffic": None}
        value, unit = round(tflops, 2), "TFLOP/s"
    roofline["kernel"] = "fp6_gemm_stream"
    roofline["per_launch_us"] = round(per_launch_s * 1e6, 3)
    roofline["algorithmic_bytes"] = abytes
    roofline["flops"] = flops

    out = {
        "metric": METRIC,
        "value": value,
        "unit": unit,
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(wall_s * 1e3 / args.steps, 6),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp16",
        "data": "synthetic",
        "config": {"workload": args.workload, "M": M, "N": N, "K": K,
                   "weights": "fp6 e3m2 + fp16 row scale (packed layout v1)",
                   "activations": "fp16", "accumulate": "fp32",
                   "rotated_weight_copies": R, "graph": not args.no_graph,
                   "variant": args.variant, "splits": args.splits},
        "weight_gbps": round(weight_gbs, 1),
        "weight_hbm_frac": round(weight_gbs / HBM_PEAK_GBS, 4),
        "tflops": round(tflops, 3),
        "mfma_frac": round(tflops / FP16_MFMA_PEAK_TFLOPS, 5),
        "roofline": roofline,
    }
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(shape, packed, scales, X)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
