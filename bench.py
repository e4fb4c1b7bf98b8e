#!/usr/bin/env python3
"""Benchmark of the fused FP6 (e3m2) weight-only linear layer on one MI355X.

One step = one fused ``fp6_linear`` call (de-quantise + fp16 MFMA GEMM) over
one batch of synthetic activations, with the packed weights already resident
in HBM.  Weight copies are rotated (>= 1 GiB in all) so every call streams
from HBM rather than the 256 MB Infinity Cache.  The timed steps are replayed
from a HIP graph captured from plain library launches on a side stream and
bracketed by torch.cuda.synchronize(); HIP events recorded on that stream give
the average launch duration.

Default workload: the Llama-70B MLP layer with one GPU's full weights, M=16,
N=28672, K=8192 (176 MB of packed FP6 weights, the memory-bound regime).  ``--workload`` selects another shape of
weight_only_fp6_amd.synth.SHAPES and ``--format`` another weight format
(e2m3, e2m2, e2m1 through ``fpx_linear``; default e3m2).  Prints ONE JSON
line.

Also reported, as context:
* ``cpu_baseline``: the plain NumPy oracle timed on this host on a bounded
  sample of the same workload (a baseline, not a target);
* ``fp16_blas``: the same layer as an fp16 torch linear (hipBLASLt) on
  de-quantised weights, with rotated cold copies -- the W16A16 reference the
  FP6-LLM pages normalise their kernel speedups to;
* ``read_ceiling_gbs``: a streaming-read probe (plain and non-temporal loads,
  the best of a few chunk counts) over a buffer of the packed-weight size (the
  practical HBM ceiling at this size);
* ``mfma_ceiling_tflops``: a loop of register-only fp16 MFMAs over the whole
  GPU (the practical dense fp16 MFMA ceiling);
* ``warm_weights``: the same launch with one weight copy reused every time,
  so that the weights stay cache-resident (labelled: not the metric).

``value`` and ``ms_per_step`` come from HIP events recorded on the launch
stream around the K timed steps; a short spin kernel ahead of the first
event covers the host's submission of the timed graph.  ``wall_ms_per_step``
is the host clock between the synchronisations that bracket them (it adds the
spin and the graph launch).

Helper modes for the committed rocprofv3 summaries (see the profile files for
the exact commands): ``--calibrate-copy`` runs a torch copy of a known size so
FETCH_SIZE/WRITE_SIZE can be scaled to bytes; ``--summarize DIR`` turns the
rocprofv3 CSV outputs in DIR into a short text summary.
"""

from __future__ import annotations

import argparse
import csv
import glob
import hashlib
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
METRIC = "W6A16 GEMM TFLOP/s + weight HBM GB/s (% of peak), Llama-shaped layers M=1..128"
DEFAULT_WORKLOAD = "llama70b_mlp_16x28672x8192"
HBM_PEAK_GBS = 8000.0           # MI355X HBM3E, vendor figure
FP16_MFMA_PEAK_TFLOPS = 2500.0  # MI355X dense fp16 MFMA, vendor figure
ROT_BYTES = 1 << 30             # >= 1 GiB of rotated copies (> 256 MB Infinity Cache)
SUBMIT_COVER_CYCLES = 400_000   # spin ahead of the timed region: ~0.17 ms (its counter runs at ~2.4 GHz)
COPY_BYTES = 1 << 30            # --calibrate-copy: bytes read (and written) per copy
CSRC = os.path.join(ROOT, "weight_only_fp6_amd", "csrc")
KERNEL_SRCS = ("fpx_device.h", "fpx_launch.h", "fpx_linear.hip", "fpx_kern_e3m2.hip",
               "fpx_kern_e2m3.hip", "fpx_kern_e2m2.hip", "fpx_kern_e2m1.hip")
FORMAT_BITS = {"e3m2": 6, "e2m3": 6, "e2m2": 5, "e2m1": 4}


# Linear layers of one decoder layer, (name, N, K) with the projections that
# share an input fused along N: Llama-7B (hidden 4096, MLP 11008) and
# Llama-70B (hidden 8192, 8 KV heads of 128, MLP 28672).
DECODERS = {
    "llama7b": [("qkv", 3 * 4096, 4096), ("o", 4096, 4096), ("gate_up", 2 * 11008, 4096),
                ("down", 4096, 11008)],
    "llama70b": [("qkv", 8192 + 2 * 1024, 8192), ("o", 8192, 8192), ("gate_up", 2 * 28672, 8192),
                 ("down", 8192, 28672)],
}


def _parse():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=2000)
    ap.add_argument("--warmup", type=int, default=50)
    ap.add_argument("--workload", default=DEFAULT_WORKLOAD)
    ap.add_argument("--format", default="e3m2", choices=sorted(FORMAT_BITS),
                    help="weight format (e3m2 = FP6 through fp6_linear; others through fpx_linear)")
    ap.add_argument("--sparse", action="store_true",
                    help="2:4-sparse FP6 e3m2 weights through fp6s_linear (K %% 512 == 0)")
    ap.add_argument("--no-graph", action="store_true", help="time direct launches instead of a graph replay")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-context", action="store_true", help="skip the fp16 BLAS and read-probe context numbers")
    ap.add_argument("--variant", type=int, default=0, help="force kernel variant (0 = automatic)")
    ap.add_argument("--splits", type=int, default=0, help="force K-splits (0 = automatic)")
    ap.add_argument("--calibrate-copy", action="store_true", help="run a known-size torch copy and exit")
    ap.add_argument("--summarize", metavar="DIR", help="summarize rocprofv3 CSVs under DIR and exit")
    ap.add_argument("--traffic", nargs=4, metavar=("FETCH_DIR", "WRITE_DIR", "COPY_FETCH_DIR", "COPY_WRITE_DIR"),
                    help="turn four rocprofv3 --pmc runs into a traffic summary for --workload and exit")
    ap.add_argument("--decoder", choices=sorted(DECODERS),
                    help="time one decoder layer's linear chain (FP6 vs fp16 hipBLASLt) at M=1..16 and exit")
    return ap.parse_args()


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    for name in KERNEL_SRCS:
        with open(os.path.join(CSRC, name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def weight_bytes(N, K, fmt="e3m2"):
    if fmt == "sparse24":
        return N * K // 2
    return N * K * FORMAT_BITS[fmt] // 8


def algorithmic_bytes(M, N, K, fmt="e3m2"):
    """Bytes one call must move at least: packed weights, scales, X, Y."""
    return weight_bytes(N, K, fmt) + 2 * N + 2 * M * K + 2 * M * N


# ---------------------------------------------------------------------------
# CPU baseline: the oracle, untuned, on a bounded row sample.
# ---------------------------------------------------------------------------
def cpu_cores():
    """Host cores this process may use, at most 16 (one GPU's share of a multi-GPU host)."""
    return max(1, min(16, len(os.sched_getaffinity(0))))


def cpu_baseline(shape, packed, scales, X, budget_s=20.0, fmt="e3m2"):
    """The oracle as it stands, on every core of this host's share: its
    functions (unpack, de-quantise, float64 GEMM) run unchanged on
    row-block chunks of the sample, one chunk per thread, BLAS limited to one
    thread per call so that the threads in use equal the cores."""
    import oracle
    from concurrent.futures import ThreadPoolExecutor
    from threadpoolctl import threadpool_limits
    cores = cpu_cores()
    M, N, K = shape.M, shape.N, shape.K
    row_bytes = weight_bytes(16, K, fmt)            # one packed row block

    def unpack(buf, n):
        if fmt == "e3m2":
            return oracle.unpack_np(buf, n, K)
        return oracle.unpack_tiles(buf, n, K, fmt)

    def dequant(buf, n, sc):
        if fmt == "sparse24":
            from oracle import sparse24
            codes, pos = sparse24.unpack_tiles(buf, n, K)
            return sparse24.dequant_ref(codes, pos, sc, K)
        return oracle.dequant_ref(unpack(buf, n), sc, fmt)

    def chunk(b0, b1):
        wdq = dequant(packed[b0 * row_bytes: b1 * row_bytes], 16 * (b1 - b0), scales[16 * b0: 16 * b1])
        oracle.gemm_ref(X, wdq)

    with threadpool_limits(limits=1), ThreadPoolExecutor(cores) as ex:
        def run(nblk):
            step = max(1, -(-nblk // cores))
            t0 = time.perf_counter()
            list(ex.map(lambda b: chunk(b, min(nblk, b + step)), range(0, nblk, step)))
            return time.perf_counter() - t0
        # Size one run to about a third of the budget (capped at the whole
        # layer), then repeat it until the budget is spent (at least 3 runs)
        # and report the median.
        nblk = max(cores, min(N // 16, (4 * 2**20) // row_bytes))
        t = run(nblk)
        nblk = int(max(1, min(N // 16, nblk * (budget_s / 3) / max(t, 1e-3))))
        ts = [run(nblk)]
        while len(ts) < 3 or (sum(ts) < budget_s and len(ts) < 101):
            ts.append(run(nblk))
        ts.sort()
        tmed = ts[len(ts) // 2]
    nrows = 16 * nblk
    wbytes = weight_bytes(nrows, K, fmt)
    return {
        "value": round(wbytes / tmed / 1e9, 4),
        "unit": "GB/s",
        "cores": cores,
        "kind": "oracle",
        "sample": f"{nrows} of {N} weight rows x K={K}, M={M}, {fmt}: oracle unpack + dequant_ref + gemm_ref "
                  f"(float64) on row-block chunks over {cores} threads (BLAS 1 thread each), median of "
                  f"{len(ts)} runs of {tmed:.2f} s ({sum(ts):.1f} s in all)",
        "tflops": round(2.0 * M * nrows * K / tmed / 1e12, 6),
    }


# ---------------------------------------------------------------------------
# Traffic from committed counter summaries (only while the kernel source is
# the one the counters were taken with).
# ---------------------------------------------------------------------------
def traffic_name(workload, fmt="e3m2"):
    return f"traffic_{workload}.txt" if fmt == "e3m2" else f"traffic_{workload}_{fmt}.txt"


def committed_traffic(workload, fmt="e3m2"):
    path = os.path.join(ROOT, "profiles", traffic_name(workload, fmt))
    if not os.path.exists(path):
        return None
    vals = {}
    with open(path) as f:
        for line in f:
            if "=" in line and not line.startswith("#"):
                k, v = line.split("=", 1)
                vals[k.strip()] = v.strip()
    if vals.get("kernel_source_sha256_16") != kernel_source_hash():
        return None
    try:
        return {"bytes_per_launch": float(vals["hbm_bytes_per_launch"]),
                "fetch_bytes": float(vals["fetch_bytes_per_launch"]),
                "write_bytes": float(vals["write_bytes_per_launch"])}
    except KeyError:
        return None


def _time_graph(torch, stream, launch, n):
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=stream):
        for i in range(n):
            launch(i)
    g.replay()
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    g.replay()
    e1.record(stream)
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) * 1e3 / n   # microseconds per launch


def fp16_blas_context(torch, fp6, stream, pk, sc, x, M, N, K, fmt="e3m2"):
    """fp16 torch linear (hipBLASLt) on the de-quantised weights, cold copies."""
    if fmt == "sparse24":
        W16 = fp6.sparse_dequant(pk, sc, N, K, stream=stream)
    else:
        W16 = fp6.dequant(pk, sc, N, K, stream=stream, fmt=fmt)
    torch.cuda.synchronize()
    R = int(min(32, max(2, math.ceil(ROT_BYTES / (2 * N * K)))))
    ws = [W16.clone() for _ in range(R)]
    ys = [torch.empty((M, N), dtype=torch.float16, device=x.device) for _ in range(R)]

    def launch(i):
        torch.matmul(x, ws[i % R].t(), out=ys[i % R])
    launch(0)
    torch.cuda.synchronize()
    us = _time_graph(torch, stream, launch, 200)
    del ws, ys, W16
    return us


def read_ceiling(torch, nbytes, stream):
    """Streaming read of a buffer of nbytes, rotated over >= 1 GiB: the best of
    plain and non-temporal loads over a few per-wave chunk counts."""
    import ctypes
    lib = ctypes.CDLL(os.path.join(ROOT, "weight_only_fp6_amd", "libfp6probe.so"))
    lib.fp6probe_read.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_int64, ctypes.c_int,
                                  ctypes.c_void_p, ctypes.c_void_p]
    nbytes = (nbytes // 1024) * 1024
    R = int(min(64, max(2, math.ceil(ROT_BYTES / nbytes))))
    bufs = [torch.empty(nbytes, dtype=torch.uint8, device="cuda") for _ in range(R)]
    out = torch.zeros(4, dtype=torch.int32, device="cuda")
    best = None
    for nt, per_wave in ((1, 8), (1, 16), (0, 8), (0, 32)):
        def launch(i):
            if lib.fp6probe_read(bufs[i % R].data_ptr(), nbytes, per_wave, nt, out.data_ptr(),
                                 stream.cuda_stream):
                raise RuntimeError("probe launch failed")
        launch(0)
        torch.cuda.synchronize()
        us = _time_graph(torch, stream, launch, 100)
        gbs = nbytes / us / 1e3
        best = gbs if best is None else max(best, gbs)
    del bufs
    return best


def mfma_ceiling(torch, stream):
    """Dense fp16 MFMA rate of a register-only MFMA loop over the whole GPU
    (TFLOP/s): 8 workgroups of 4 waves per CU, each wave 8 independent
    16x16x32 MFMA chains."""
    import ctypes
    lib = ctypes.CDLL(os.path.join(ROOT, "weight_only_fp6_amd", "libfp6probe.so"))
    lib.fp6probe_mfma.argtypes = [ctypes.c_int64, ctypes.c_int64, ctypes.c_void_p, ctypes.c_void_p]
    chains = lib.fp6probe_mfma_chains()
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    blocks, iters = 8 * cus, 4096
    out = torch.zeros(4, dtype=torch.float32, device="cuda")

    def launch(i):
        if lib.fp6probe_mfma(iters, blocks, out.data_ptr(), stream.cuda_stream):
            raise RuntimeError("probe launch failed")
    launch(0)
    torch.cuda.synchronize()
    us = _time_graph(torch, stream, launch, 10)
    return blocks * 4 * iters * chains * 16384 / us / 1e6


# ---------------------------------------------------------------------------
# rocprofv3 summaries
# ---------------------------------------------------------------------------
def summarize(directory):
    lines = []
    for path in sorted(glob.glob(os.path.join(directory, "**", "*_kernel_stats.csv"), recursive=True)):
        lines.append(f"# kernel stats: {os.path.relpath(path, directory)}")
        lines.append("name | calls | average_ns | min_ns | max_ns | percent")
        with open(path) as f:
            for r in csv.DictReader(f):
                lines.append(f"{r['Name'][:110]} | {r['Calls']} | {float(r['AverageNs']):.1f} | "
                             f"{r['MinNs']} | {r['MaxNs']} | {float(r['Percentage']):.2f}")
    for path in sorted(glob.glob(os.path.join(directory, "**", "*_counter_collection.csv"), recursive=True)):
        agg = {}
        with open(path) as f:
            for r in csv.DictReader(f):
                key = (r["Kernel_Name"][:110], r["Counter_Name"])
                agg.setdefault(key, []).append(float(r["Counter_Value"]))
        lines.append(f"# counters: {os.path.relpath(path, directory)}")
        lines.append("kernel | counter | dispatches | mean_per_dispatch")
        for (k, c), v in sorted(agg.items()):
            lines.append(f"{k} | {c} | {len(v)} | {sum(v) / len(v):.1f}")
    print("\n".join(lines))


def _pmc_mean(directory, counter, name_filter):
    vals = []
    for path in glob.glob(os.path.join(directory, "**", "*_counter_collection.csv"), recursive=True):
        with open(path) as f:
            for r in csv.DictReader(f):
                if r["Counter_Name"] == counter and name_filter(r["Kernel_Name"]):
                    vals.append(float(r["Counter_Value"]))
    if not vals:
        raise SystemExit(f"no {counter} samples in {directory}")
    return sum(vals) / len(vals), len(vals)


def traffic_summary(workload, fetch_dir, write_dir, copy_fetch_dir, copy_write_dir):
    """FETCH_SIZE/WRITE_SIZE (KiB per dispatch) of the fp6 kernel, scaled by
    what the same counters read for a torch copy of COPY_BYTES."""
    is_fp6 = lambda n: "fp6_gemm" in n
    is_copy = lambda n: "fp6" not in n and ("copy" in n.lower() or "elementwise" in n)
    f_kib, nf = _pmc_mean(fetch_dir, "FETCH_SIZE", is_fp6)
    w_kib, nw = _pmc_mean(write_dir, "WRITE_SIZE", is_fp6)
    cf_kib, _ = _pmc_mean(copy_fetch_dir, "FETCH_SIZE", is_copy)
    cw_kib, _ = _pmc_mean(copy_write_dir, "WRITE_SIZE", is_copy)
    kf = COPY_BYTES / (cf_kib * 1024)
    kw = COPY_BYTES / (cw_kib * 1024)
    fetch = f_kib * 1024 * kf
    write = w_kib * 1024 * kw
    print(f"# HBM traffic of the fp6 kernel for workload {workload}")
    print(f"# FETCH_SIZE {f_kib:.1f} KiB/dispatch over {nf} dispatches, WRITE_SIZE {w_kib:.1f} KiB over {nw};")
    print(f"# a torch copy of {COPY_BYTES} bytes reads FETCH_SIZE {cf_kib:.1f} KiB and WRITE_SIZE {cw_kib:.1f} KiB,")
    print(f"# so the counters are scaled by {kf:.4f} (fetch) and {kw:.4f} (write).")
    print(f"workload = {workload}")
    print(f"kernel_source_sha256_16 = {kernel_source_hash()}")
    print(f"fetch_scale = {kf:.6f}")
    print(f"write_scale = {kw:.6f}")
    print(f"fetch_bytes_per_launch = {fetch:.0f}")
    print(f"write_bytes_per_launch = {write:.0f}")
    print(f"hbm_bytes_per_launch = {fetch + write:.0f}")


def decoder_chain(name, fmt="e3m2"):
    """One decoder layer's four linears at M = 1, 2, 4, 8, 16: the fused path
    vs the same chain in fp16 (hipBLASLt) on the de-quantised weights.  Codes
    are uniform over all codes of the format (timing does not depend on them);
    enough layer copies rotate to keep the weights out of the 256 MB Infinity
    Cache."""
    import torch
    import weight_only_fp6_amd as fp6
    from weight_only_fp6_amd import synth
    layers = DECODERS[name]
    sparse = fmt == "sparse24"
    if sparse and any(k % 512 for _, _, k in layers):
        print(f"{name}: the 2:4-sparse path needs K % 512 == 0 for every layer", file=sys.stderr)
        sys.exit(2)
    dev = torch.device("cuda:0")
    stream = torch.cuda.Stream()
    torch.cuda.set_stream(stream)
    fp6_bytes = sum(weight_bytes(n, k, fmt) for _, n, k in layers)
    ncode = 64 if sparse else 1 << FORMAT_BITS[fmt]
    fid = fp6.FORMATS.get(fmt, 0)
    copies = int(max(1, math.ceil(ROT_BYTES / fp6_bytes)))
    packed, scales, w16 = [], [], []
    for ci in range(copies):
        pc, sc, wc = [], [], []
        for li, (_, n, k) in enumerate(layers):
            s_ = np.full(n, 0.003, dtype=np.float16)
            if sparse:
                codes = synth.codes_uniform(n, k // 2, seed=100 * ci + li)
                pos = np.tile(np.array([0, 2], np.uint8), (n, k // 4))
                pk = torch.from_numpy(fp6.sparse_prepack(codes, pos, s_, k)).to(dev)
            else:
                codes = synth.codes_uniform(n, k, seed=100 * ci + li) % ncode
                pk = torch.from_numpy(fp6.prepack(codes, s_, fmt)).to(dev)
            st = torch.from_numpy(s_).to(dev)
            pc.append(pk)
            sc.append(st)
            if ci == 0:
                wc.append(fp6.sparse_dequant(pk, st, n, k, stream=stream) if sparse else
                          fp6.dequant(pk, st, n, k, stream=stream, fmt=fmt))
        packed.append(pc)
        scales.append(sc)
        if ci == 0:
            w16 = wc
    torch.cuda.synchronize()
    w16_copies = int(max(1, math.ceil(ROT_BYTES / sum(2 * n * k for _, n, k in layers))))
    w16s = [w16] + [[w.clone() for w in w16] for _ in range(w16_copies - 1)]
    rows = []
    for M in (1, 2, 4, 8, 16):
        xs = {k: torch.randn(M, k, device=dev).to(torch.float16) for _, _, k in layers}
        ys = [torch.empty(M, n, dtype=torch.float16, device=dev) for _, n, _ in layers]
        L = fp6.lib

        def fp6_step(i):
            c = i % copies
            for li, (_, n, k) in enumerate(layers):
                args = (xs[k].data_ptr(), packed[c][li].data_ptr(), scales[c][li].data_ptr(),
                        ys[li].data_ptr(), M, n, k, stream.cuda_stream)
                st = L.fp6s_linear(*args) if sparse else L.fpx_linear(fid, *args)
                if st:
                    raise fp6.FP6Error("linear", st)

        def f16_step(i):
            c = i % w16_copies
            for li, (_, n, k) in enumerate(layers):
                torch.matmul(xs[k], w16s[c][li].t(), out=ys[li])
        fp6_step(0)
        f16_step(0)
        torch.cuda.synchronize()
        t6 = _time_graph(torch, stream, fp6_step, 100)
        t16 = _time_graph(torch, stream, f16_step, 100)
        rows.append({"M": M, "fp6_us": round(t6, 2), "fp16_blas_us": round(t16, 2),
                     "speedup": round(t16 / t6, 3),
                     "fp6_weight_gbps": round(fp6_bytes / t6 / 1e3, 1)})
    print(json.dumps({"metric": "decoder-layer linear chain latency (qkv, o, gate_up, down)",
                      "model_shapes": name, "layers": [[a, n, k] for a, n, k in layers],
                      "unit": "us", "fp6_weight_bytes": fp6_bytes, "rows": rows,
                      "format": fmt, "data": f"synthetic (uniform {fmt} codes)"}), flush=True)


def calibrate_copy():
    import torch
    src = torch.empty(COPY_BYTES, dtype=torch.uint8, device="cuda")
    dst = torch.empty(COPY_BYTES, dtype=torch.uint8, device="cuda")
    for _ in range(5):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"calibrate_copy_bytes": COPY_BYTES, "copies": 5}))


def main():
    args = _parse()
    if args.summarize:
        summarize(args.summarize)
        return
    if args.traffic:
        fmt = "sparse24" if args.sparse else args.format
        traffic_summary(args.workload if fmt == "e3m2" else f"{args.workload} ({fmt})", *args.traffic)
        return
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (the library has no multi-GPU path); got --gpus {args.gpus}",
              file=sys.stderr)
        sys.exit(2)
    import torch
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(3)
    if args.calibrate_copy:
        calibrate_copy()
        return
    if args.decoder:
        decoder_chain(args.decoder, "sparse24" if args.sparse else args.format)
        return
    import weight_only_fp6_amd as fp6
    from weight_only_fp6_amd import synth

    if args.workload not in synth.SHAPES:
        print(f"unknown workload {args.workload}; choose from {sorted(synth.SHAPES)}", file=sys.stderr)
        sys.exit(2)
    shape = synth.SHAPES[args.workload]
    M, N, K = shape.M, shape.N, shape.K
    dev = torch.device("cuda:0")

    # ---- inputs: host quantise + prepack, then R rotated device copies ----
    fmt = "sparse24" if args.sparse else args.format
    if args.sparse and args.format != "e3m2":
        print("--sparse uses FP6 e3m2 weights", file=sys.stderr)
        sys.exit(2)
    W = synth.weights(N, K, shape.seed_w)
    if args.sparse:
        codes, pos, scales = fp6.prune_quantize(W)
        packed = fp6.sparse_prepack(codes, pos, scales, K)
        del pos
    else:
        codes, scales = fp6.quantize_rows(W, fmt)
        packed = fp6.prepack(codes, scales, fmt)
    del W
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
    if args.variant:
        variant, splits = args.variant, args.splits
    elif args.sparse:
        variant, splits = fp6.sparse_plan_query(M, N, K)
    else:
        variant, splits = fp6.plan_query(M, N, K)
    fid = fp6.FORMATS.get(fmt, 0)

    def launch(i):
        x, w, s, y = ptrs[i % R]
        if fmt == "sparse24":
            st = L.fp6s_linear_plan(x, w, s, y, M, N, K, args.variant, args.splits, sh)
        elif fmt == "e3m2":
            st = L.fp6_linear_plan(x, w, s, y, M, N, K, args.variant, args.splits, sh)
        else:
            st = L.fpx_linear_plan(fid, x, w, s, y, M, N, K, args.variant, args.splits, sh)
        if st != 0:
            raise fp6.FP6Error("linear_plan", st)

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
    # A short spin kernel ahead of the first event keeps the GPU busy while
    # the host submits the timed graph (35-70 us measured for 20 launches),
    # so that the events bracket the K launches alone; the wall clock
    # includes both.
    torch.cuda._sleep(SUBMIT_COVER_CYCLES)
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
    per_launch_s = ev0.elapsed_time(ev1) / 1e3 / args.steps

    wbytes = weight_bytes(N, K, fmt)
    abytes = algorithmic_bytes(M, N, K, fmt)
    flops = 2.0 * M * N * K
    weight_gbs = wbytes / per_launch_s / 1e9
    tflops = flops / per_launch_s / 1e12
    # Ridge: 2500 TFLOP/s / 8 TB/s = 312.5 flop/byte; per packed weight byte the
    # layer does 2*M*N*K / (bits/8*N*K) = 16*M/bits flop, so FP6 is HBM-bound
    # for M < 117 (FP5 98, FP4 78; 2:4-sparse FP6, 0.5 byte per dense weight,
    # 78 in dense-equivalent flops).
    traffic = committed_traffic(args.workload, fmt) if not args.variant else None
    eff_bits = 4 if fmt == "sparse24" else FORMAT_BITS[fmt]
    if M < 312.5 * eff_bits / 16:
        achieved = abytes / per_launch_s / 1e9
        roofline = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                    "frac": round(achieved / HBM_PEAK_GBS, 4),
                    "traffic": round(traffic["bytes_per_launch"]) if traffic else None}
        value, unit = round(weight_gbs, 1), "GB/s"
    else:
        achieved = flops / per_launch_s / 1e12
        roofline = {"bound": "mfma", "achieved": round(achieved, 1), "peak": FP16_MFMA_PEAK_TFLOPS,
                    "unit": "TFLOP/s", "frac": round(achieved / FP16_MFMA_PEAK_TFLOPS, 4),
                    "traffic": round(traffic["bytes_per_launch"]) if traffic else None}
        value, unit = round(tflops, 2), "TFLOP/s"
    if fmt == "sparse24":
        roofline["kernel"] = fp6.SPARSE_KERNEL_NAMES.get(variant, str(variant))
    else:
        roofline["kernel"] = fp6.KERNEL_NAMES.get(variant, str(variant))
    roofline["splits"] = splits
    roofline["per_launch_us"] = round(per_launch_s * 1e6, 3)
    roofline["algorithmic_bytes"] = abytes
    roofline["flops"] = flops
    roofline["traffic_unit"] = "HBM bytes/launch (rocprofv3 FETCH_SIZE+WRITE_SIZE, copy-calibrated)"

    out = {
        "metric": METRIC,
        "value": value,
        "unit": unit,
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(per_launch_s * 1e3, 6),
        "wall_ms_per_step": round(wall_s * 1e3 / args.steps, 6),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp16",
        "data": "synthetic",
        "config": {"workload": args.workload if fmt == "e3m2" else f"{args.workload}_{fmt}",
                   "M": M, "N": N, "K": K,
                   "weights": ("fp6 e3m2, 2:4 sparse (magnitude-pruned), + fp16 row scale (packed 2:4 layout)"
                               if fmt == "sparse24" else
                               f"fp{FORMAT_BITS[fmt]} {fmt} + fp16 row scale (packed layout v3)"),
                   "activations": "fp16", "accumulate": "fp32",
                   "rotated_weight_copies": R, "graph": not args.no_graph},
        "weight_gbps": round(weight_gbs, 1),
        "weight_hbm_frac": round(weight_gbs / HBM_PEAK_GBS, 4),
        "tflops": round(tflops, 3),
        "mfma_frac": round(tflops / FP16_MFMA_PEAK_TFLOPS, 5),
        "roofline": roofline,
    }
    if not args.no_context:
        blas_us = fp16_blas_context(torch, fp6, stream, pk_d[0], sc_d[0], x_d[0], M, N, K, fmt)
        out["fp16_blas"] = {"kind": "torch.matmul fp16 (hipBLASLt), de-quantised weights, cold copies",
                            "us": round(blas_us, 3),
                            "fp6_speedup": round(blas_us / (per_launch_s * 1e6), 3)}
        ceil_gbs = read_ceiling(torch, wbytes, stream)
        out["read_ceiling_gbs"] = round(ceil_gbs, 1)
        out["weight_frac_of_read_ceiling"] = round(wbytes / per_launch_s / 1e9 / ceil_gbs, 4)
        mfma_tf = mfma_ceiling(torch, stream)
        out["mfma_ceiling_tflops"] = round(mfma_tf, 1)
        out["mfma_frac_of_probe"] = round(tflops / mfma_tf, 5)
        # Not the metric: every launch reads the same weight copy, which then
        # stays in the caches (the 256 MB Infinity Cache holds any layer here).
        warm_us = _time_graph(torch, stream, lambda i: launch(0), 200)
        out["warm_weights"] = {"us": round(warm_us, 3),
                               "note": "one weight copy for every launch (cache-resident); not the metric"}
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(shape, packed, scales, X, fmt=fmt)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
