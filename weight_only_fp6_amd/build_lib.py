"""Build the HIP library ``libfp6amd.so`` in-tree for gfx950.

Host code (fp6_host.cpp) is compiled with g++; the host dispatch and device
entry points (fpx_linear.hip) and the kernels, one translation unit per
weight format (fpx_kern_*.hip, compiled in parallel), with hipcc; all are
linked into one shared library next to this file.  Run
``python weight_only_fp6_amd/build_lib.py`` (by path, so the package -- which
loads the library -- is not imported first).
"""

from __future__ import annotations

import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libfp6amd.so")
PROBE_LIB = os.path.join(PKG, "libfp6probe.so")

ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")
HIPCC = os.path.join(ROCM, "bin", "hipcc")
ARCH = "gfx950"

# Packed-fp32 instruction selection is switched off for every device
# compilation (see the library's design notes on v_pk_*_f32).
HIP_FLAGS = [
    "-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function",
]
HOST_FLAGS = ["-O2", "-std=c++17", "-fPIC", "-Wall", "-Wextra"]


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        sys.stderr.write(res.stdout + res.stderr)
        raise RuntimeError(f"build step failed: {' '.join(cmd[:3])} ...")
    return res


HIP_SOURCES = ["fpx_linear.hip", "fpx_kern_e3m2.hip", "fpx_kern_e2m3.hip", "fpx_kern_e2m2.hip",
               "fpx_kern_e2m1.hip", "fpx_sparse.hip"]


def _run_parallel(cmds, verbose):
    procs = []
    for cmd in cmds:
        if verbose:
            print(" ".join(cmd), flush=True)
        procs.append((cmd, subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)))
    failed = None
    for cmd, p in procs:
        out, _ = p.communicate()
        if p.returncode != 0 and failed is None:
            sys.stderr.write(out)
            failed = cmd
    if failed:
        raise RuntimeError(f"build step failed: {' '.join(failed[:3])} ...")


def build(verbose: bool = False) -> str:
    """Compile and link the library; returns its path.  Always rebuilds."""
    os.makedirs(BUILD, exist_ok=True)
    inc = ["-I", INCLUDE, "-I", CSRC]
    host_o = os.path.join(BUILD, "fp6_host.o")
    objs = [host_o]
    cmds = [["g++", *HOST_FLAGS, *inc, "-c", os.path.join(CSRC, "fp6_host.cpp"), "-o", host_o]]
    for src in HIP_SOURCES:
        obj = os.path.join(BUILD, src.replace(".hip", ".o"))
        objs.append(obj)
        cmds.append([HIPCC, *HIP_FLAGS, *inc, "-c", os.path.join(CSRC, src), "-o", obj])
    _run_parallel(cmds, verbose)
    tmp = LIB + ".tmp"
    _run([HIPCC, "-shared", f"--offload-arch={ARCH}", "-o", tmp, *objs], verbose)
    shutil.move(tmp, LIB)
    # Bandwidth probe used only by the benchmark's roofline measurement.
    probe_tmp = PROBE_LIB + ".tmp"
    _run([HIPCC, *HIP_FLAGS, "-shared", os.path.join(CSRC, "fp6_probe.hip"), "-o", probe_tmp], verbose)
    shutil.move(probe_tmp, PROBE_LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
