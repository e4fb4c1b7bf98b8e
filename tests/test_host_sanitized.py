"""The host half of the library (quantiser, packers of every format, 2:4
pruning, size rules, every host-side argument error) built with
AddressSanitizer and UndefinedBehaviorSanitizer and run on the CPU.

tests/host_sanitize/driver.cpp is compiled with fp6_host.cpp by g++ (no HIP
code involved); its outputs must equal the normal library build's bit for bit
and the oracle's codes and scales, and the sanitizers must report nothing.
"""

import os
import shutil
import subprocess

import numpy as np
import pytest

import oracle
from oracle import sparse24
import weight_only_fp6_amd as fp6
from weight_only_fp6_amd import synth

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "weight_only_fp6_amd", "csrc")
DRIVER = os.path.join(ROOT, "tests", "host_sanitize", "driver.cpp")
ENV = dict(os.environ,
           ASAN_OPTIONS="detect_leaks=1:abort_on_error=0:halt_on_error=1:verify_asan_link_order=0",
           UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
ENV.pop("LD_PRELOAD", None)


@pytest.fixture(scope="module")
def driver(tmp_path_factory):
    if shutil.which("g++") is None:
        pytest.skip("g++ not available")
    out = str(tmp_path_factory.mktemp("asan") / "driver")
    cmd = ["g++", "-std=c++17", "-O1", "-g", "-fno-omit-frame-pointer",
           "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
           "-I", os.path.join(ROOT, "include"), "-I", CSRC,
           DRIVER, os.path.join(CSRC, "fp6_host.cpp"), "-o", out]
    res = subprocess.run(cmd, capture_output=True, text=True)
    assert res.returncode == 0, res.stderr
    return out


def _run(driver, *args):
    res = subprocess.run([driver, *map(str, args)], capture_output=True, text=True, env=ENV, timeout=300)
    assert "Sanitizer" not in res.stderr and "runtime error" not in res.stderr, res.stderr
    return res


def _weights(N, K, seed):
    W = synth.weights(N, K, seed)
    W[0] = 0.0                                    # zero row -> scale 0
    W[1, :] = -1e-9
    W[1, 3] = 0.5                                 # codes -0 around one outlier
    W[2, ::2] = 1.0
    W[2, 1::2] = -1.0                             # saturation at +-max
    return W


def test_host_error_paths_are_clean(driver):
    res = _run(driver, "errors")
    assert res.returncode == 0, (res.returncode, res.stdout, res.stderr)
    assert res.stdout.startswith("errors ok")


@pytest.mark.parametrize("fmt", ["e3m2", "e2m3", "e2m2", "e2m1"])
@pytest.mark.parametrize("N, K", [(16, 256), (48, 768), (32, 2816)])
def test_quantize_and_prepack_match_the_library(driver, tmp_path, fmt, N, K):
    W = _weights(N, K, N * 31 + K)
    wpath = tmp_path / "w.f32"
    W.tofile(wpath)
    out = str(tmp_path / "o")
    res = _run(driver, "quant", fp6.FORMATS[fmt], N, K, wpath, out)
    assert res.returncode == 0, (res.returncode, res.stderr)
    codes = np.fromfile(out + ".codes", np.uint8).reshape(N, K)
    scales = np.fromfile(out + ".scales", np.uint16)
    packed = np.fromfile(out + ".packed", np.uint8)
    c_lib, s_lib = fp6.quantize_rows(W, fmt)
    assert np.array_equal(codes, c_lib) and np.array_equal(scales, s_lib.view(np.uint16))
    assert np.array_equal(packed, fp6.prepack(c_lib, s_lib, fmt))
    c_ref, s_ref = oracle.quantize_rows(W, fmt)
    assert np.array_equal(codes, c_ref) and np.array_equal(scales, s_ref.view(np.uint16))


@pytest.mark.parametrize("N, K", [(16, 512), (48, 1536)])
def test_sparse_prune_and_prepack_match_the_library(driver, tmp_path, N, K):
    W = _weights(N, K, N * 7 + K)
    W[3, :8] = [0.25, -0.25, 0.25, -0.25, 0.5, 0.5, 0.5, 0.5]   # equal magnitudes
    wpath = tmp_path / "w.f32"
    W.tofile(wpath)
    out = str(tmp_path / "o")
    res = _run(driver, "sparse", N, K, wpath, out)
    assert res.returncode == 0, (res.returncode, res.stderr)
    codes = np.fromfile(out + ".codes", np.uint8).reshape(N, K // 2)
    pos = np.fromfile(out + ".pos", np.uint8).reshape(N, K // 2)
    scales = np.fromfile(out + ".scales", np.uint16)
    packed = np.fromfile(out + ".packed", np.uint8)
    c, p, s = fp6.prune_quantize(W)
    assert np.array_equal(codes, c) and np.array_equal(pos, p) and np.array_equal(scales, s.view(np.uint16))
    assert np.array_equal(packed, fp6.sparse_prepack(c, p, s, K))
    oc, op, osc = sparse24.quantize_sparse(W)
    assert np.array_equal(codes, oc) and np.array_equal(pos, op) and np.array_equal(scales, osc.view(np.uint16))
