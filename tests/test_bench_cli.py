"""bench.py's command line on a host without a GPU: the help text renders,
a multi-GPU request is refused with a message, and the roofline arithmetic
helpers give the byte counts the measurement is priced on."""

import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402


def _run(*args):
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args],
                          capture_output=True, text=True, timeout=120)


def test_help_renders():
    r = _run("--help")
    assert r.returncode == 0, r.stderr
    assert "--workload" in r.stdout and "--sparse" in r.stdout


def test_more_than_one_gpu_is_refused():
    r = _run("--gpus", "2")
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def test_algorithmic_bytes_of_the_llama70b_mlp_layer():
    # 6 bits per weight, fp16 scales per row, fp16 X and Y.
    M, N, K = 16, 28672, 8192
    assert bench.weight_bytes(N, K) == N * K * 3 // 4
    assert bench.weight_bytes(N, K, "e2m1") == N * K // 2
    assert bench.weight_bytes(N, K, "sparse24") == N * K // 2
    assert bench.algorithmic_bytes(M, N, K) == N * K * 3 // 4 + 2 * N + 2 * M * K + 2 * M * N
