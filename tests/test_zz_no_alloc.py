"""fp6_linear_noalloc (split-K scratch in a static device array, no
allocation) against fp6_linear, through the C ABI (needs an MI355X).

Two split-K calls in a row share the one scratch array, the second on a
smaller layer: each must equal fp6_linear's result bit for bit (same plan and
kernels) and lie within the oracle tolerance.  A third call repeats the
first, so the arrival counters the earlier calls left behind must be zero.
"""

import numpy as np
import pytest

import oracle

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():  # pragma: no cover - CPU container
    pytest.skip("no GPU", allow_module_level=True)

import weight_only_fp6_amd as fp6  # noqa: E402

from _workloads import workload  # noqa: E402

DEV = torch.device("cuda:0")


def _noalloc(X, P, S, N, K, out):
    st = fp6.lib.fp6_linear_noalloc(X.data_ptr(), P.data_ptr(), S.data_ptr(), out.data_ptr(),
                                    X.shape[0], N, K, torch.cuda.current_stream().cuda_stream)
    assert st == 0, fp6.STATUS_NAMES.get(st, st)


def test_noalloc_matches_fp6_linear_on_consecutive_calls():
    # OPT-30B QKV M=128: tiled kernel with 3 K-splits (31.5 MiB of partial
    # sums); then the smaller Llama-7B MLP down projection (k-split kernel, 3
    # K-splits); then M=256, stream-K (53 MiB); then the first layer again.
    # And a plan without K-splits.
    names = ["opt30b_qkv_128x21504x7168", "llama7b_mlp_down_16x4096x11008",
             "llama70b_mlp_16x28672x8192", "opt30b_qkv_256x21504x7168"]
    runs = []
    for name in names:
        ws, X, yref = workload(name)
        P, S = ws.to_device()
        Xd = torch.from_numpy(X).to(DEV)
        want = fp6.linear(Xd, P, S, ws.N, ws.K)
        runs.append((name, Xd, P, S, ws.N, ws.K, want, yref))
    torch.cuda.synchronize()
    assert fp6.plan_query(128, 21504, 7168)[1] > 1 and fp6.plan_query(16, 4096, 11008)[1] > 1
    order = [0, 1, 3, 0, 2]
    outs = []
    for i in order:
        name, Xd, P, S, N, K, _, _ = runs[i]
        out = torch.full((Xd.shape[0], N), float("nan"), dtype=torch.float16, device=DEV)
        _noalloc(Xd, P, S, N, K, out)
        outs.append(out)
    torch.cuda.synchronize()
    for i, out in zip(order, outs):
        name, _, _, _, _, _, want, yref = runs[i]
        assert torch.equal(out.view(torch.int16), want.view(torch.int16)), name
        rep = oracle.tolerance_report(out.cpu().numpy().astype(np.float64), yref)
        assert rep["ok"], (name, rep)


def test_noalloc_m_zero_and_argument_errors():
    N, K = 16, 256
    L = fp6.lib
    assert L.fp6_linear_noalloc(None, None, None, None, 0, N, K, None) == 0
    A = 1 << 20   # never dereferenced: every check fails before a launch
    assert L.fp6_linear_noalloc(A, A, A, A, 4, 24, 256, None) == 2
    assert L.fp6_linear_noalloc(None, A, A, A, 4, 16, 256, None) == 1
    assert L.fp6_linear_noalloc(A + 8, A, A, A, 4, 16, 256, None) == 3
