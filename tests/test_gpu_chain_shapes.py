"""GPU parity at the decoder-layer chain shapes (needs an MI355X).

The linear layers of one Llama-7B and one Llama-70B decoder layer (qkv, o,
gate_up, down, with the projections that share an input fused along N) at the
batch sizes the chain is timed at, M = 1, 2, 4, 8 and 16, through the
automatic plan of FP6 e3m2 (fp6_linear), FP4 e2m1 (fpx_linear) and 2:4-sparse
FP6 (fp6s_linear; layers with K % 512 == 0).  Codes are uniform over every
code of the format and row scales random in [0.002, 0.004), the inputs the
chain is timed with; every output element is compared with the oracle
(|Y - Y_ref| <= 2e-3 (|Y_ref| + rms), relative Frobenius <= 5e-4) and the
whole de-quantised weight matrix bit for bit.
"""

import numpy as np
import pytest

import oracle
from weight_only_fp6_amd import synth

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():  # pragma: no cover - CPU container
    pytest.skip("no GPU", allow_module_level=True)

import weight_only_fp6_amd as fp6  # noqa: E402

from _workloads import uniform_code_weight_set, y_ref  # noqa: E402

DEV = torch.device("cuda:0")
CHAIN_M = (1, 2, 4, 8, 16)
# (N, K) of the fused linears: Llama-7B (hidden 4096, MLP 11008) and
# Llama-70B (hidden 8192, 8 KV heads of 128, MLP 28672).
LAYERS = [(12288, 4096), (4096, 4096), (22016, 4096), (4096, 11008),
          (10240, 8192), (8192, 8192), (57344, 8192), (8192, 28672)]
CASES = [(kind, N, K) for kind in ("e3m2", "e2m1", "sparse") for (N, K) in LAYERS
         if kind != "sparse" or K % 512 == 0]


@pytest.mark.parametrize("kind, N, K", CASES)
def test_chain_layer(kind, N, K):
    sparse = kind == "sparse"
    fmt = "e3m2" if sparse else kind
    seed = N + 3 * K + {"e3m2": 0, "e2m1": 1, "sparse": 2}[kind]
    ws = uniform_code_weight_set(N, K, seed, fmt, sparse)
    packed, s = ws.to_device()
    # Y_ref for every batch size from one stacked activation matrix
    Xall = synth.activations(sum(CHAIN_M), K, seed + 5)
    yall = y_ref(Xall, ws.wdq_ref)
    r0 = 0
    for M in CHAIN_M:
        X = torch.from_numpy(Xall[r0:r0 + M]).to(DEV)
        if sparse:
            Y = fp6.sparse_linear(X, packed, s, N, K)
            plan = fp6.sparse_plan_query(M, N, K)
        else:
            Y = fp6.linear(X, packed, s, N, K, fmt=fmt)
            plan = fp6.plan_query(M, N, K)
        torch.cuda.synchronize()
        rep = oracle.tolerance_report(Y.cpu().numpy().astype(np.float64), yall[r0:r0 + M])
        assert rep["ok"], (kind, M, N, K, plan, rep)
        r0 += M
    W16 = fp6.sparse_dequant(packed, s, N, K) if sparse else fp6.dequant(packed, s, N, K, fmt=fmt)
    torch.cuda.synchronize()
    assert np.array_equal(W16.cpu().numpy().view(np.uint16), ws.wdq_ref.view(np.uint16)), (kind, N, K)
