"""HIP-graph capture of the fused linear (needs an MI355X).

The split-K paths reuse one workspace whose per-unit arrival counters reset
themselves, so a captured launch must give the same result on every replay.
Each case runs eagerly first on the stream it is then captured on (the
workspace is kept per stream, so this sizes it and nothing is allocated
during capture), is captured on that side stream, and is replayed
several times with eager launches and synchronisations in between; every
replay must equal the eager output bit for bit.  Nothing in the captured
region clears memory: the output is cleared eagerly before each replay.
"""

import pytest

from weight_only_fp6_amd import synth

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():  # pragma: no cover - CPU container
    pytest.skip("no GPU", allow_module_level=True)

import weight_only_fp6_amd as fp6  # noqa: E402

DEV = torch.device("cuda:0")

# (M, N, K, variant, splits): automatic plans that split K across
# workgroups, forced streaming and tiled plans with the fix-up, and plans
# without a workspace.
DENSE = [
    (16, 8192, 8192, 0, 0),      # k-split, 2 K-splits
    (1, 4096, 11008, 12, 3),     # k-split, 3 K-splits, M = 1 staging
    (16, 4096, 11008, 12, 3),
    (16, 11008, 4096, 0, 0),     # k-split, no workspace
    (32, 4096, 4096, 0, 0),      # streaming, 32 columns, K-splits
    (5, 2048, 28672, 15, 2),     # streaming, ragged M
    (128, 2048, 7168, 10, 3),    # tiled
    (128, 2048, 7168, 23, 3),    # tiled, weights staged in LDS (probe-first fix-up)
    (256, 4096, 7168, 25, 0),    # tiled, stream-K
    (1, 4096, 4096, 0, 0),       # k-slice
]
SPARSE = [
    (16, 8192, 8192, 0, 0),      # sparse k-split, 2 K-splits
    (32, 4096, 4096, 0, 0),      # sparse streaming, 32 columns
    (16, 4096, 8192, 2, 4),
    (64, 2048, 4096, 4, 2),      # sparse tiled
]


def _prepare(N, K, seed, sparse):
    W = synth.weights(N, K, seed)
    if sparse:
        c, pos, s = fp6.prune_quantize(W)
        packed = fp6.sparse_prepack(c, pos, s, K)
    else:
        c, s = fp6.quantize_rows(W)
        packed = fp6.prepack(c, s)
    return torch.from_numpy(packed).to(DEV), torch.from_numpy(s.copy()).to(DEV)


@pytest.mark.parametrize("sparse", [False, True])
def test_graph_replays_match_eager(sparse):
    run = fp6.sparse_linear_plan if sparse else fp6.linear_plan
    stream = torch.cuda.Stream()
    for i, (M, N, K, variant, splits) in enumerate(SPARSE if sparse else DENSE):
        what = (M, N, K, variant, splits)
        print("graph case", sparse, what, flush=True)
        P, S = _prepare(N, K, 700 + i, sparse)
        X = torch.from_numpy(synth.activations(M, K, 710 + i)).to(DEV)
        with torch.cuda.stream(stream):
            want = run(X, P, S, N, K, variant=variant, splits=splits, stream=stream).clone()
        torch.cuda.synchronize()
        out = torch.empty_like(want)
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=stream):
            run(X, P, S, N, K, variant=variant, splits=splits, out=out, stream=stream)
        torch.cuda.synchronize()
        for rep in range(4):
            out.zero_()
            torch.cuda.synchronize()
            g.replay()
            torch.cuda.synchronize()
            assert torch.equal(out.view(torch.int16), want.view(torch.int16)), (what, rep)
            again = run(X, P, S, N, K, variant=variant, splits=splits)
            torch.cuda.synchronize()
            assert torch.equal(again.view(torch.int16), want.view(torch.int16)), (what, rep)
        del g


def test_workspace_keeps_the_largest_sizes_for_capture():
    # Plan A needs many arrival counters and a small partial buffer, plan B
    # a larger buffer and fewer counters.  After eager calls of A then B on
    # a stream, both must be capturable there (the workspace only grows, so
    # neither reallocates during capture) and replay to the eager result.
    # torch hands out pooled stream handles, which earlier tests may already
    # have given a large workspace: release every workspace first so that A
    # and B grow a fresh one, in that order.
    torch.cuda.synchronize()
    fp6.release()
    stream = torch.cuda.Stream()
    cases = [(16, 10240, 2048, 12, 2), (16, 4096, 8192, 14, 8)]
    runs = []
    for i, (M, N, K, v, sp) in enumerate(cases):
        P, S = _prepare(N, K, 900 + i, False)
        X = torch.from_numpy(synth.activations(M, K, 910 + i)).to(DEV)
        runs.append((X, P, S, N, K, v, sp))
    wants = []
    with torch.cuda.stream(stream):
        for X, P, S, N, K, v, sp in runs:
            wants.append(fp6.linear_plan(X, P, S, N, K, variant=v, splits=sp, stream=stream).clone())
    torch.cuda.synchronize()
    for (X, P, S, N, K, v, sp), want in zip(runs, wants):
        out = torch.empty_like(want)
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=stream):
            fp6.linear_plan(X, P, S, N, K, variant=v, splits=sp, out=out, stream=stream)
        torch.cuda.synchronize()
        for rep in range(2):
            out.zero_()
            torch.cuda.synchronize()
            g.replay()
            torch.cuda.synchronize()
            assert torch.equal(out.view(torch.int16), want.view(torch.int16)), (N, K, v, sp, rep)
        del g


def test_graph_survives_a_later_workspace_growth():
    # A graph captured with a small split plan stays valid after a larger
    # split plan grows the stream's workspace: the grown workspace's old
    # buffers stay allocated until fp6_release, so every replay of the first
    # graph still equals its eager result, with eager calls of the larger
    # plan (on the new buffers) in between.
    torch.cuda.synchronize()
    fp6.release()
    stream = torch.cuda.Stream()
    small = (16, 4096, 8192, 15, 2)      # streaming, 2 K-splits: 512 KB of partial sums
    large = (16, 8192, 28672, 18, 8)     # streaming, 8 K-splits: 4 MB, more counters
    runs = []
    for i, (M, N, K, v, sp) in enumerate((small, large)):
        P, S = _prepare(N, K, 950 + i, False)
        X = torch.from_numpy(synth.activations(M, K, 960 + i)).to(DEV)
        runs.append((X, P, S, N, K, v, sp))
    Xs, Ps, Ss, Ns, Ks, vs, sps = runs[0]
    Xl, Pl, Sl, Nl, Kl, vl, spl = runs[1]
    with torch.cuda.stream(stream):
        want_s = fp6.linear_plan(Xs, Ps, Ss, Ns, Ks, variant=vs, splits=sps, stream=stream).clone()
    torch.cuda.synchronize()
    out = torch.empty_like(want_s)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=stream):
        fp6.linear_plan(Xs, Ps, Ss, Ns, Ks, variant=vs, splits=sps, out=out, stream=stream)
    torch.cuda.synchronize()
    with torch.cuda.stream(stream):
        want_l = fp6.linear_plan(Xl, Pl, Sl, Nl, Kl, variant=vl, splits=spl, stream=stream).clone()
    torch.cuda.synchronize()
    for rep in range(3):
        out.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int16), want_s.view(torch.int16)), rep
        with torch.cuda.stream(stream):
            again = fp6.linear_plan(Xl, Pl, Sl, Nl, Kl, variant=vl, splits=spl, stream=stream)
        torch.cuda.synchronize()
        assert torch.equal(again.view(torch.int16), want_l.view(torch.int16)), rep
    del g
    torch.cuda.synchronize()
    fp6.release()
