"""Chain calls captured in a HIP graph and replayed.

A replay reuses the captured launch arguments, so a top-k chain replays with the tag of
the captured call: its hand-over words must be left zero by every replay, and the
no-allocation entry point (for callers that capture graphs) must find its scratch as the
captured call left it.  Each captured call is replayed several times, with eager calls
on other inputs (on another workspace, or on the same no-allocation scratch) and
synchronisations between the replays; every replay must reproduce the eager result of
its inputs bit for bit (the kernels are deterministic).  Workspaces and outputs are
allocated and zeroed before capture, so the graphs hold kernels only.
"""

import numpy as np
import pytest

from parity import to_torch
from rejection_sampling_verify_10_amd import workloads as W

pytestmark = pytest.mark.gpu

REPLAYS = 4


@pytest.fixture(scope="module")
def R():
    import torch
    import rejection_sampling_verify_10_amd as R
    assert torch.cuda.is_available(), "GPU test without a GPU"
    R.lib()
    return R


def inputs(ci):
    return [to_torch(a) for a in (ci.logits, ci.draft_probs, ci.draft_tokens, ci.uniforms)]


def outputs(B, K, dev):
    import torch
    return (torch.full((B, K + 1), -7, dtype=torch.int32, device=dev),
            torch.full((B,), -7, dtype=torch.int32, device=dev),
            torch.full((B, 2 * K + 2), -7.0, dtype=torch.float32, device=dev))


def same(a, b):
    return all(np.array_equal(x.cpu().numpy(), y.cpu().numpy(), equal_nan=True) for x, y in zip(a, b))


@pytest.mark.parametrize("T,top_k,B,cid", [(0.7, 50, 16, 2), (1.0, 0, 512, 4), (0.0, 0, 16, 2), (1.0, 0, 8, 1),
                                           (0.8, 0, 8, 1)])
def test_chain_graph_replays(R, T, top_k, B, cid):
    """spec_verify_chain on a workspace zeroed once: top-k chain (tags reused by every
    replay), the dense walk (T = 1, B*(K+1) > 1344), greedy, and the all-rows route with
    its draw split over several workgroups per row (c1's shape, T = 1 and a transformed
    draft: statistics, power sums, draw slices and their combine in one graph)."""
    import torch
    dev = torch.device("cuda")
    ci = W.with_transform(W.config(cid, 80, B=B), temperature=T, top_k=top_k)
    other = W.with_transform(W.config(cid, 81, B=B), temperature=T, top_k=top_k)
    K, V = ci.K, ci.V
    z, q, x, u = inputs(ci)
    zo, qo, xo, uo = inputs(other)
    need = R.chain_workspace_bytes(B, K, V, ci.dtype, T, top_k)
    ws = R.new_workspace(need, dev)
    ws_other = R.new_workspace(need, dev)
    want = R.verify_chain(z, q, x, u, T, top_k, diag=True, workspace=R.new_workspace(need, dev))
    want_other = R.verify_chain(zo, qo, xo, uo, T, top_k, diag=True, workspace=R.new_workspace(need, dev))
    out = outputs(B, K, dev)
    torch.cuda.synchronize()
    print(f"[case] graph capture T={T} top_k={top_k} B={B}", flush=True)
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            R.verify_chain(z, q, x, u, T, top_k, diag=True, out=out, workspace=ws)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    for rep in range(REPLAYS):
        for o in out:
            o.fill_(-7)
        g.replay()
        torch.cuda.synchronize()
        assert same(out, want), f"replay {rep} differs from the eager call"
        got = R.verify_chain(zo, qo, xo, uo, T, top_k, diag=True, workspace=ws_other)
        torch.cuda.synchronize()
        assert same(got, want_other), f"eager call after replay {rep} differs"
    print(f"[graph] {REPLAYS} replays match", flush=True)


@pytest.mark.parametrize("T,top_k,B,cid", [(0.7, 50, 16, 2), (1.0, 0, 512, 4)])
def test_noalloc_graph_replays(R, T, top_k, B, cid):
    """spec_verify_chain_noalloc captured after one eager call on the device; replays
    alternate with eager calls of the same kind on the same scratch (a top-k chain leaves
    its words zero; the dense walk keeps nothing there).  The zero-fill decision is taken
    when a call is issued, so replays are not interleaved with calls that leave scratch
    behind."""
    import torch
    dev = torch.device("cuda")
    ci = W.with_transform(W.config(cid, 82, B=B), temperature=T, top_k=top_k)
    K, V = ci.K, ci.V
    z, q, x, u = inputs(ci)
    gi = W.with_transform(W.config(cid, 83, B=B), temperature=T, top_k=top_k)
    zg, qg, xg, ug = inputs(gi)
    need = R.chain_workspace_bytes(B, K, V, ci.dtype, T, top_k)
    want = R.verify_chain(z, q, x, u, T, top_k, diag=True, workspace=R.new_workspace(need, dev))
    want_g = R.verify_chain(zg, qg, xg, ug, T, top_k, diag=True, workspace=R.new_workspace(need, dev))
    R.verify_chain_noalloc(z, q, x, u, T, top_k, diag=True, out=outputs(B, K, dev))   # looks the scratch up
    out = outputs(B, K, dev)
    torch.cuda.synchronize()
    print(f"[case] no-allocation graph capture T={T} top_k={top_k} B={B}", flush=True)
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            R.verify_chain_noalloc(z, q, x, u, T, top_k, diag=True, out=out)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    for rep in range(REPLAYS):
        for o in out:
            o.fill_(-7)
        g.replay()
        torch.cuda.synchronize()
        assert same(out, want), f"replay {rep} differs from the eager call"
        got = R.verify_chain_noalloc(zg, qg, xg, ug, T, top_k, diag=True)
        torch.cuda.synchronize()
        assert same(got, want_g), f"eager call after replay {rep} differs"
    print(f"[graph] {REPLAYS} no-allocation replays match", flush=True)


def test_tree_sample_ws_graph_replays(R):
    """spec_verify_tree_sample_ws (each batch row's walk shared by a cluster of workgroups
    exchanging words through the workspace) captured once and replayed: the words are left
    zero by every call, so every replay reproduces the eager result."""
    import torch
    dev = torch.device("cuda")
    ti, other = W.config(5, 90), W.config(5, 91)

    def args(t):
        return [to_torch(a) for a in (t.logits, t.draft_probs, t.node_tokens, t.uniforms)]

    a0, a1 = args(ti), args(other)
    B, N = ti.B, ti.N
    par = ti.parents.tolist()
    need = R.tree_sample_workspace_bytes(B, N)
    ws, ws_other = R.new_workspace(need, dev), R.new_workspace(need, dev)
    want = R.verify_tree_sample(*a0, par, ti.temperature, 0, workspace=R.new_workspace(need, dev))
    want_other = R.verify_tree_sample(*a1, par, other.temperature, 0, workspace=R.new_workspace(need, dev))
    D = want[0].shape[1] - 1
    out = (torch.full((B, D + 1), -7, dtype=torch.int32, device=dev),
           torch.full((B, D + 1), -7, dtype=torch.int32, device=dev),
           torch.full((B,), -7, dtype=torch.int32, device=dev))
    torch.cuda.synchronize()
    print(f"[case] tree-sample graph capture B={B} N={N}", flush=True)
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            R.verify_tree_sample(*a0, par, ti.temperature, 0, out=out, workspace=ws)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    for rep in range(REPLAYS):
        for o in out:
            o.fill_(-7)
        g.replay()
        torch.cuda.synchronize()
        assert same(out, want), f"replay {rep} differs from the eager call"
        assert int(torch.count_nonzero(ws)) == 0
        got = R.verify_tree_sample(*a1, par, other.temperature, 0, workspace=ws_other)
        torch.cuda.synchronize()
        assert same(got, want_other), f"eager call after replay {rep} differs"
    print(f"[graph] {REPLAYS} tree-sample replays match", flush=True)
