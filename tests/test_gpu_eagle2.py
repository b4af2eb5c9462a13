"""Parity of spec_tree_expand and spec_tree_rerank with the CPU oracle (bit-exact:
every output is an index, a mask bit or a float32 product decided on float32)."""

import dataclasses

import numpy as np
import pytest

from parity import to_torch
from rejection_sampling_verify_10_amd import workloads as W

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def R():
    import torch
    import rejection_sampling_verify_10_amd as R
    assert torch.cuda.is_available(), "GPU test without a GPU"
    R.lib()
    return R


def run_expand(R, orc, e, name, q=None, nv=None):
    import torch
    q = e.draft_probs if q is None else q
    nv = e.node_values if nv is None else nv
    print(f"[case] expand {name}: B={e.B} E={e.E} V={e.V} top_k={e.top_k} k_next={e.k_next}", flush=True)
    toks, vals, nxt = R.tree_expand(to_torch(q), to_torch(nv), e.top_k, e.k_next)
    torch.cuda.synchronize()
    o = orc.tree_expand(q, nv, e.top_k, e.k_next)
    assert np.array_equal(toks.cpu().numpy(), o["tokens"]), name
    assert np.array_equal(vals.cpu().numpy().view(np.uint32), o["values"].view(np.uint32)), name
    assert np.array_equal(nxt.cpu().numpy(), o["next"]), name
    return o


def test_expand_workload6_full(R, orc):
    """B=64, ten expanded nodes, V=128256, ten children each, ten kept: the launch bench.py times."""
    for seed in range(2):
        run_expand(R, orc, W.config(6, seed), f"workload 6 seed {seed}")


@pytest.mark.parametrize("E,V,K,kn", [(1, 1000, 1, 1), (3, 999, 5, 7), (10, 32000, 10, 10), (16, 4096, 64, 1024),
                                      (2, 300000, 8, 16), (5, 64, 64, 3)])
def test_expand_shapes(R, orc, E, V, K, kn):
    """One to sixteen nodes, a single chunk to several, an odd V (scalar loads), top_k up to 64,
    the largest layer (E*top_k = 1024)."""
    run_expand(R, orc, W.make_expand(8, E, V, top_k=K, k_next=kn, config_id=61, seed=E * K), f"E={E} V={V} K={K}")


def test_expand_ties_and_errors(R, orc):
    e = W.make_expand(8, 4, 5000, top_k=6, k_next=9, config_id=62, seed=0)
    q, nv = e.draft_probs.copy(), e.node_values.copy()
    q[0, 1, [10, 20, 4000]] = q[0, 1].max() * 2            # equal top probabilities across chunks
    q[1] = np.round(q[1] * 1e4) / 1e4                       # many equal values
    nv[2] = nv[2, 0]                                        # equal node values: equal products
    q[3, 2, 17] = np.nan
    q[4, 0, 5] = -1e-3
    q[5, 3, 4999] = np.inf
    nv[6, 1] = -0.5
    o = run_expand(R, orc, e, "ties and errors", q.astype(np.float32), nv.astype(np.float32))
    assert np.all(o["next"][3:7] == -1) and np.all(o["next"][[0, 1, 2, 7]] >= 0)


def run_rerank(R, orc, r, name, par=None, val=None):
    import torch
    par = r.parents if par is None else par
    val = r.values if val is None else val
    print(f"[case] rerank {name}: B={r.B} M={r.M} m={r.m}", flush=True)
    nodes, ppos, mask = R.tree_rerank(to_torch(par), to_torch(val), r.m)
    torch.cuda.synchronize()
    o = orc.tree_rerank(par, val, r.m)
    assert np.array_equal(nodes.cpu().numpy(), o["nodes"]), name
    assert np.array_equal(ppos.cpu().numpy(), o["parent_pos"]), name
    assert np.array_equal(mask.cpu().numpy(), o["mask"]), name
    return o


@pytest.mark.parametrize("k,depth,m", [(2, 2, 1), (4, 4, 10), (10, 6, 60), (8, 16, 200), (8, 16, 968),
                                       (1, 30, 30), (31, 2, 40)])
def test_rerank_shapes(R, orc, k, depth, m):
    """From two candidates to 968 (a 1024-slot sort with padding), m from 1 to M, a path
    (k = 1) and a wide two-layer tree; every fourth tree has coarse (tied) values."""
    run_rerank(R, orc, W.make_rerank(12, k=k, depth=depth, m=m, config_id=63, seed=k * depth), f"k={k} d={depth}")


def test_rerank_all_equal_and_errors(R, orc):
    r = W.make_rerank(6, k=3, depth=4, m=12, config_id=64, seed=0)
    run_rerank(R, orc, r, "all equal", val=np.ones_like(r.values))
    par, val = r.parents.copy(), r.values.copy()
    val[1, 3] = 0.999
    val[1, int(par[1, 3])] = 1e-6
    par[2, 5] = 7
    val[3, 0] = np.nan
    par[4, 9] = -2
    o = run_rerank(R, orc, r, "errors", par, val)
    assert np.all(o["nodes"][1:5] == -1) and np.all(o["nodes"][[0, 5]] >= 0)


def test_two_layers_then_rerank(R, orc):
    """An expansion layer from the root, a second from the kept children, then the
    reranking of all children so far: the GPU chain of calls against the oracle's."""
    import torch
    V, K, B = 20000, 6, 4
    root = W.make_expand(B, 1, V, top_k=K, k_next=K, config_id=65, seed=0)
    o1 = run_expand(R, orc, root, "layer 1", nv=np.ones((B, 1), np.float32))
    lay2 = W.make_expand(B, K, V, top_k=K, k_next=K, config_id=65, seed=1)
    nv2 = np.take_along_axis(o1["values"].reshape(B, -1), o1["next"], axis=1).astype(np.float32)
    o2 = run_expand(R, orc, lay2, "layer 2", nv=nv2)
    M = K + K * K
    par = np.concatenate([np.full((B, K), -1, np.int32), np.repeat(o1["next"], K, axis=1)], axis=1)
    val = np.concatenate([o1["values"].reshape(B, -1), o2["values"].reshape(B, -1)], axis=1).astype(np.float32)
    r = W.RerankInputs(B, M, 16, par.astype(np.int32), val)
    o = run_rerank(R, orc, r, "two layers")
    assert np.all(o["nodes"] >= 0)


def _row_oracle(orc, fn, B, N, parents_rows, *args):
    """The oracle row by row with each row's own tree, outputs padded to N entries."""
    path = np.full((B, N), -1, np.int32)
    toks = np.full((B, N), -1, np.int32)
    alen = np.full(B, -1, np.int32)
    margins = []
    for b in range(B):
        par = parents_rows[b]
        ok = par[0] == -1 and all(0 <= par[n] < n for n in range(1, N))
        if not ok:
            margins.append(None)
            continue
        o = fn(b, par, *args)
        D1 = o["path"].shape[1]
        path[b, :D1], toks[b, :D1], alen[b] = o["path"][0], o["tokens"][0], o["accept_len"][0]
        margins.append(o)
    return path, toks, alen, margins


def _reranked_trees(R, B, N, seed):
    """Per-row trees from the GPU's own reranking: parents[b][0] = -1, node p + 1's parent
    is the kept node's parent position."""
    import torch
    r = W.make_rerank(B, k=4, depth=4, m=N - 1, config_id=66, seed=seed)
    _, ppos, _ = R.tree_rerank(to_torch(r.parents), to_torch(r.values), N - 1)
    torch.cuda.synchronize()
    par = np.concatenate([np.full((B, 1), -1, np.int32), ppos.cpu().numpy()], axis=1)
    return par


def test_reranked_trees_verified_greedy(R, orc):
    """Greedy verification with a tree per batch row (spec_verify_tree_greedy_rows), the
    trees from spec_tree_rerank; one malformed row."""
    import torch
    B, N, V = 16, 21, 5000
    par = _reranked_trees(R, B, N, 0)
    par[5, 7] = 9                                    # a parent after its child: an error row
    ti = W.make_tree(B, V, parents=W.EAGLE_TREE_PARENTS[:N], config_id=67, seed=0)
    # node tokens: for half the nodes the argmax of the parent's row, so that paths go deep
    z = ti.logits_f32()
    tok = ti.node_tokens.copy()
    for b in range(B):
        for n in range(1, N):
            p = par[b, n] if 0 <= par[b, n] < n else 0
            tok[b, n] = int(np.argmax(z[b, p])) if (n + b) % 2 else (int(np.argmax(z[b, p])) + 1) % V
    path, toks, alen = R.verify_tree_greedy(to_torch(ti.logits), to_torch(tok), torch.from_numpy(par).cuda())
    torch.cuda.synchronize()
    op, ot, oa, _ = _row_oracle(orc, lambda b, p: orc.verify_tree_greedy(ti.logits[b:b + 1], ti.dtype,
                                                                        tok[b:b + 1], p), B, N, par)
    assert np.array_equal(alen.cpu().numpy(), oa)
    assert np.array_equal(path.cpu().numpy(), op) and np.array_equal(toks.cpu().numpy(), ot)
    assert oa[5] == -1 and np.max(oa) >= 2


def test_reranked_trees_verified_sampled(R, orc):
    """Sampling verification with a tree per batch row (spec_verify_tree_sample_rows)."""
    import torch
    from parity import MARGIN
    B, N, V = 24, 21, 8000
    par = _reranked_trees(R, B, N, 1)
    par[3, 0] = 0                                    # the root must have no parent: an error row
    ts = W.make_tree_sampled(B, V, parents=W.EAGLE_TREE_PARENTS[:N], config_id=68, seed=0)
    path, toks, alen = R.verify_tree_sample(to_torch(ts.logits), to_torch(ts.draft_probs), to_torch(ts.node_tokens),
                                            to_torch(ts.uniforms), torch.from_numpy(par).cuda(), 1.0, 0)
    torch.cuda.synchronize()
    path, toks, alen = path.cpu().numpy(), toks.cpu().numpy(), alen.cpu().numpy()
    op, ot, oa, outs = _row_oracle(
        orc, lambda b, p: orc.verify_tree_sample(ts.logits[b:b + 1], ts.dtype, ts.draft_probs[b:b + 1],
                                                 ts.node_tokens[b:b + 1], ts.uniforms[b:b + 1], p, 1.0, 0),
        B, N, par)
    assert alen[3] == -1 and oa[3] == -1
    for b in range(B):
        if np.array_equal(path[b], op[b]) and np.array_equal(toks[b], ot[b]):
            continue
        o = outs[b]                                  # a differing decision must sit on a tiny margin
        assert o is not None and (np.nanmin(o["m_test"][0]) < MARGIN or o["m_draw"][0] < MARGIN), b
