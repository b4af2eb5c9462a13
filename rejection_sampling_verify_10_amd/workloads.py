"""Seeded synthetic inputs for the speculative-decoding verification step.

This module only draws random data.  It holds none of the verification
arithmetic (no ratio test, no residual, no verification-side top-k or
temperature transform); both the HIP library and the CPU oracle are fed the
arrays it returns, and nothing else is shared between them.

Recipe (one batch row ``b`` at a time, from ``numpy.random.default_rng(
[config_id, seed, b])`` so that rows are independent and can be drawn in
parallel threads with a result that does not depend on the thread count):

1. for every target row (position ``k`` of a chain, or node ``n`` of a tree)
   a fresh permutation ``rank`` of ``1..V``;
2. target noise ``n_t ~ N(0,1)`` of shape ``[rows, V]``;
   target logits ``z = 3*n_t - 1.1*ln(rank)`` (float32), stored as bfloat16
   (round to nearest even) or float32;
3. draft noise ``n_d ~ N(0,1)``; draft logits ``zd = z + sigma_b*n_d`` built
   from the *unrounded* float32 ``z``; draft probabilities
   ``q = softmax(zd)`` computed in float64 and stored as float32;
4. ``sigma_b`` is fixed per config, split by batch half, or drawn per batch
   row from ``U(lo, hi)`` (drawn after the draft noise);
5. draft tokens: one uniform per draft position, turned into a token of the
   draft model's own sampling distribution -- ``softmax(zd/T)`` restricted to
   the ``top_k`` largest draft logits when a temperature or top-k is in force,
   else ``q`` itself -- by ``numpy.searchsorted`` on its cumulative sum
   (this is the draft model sampling its proposal, not the verifier);
6. verification uniforms ``u ~ U[0,1)`` float32 of shape ``[K+1]``.

Trees (greedy verification) draw, per batch row: a permutation and noise
for each of the N node rows as above, draft noise per node row, and give the
children of node ``p`` the best draft tokens of ``zd_p`` in sibling order.

Sampled trees draw, per batch row: target rows and draft noise for the N
nodes as above, the draft probabilities ``q_n = softmax(zd_n)`` of every node
(row ``n`` is the draft model's distribution at node ``n``, from which its
children are drawn), then for each node ``p`` in order its children's tokens,
independently, from the draft model's sampling distribution at ``p`` (step
5), and last the N verification uniforms.

A KV commit draws random cache contents (bf16 bits), a prefix length per
batch row and the path from the root to a node of the tree picked at a
uniformly drawn depth.

Draft-tree construction (EAGLE-2) draws, per batch row: for an expansion
layer, E draft rows as in step 3 (q = softmax(z + sigma*N(0,1)) of a fresh
target-like row) and the E expanded nodes' values, sorted descending in
(0.05, 1]; for reranking, a layered candidate tree -- each layer gives k
children to k nodes picked at random from the layer before -- whose node
values are the parent's value times a confidence in (0, 1] (float32; every
fourth tree draws confidences from a coarse grid so that equal values occur).

The value distribution follows the workloads described for the method: a
Zipf-like ``-1.1*ln(rank)`` prior plus Gaussian spread gives a long-tailed
next-token distribution, and the draft is the same distribution seen through
extra logit noise, which sets the acceptance rate.
"""

from __future__ import annotations

import dataclasses
import math
import os
from concurrent.futures import ThreadPoolExecutor
from typing import Callable, Optional, Sequence

import numpy as np

# Parent array of the static draft tree: 27 nodes in breadth-first order,
# depth 5, with 3, 3, 2, 2, 1 children along the left-most (top) path and more
# nodes on the upper-left side than the lower-right.
EAGLE_TREE_PARENTS = np.array(
    [-1, 0, 0, 0, 1, 1, 1, 2, 2, 3, 4, 4, 5, 5, 6, 7, 7, 8, 9,
     10, 10, 11, 12, 15, 19, 20, 21], dtype=np.int32)

DTYPE_F32 = 0
DTYPE_BF16 = 1


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16 (nearest, ties to even); return uint16 bits."""
    b = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    r = (b + np.uint32(0x7FFF) + ((b >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)
    return r.astype(np.uint16)


def bf16_bits_to_f32(h: np.ndarray) -> np.ndarray:
    """Widen bfloat16 bits (uint16) to float32 exactly."""
    return (np.asarray(h, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


@dataclasses.dataclass
class ChainInputs:
    """Inputs of one batched chain verification call (all row-major, contiguous)."""
    B: int
    K: int
    V: int
    dtype: int                 # DTYPE_BF16 (logits as uint16 bits) or DTYPE_F32
    temperature: float
    top_k: int
    logits: np.ndarray         # [B, K+1, V] uint16 (bf16 bits) or float32
    draft_probs: np.ndarray    # [B, K, V] float32
    draft_tokens: np.ndarray   # [B, K] int32
    uniforms: np.ndarray       # [B, K+1] float32 in [0, 1)
    sigma: np.ndarray          # [B] draft noise scale per batch row (for reports)

    def logits_f32(self) -> np.ndarray:
        return bf16_bits_to_f32(self.logits) if self.dtype == DTYPE_BF16 else self.logits


@dataclasses.dataclass
class TreeInputs:
    """Inputs of one batched greedy tree verification call."""
    B: int
    N: int
    V: int
    dtype: int
    logits: np.ndarray         # [B, N, V] uint16 (bf16 bits) or float32
    node_tokens: np.ndarray    # [B, N] int32 (entry 0, the root, is ignored and set to -1)
    parents: np.ndarray        # [N] int32, parents[0] = -1, 0 <= parents[i] < i

    def logits_f32(self) -> np.ndarray:
        return bf16_bits_to_f32(self.logits) if self.dtype == DTYPE_BF16 else self.logits


def _log_rank_table(V: int) -> np.ndarray:
    return np.log(np.arange(1, V + 1, dtype=np.float64)).astype(np.float32)


def _target_rows(rng: np.random.Generator, rows: int, V: int, log_rank: np.ndarray) -> np.ndarray:
    perms = np.stack([rng.permutation(V) for _ in range(rows)])
    noise = rng.standard_normal((rows, V), dtype=np.float32)
    return (np.float32(3.0) * noise - np.float32(1.1) * log_rank[perms]).astype(np.float32)


def _softmax64(a: np.ndarray) -> np.ndarray:
    e = np.exp(a - a.max(axis=-1, keepdims=True))
    return e / e.sum(axis=-1, keepdims=True)


def _draft_sampler_cdf(zd_row: np.ndarray, T: float, top_k: int, top_p: float = 1.0) -> np.ndarray:
    """Cumulative sum of the draft model's own sampling distribution (float64), with its
    own nucleus when top_p < 1."""
    V = zd_row.shape[0]
    if top_p < 1.0:
        w = np.diff(_draft_sampler_cdf(zd_row, T, top_k), prepend=0.0)
        order = np.argsort(-w, kind="stable")
        n = int(np.searchsorted(np.cumsum(w[order]), top_p * w.sum(), side="left")) + 1
        keep = np.zeros(V, dtype=bool)
        keep[order[:n]] = True
        return np.cumsum(np.where(keep, w, 0.0))
    if T == 0.0:                        # greedy draft: its argmax
        w = np.zeros(V, dtype=np.float64)
        w[int(np.argmax(zd_row))] = 1.0
        return np.cumsum(w)
    if T == 1.0 and not (0 < top_k < V):
        w = _softmax64(zd_row)
    else:
        w = np.zeros(V, dtype=np.float64)
        keep = np.arange(V) if not (0 < top_k < V) else np.argpartition(-zd_row, top_k - 1)[:top_k]
        w[keep] = _softmax64(zd_row[keep] / T)
    return np.cumsum(w)


SigmaSpec = Callable[[np.random.Generator, int, int], float]


def sigma_const(s: float) -> SigmaSpec:
    return lambda rng, b, B: s


def sigma_halves(lo_half: float, hi_half: float) -> SigmaSpec:
    return lambda rng, b, B: lo_half if b < B // 2 else hi_half


def sigma_uniform(lo: float, hi: float) -> SigmaSpec:
    return lambda rng, b, B: float(rng.uniform(lo, hi))


def _workers() -> int:
    return max(1, min(16, os.cpu_count() or 1))


def make_chain(B: int, K: int, V: int, *, dtype: int, temperature: float, top_k: int,
               sigma: SigmaSpec, config_id: int, seed: int,
               threads: Optional[int] = None, top_p: float = 1.0) -> ChainInputs:
    """Draw one chain-verification input set (see the module docstring for the recipe)."""
    log_rank = _log_rank_table(V)
    logits = np.empty((B, K + 1, V), dtype=np.uint16 if dtype == DTYPE_BF16 else np.float32)
    q = np.empty((B, K, V), dtype=np.float32)
    x = np.empty((B, K), dtype=np.int32)
    u = np.empty((B, K + 1), dtype=np.float32)
    sig = np.empty(B, dtype=np.float64)

    def one(b: int) -> None:
        rng = np.random.default_rng([config_id, seed, b])
        z = _target_rows(rng, K + 1, V, log_rank)
        nd = rng.standard_normal((K, V), dtype=np.float32)
        s = sigma(rng, b, B)
        sig[b] = s
        zd = z[:K].astype(np.float64) + s * nd.astype(np.float64)
        q[b] = _softmax64(zd).astype(np.float32)
        ud = rng.random(K)
        for k in range(K):
            cdf = _draft_sampler_cdf(zd[k], temperature, top_k, top_p)
            x[b, k] = min(int(np.searchsorted(cdf, ud[k] * cdf[-1], side="right")), V - 1)
        u[b] = rng.random(K + 1, dtype=np.float32)
        logits[b] = f32_to_bf16_bits(z) if dtype == DTYPE_BF16 else z

    with ThreadPoolExecutor(threads or _workers()) as ex:
        list(ex.map(one, range(B)))
    return ChainInputs(B, K, V, dtype, float(temperature), int(top_k), logits, q, x, u, sig)


def make_tree(B: int, V: int, *, parents: np.ndarray = EAGLE_TREE_PARENTS, dtype: int = DTYPE_BF16,
              sigma: float = 0.5, config_id: int, seed: int, threads: Optional[int] = None) -> TreeInputs:
    """Draw one greedy tree-verification input set (node tokens from the parent's draft logits)."""
    parents = np.ascontiguousarray(parents, dtype=np.int32)
    N = parents.shape[0]
    log_rank = _log_rank_table(V)
    logits = np.empty((B, N, V), dtype=np.uint16 if dtype == DTYPE_BF16 else np.float32)
    tok = np.full((B, N), -1, dtype=np.int32)
    children = [[c for c in range(N) if parents[c] == p] for p in range(N)]

    def one(b: int) -> None:
        rng = np.random.default_rng([config_id, seed, b])
        z = _target_rows(rng, N, V, log_rank)
        nd = rng.standard_normal((N, V), dtype=np.float32)
        for p in range(N):
            if not children[p]:
                continue
            zd = z[p].astype(np.float64) + sigma * nd[p].astype(np.float64)
            best = np.argsort(-zd, kind="stable")[:len(children[p])]
            for r, c in enumerate(children[p]):
                tok[b, c] = best[r]
        logits[b] = f32_to_bf16_bits(z) if dtype == DTYPE_BF16 else z

    with ThreadPoolExecutor(threads or _workers()) as ex:
        list(ex.map(one, range(B)))
    return TreeInputs(B, N, V, dtype, logits, tok, parents)


@dataclasses.dataclass
class SampledTreeInputs:
    """Inputs of one batched sampling tree verification call."""
    B: int
    N: int
    V: int
    dtype: int
    temperature: float
    top_k: int
    logits: np.ndarray         # [B, N, V] uint16 (bf16 bits) or float32
    draft_probs: np.ndarray    # [B, N, V] float32, row n: the draft distribution at node n
    node_tokens: np.ndarray    # [B, N] int32 (entry 0, the root, is -1)
    uniforms: np.ndarray       # [B, N] float32: u[n] tests node n, u[0] drives the final draw
    parents: np.ndarray        # [N] int32

    def logits_f32(self) -> np.ndarray:
        return bf16_bits_to_f32(self.logits) if self.dtype == DTYPE_BF16 else self.logits


def make_tree_sampled(B: int, V: int, *, parents: np.ndarray = EAGLE_TREE_PARENTS, dtype: int = DTYPE_BF16,
                      temperature: float = 1.0, top_k: int = 0, sigma: float = 0.5, config_id: int,
                      seed: int, threads: Optional[int] = None) -> SampledTreeInputs:
    """Draw one sampling tree-verification input set (children drawn independently from
    the draft model's distribution at their parent)."""
    parents = np.ascontiguousarray(parents, dtype=np.int32)
    N = parents.shape[0]
    log_rank = _log_rank_table(V)
    logits = np.empty((B, N, V), dtype=np.uint16 if dtype == DTYPE_BF16 else np.float32)
    q = np.empty((B, N, V), dtype=np.float32)
    tok = np.full((B, N), -1, dtype=np.int32)
    u = np.empty((B, N), dtype=np.float32)
    children = [[c for c in range(N) if parents[c] == p] for p in range(N)]

    def one(b: int) -> None:
        rng = np.random.default_rng([config_id, seed, b])
        z = _target_rows(rng, N, V, log_rank)
        nd = rng.standard_normal((N, V), dtype=np.float32)
        zd = z.astype(np.float64) + sigma * nd.astype(np.float64)
        q[b] = _softmax64(zd).astype(np.float32)
        for p in range(N):
            if not children[p]:
                continue
            cdf = _draft_sampler_cdf(zd[p], temperature, top_k)
            ud = rng.random(len(children[p]))
            for r, c in enumerate(children[p]):
                tok[b, c] = min(int(np.searchsorted(cdf, ud[r] * cdf[-1], side="right")), V - 1)
        u[b] = rng.random(N, dtype=np.float32)
        logits[b] = f32_to_bf16_bits(z) if dtype == DTYPE_BF16 else z

    with ThreadPoolExecutor(threads or _workers()) as ex:
        list(ex.map(one, range(B)))
    return SampledTreeInputs(B, N, V, dtype, float(temperature), int(top_k), logits, q, tok, u, parents)


@dataclasses.dataclass
class ExpandInputs:
    """Inputs of one EAGLE-2 expansion layer."""
    B: int
    E: int
    V: int
    top_k: int
    k_next: int
    draft_probs: np.ndarray    # [B, E, V] float32
    node_values: np.ndarray    # [B, E] float32


@dataclasses.dataclass
class RerankInputs:
    """A batch of candidate draft trees for EAGLE-2 reranking (root excluded)."""
    B: int
    M: int
    m: int
    parents: np.ndarray        # [B, M] int32, -1 = child of the root, else < own index
    values: np.ndarray         # [B, M] float32


def make_expand(B: int, E: int, V: int, *, top_k: int, k_next: int, sigma: float = 0.5, config_id: int,
                seed: int, threads: Optional[int] = None) -> ExpandInputs:
    """Draw one expansion-layer input set (see the module docstring)."""
    log_rank = _log_rank_table(V)
    q = np.empty((B, E, V), dtype=np.float32)
    nv = np.empty((B, E), dtype=np.float32)

    def one(b: int) -> None:
        rng = np.random.default_rng([config_id, seed, b])
        z = _target_rows(rng, E, V, log_rank)
        nd = rng.standard_normal((E, V), dtype=np.float32)
        q[b] = _softmax64(z.astype(np.float64) + sigma * nd.astype(np.float64)).astype(np.float32)
        nv[b] = np.sort(rng.uniform(0.05, 1.0, E))[::-1].astype(np.float32)

    with ThreadPoolExecutor(threads or _workers()) as ex:
        list(ex.map(one, range(B)))
    return ExpandInputs(B, E, V, int(top_k), int(k_next), q, nv)


def make_rerank(B: int, *, k: int, depth: int, m: int, config_id: int, seed: int) -> RerankInputs:
    """Draw B layered candidate trees of k children per expanded node (see the module docstring)."""
    M = k + (depth - 1) * k * k
    par = np.empty((B, M), dtype=np.int32)
    val = np.empty((B, M), dtype=np.float32)
    for b in range(B):
        rng = np.random.default_rng([config_id, seed, b])
        coarse = b % 4 == 3

        def conf(n):
            if coarse:
                return (rng.integers(1, 5, n) / 4.0).astype(np.float32)
            return rng.uniform(1e-3, 1.0, n).astype(np.float32)

        par[b, :k] = -1
        val[b, :k] = conf(k)
        layer = list(range(k))
        nxt = k
        for _ in range(depth - 1):
            picked = rng.choice(layer, size=k, replace=False)
            new = []
            for p in picked:
                c = conf(k)
                for j in range(k):
                    par[b, nxt] = p
                    val[b, nxt] = np.float32(val[b, p]) * c[j]
                    new.append(nxt)
                    nxt += 1
            layer = new
    return RerankInputs(B, M, int(m), par, val)


@dataclasses.dataclass
class KVCommitInputs:
    """A KV cache holding each batch row's prefix and its N tree nodes, and the accepted paths."""
    B: int
    planes: int
    S: int
    row: int                   # elements (bf16 bits, uint16) per row
    N: int
    kv: np.ndarray             # [planes, B, S, row] uint16
    prefix: np.ndarray         # [B] int32: where node 0 sits
    path: np.ndarray           # [B, D+1] int32: node ids root..n*, -1 padded
    accept_len: np.ndarray     # [B] int32: depth of n*


def make_kv_commit(B: int, *, planes: int, row: int, parents: np.ndarray = EAGLE_TREE_PARENTS, max_prefix: int,
                   config_id: int, seed: int) -> KVCommitInputs:
    """Random cache contents; per batch row a prefix length in [0, max_prefix] and the path to a
    random node of the tree (deeper nodes about as likely as shallow ones)."""
    rng = np.random.default_rng([config_id, seed])
    parents = np.asarray(parents, dtype=np.int32)
    N = parents.shape[0]
    depth = np.zeros(N, np.int64)
    for n in range(1, N):
        depth[n] = depth[parents[n]] + 1
    D = int(depth.max())
    S = max_prefix + N
    kv = rng.integers(0, 1 << 16, (planes, B, S, row), dtype=np.uint16)
    prefix = rng.integers(0, max_prefix + 1, B).astype(np.int32)
    path = np.full((B, D + 1), -1, np.int32)
    alen = np.empty(B, np.int32)
    for b in range(B):
        d = int(rng.integers(0, D + 1))
        cands = np.flatnonzero(depth == d)
        n = int(rng.choice(cands))
        alen[b] = d
        for t in range(d, -1, -1):
            path[b, t] = n
            n = parents[n] if n > 0 else 0
    return KVCommitInputs(B, planes, S, row, N, kv, prefix, path, alen)


@dataclasses.dataclass
class LMHeadInputs:
    """A chain verification fed by hidden states and LM-head weights instead of logits."""
    B: int
    K: int
    V: int
    H: int
    temperature: float
    top_k: int
    hidden: np.ndarray         # [B, K+1, H] uint16 (bf16 bits): last hidden states of the target
    weight: np.ndarray         # [V, H] uint16 (bf16 bits): the LM head (no bias)
    draft_probs: np.ndarray    # [B, K, V] float32
    draft_tokens: np.ndarray   # [B, K] int32
    uniforms: np.ndarray       # [B, K+1] float32


def make_lm_head(B: int, K: int, V: int, H: int, *, temperature: float, top_k: int, sigma: SigmaSpec,
                 config_id: int, seed: int, threads: Optional[int] = None) -> LMHeadInputs:
    """Hidden states and head weights whose logits follow the chain recipe in shape.

    The head is drawn once per (config, seed): a permutation ``rank`` of 1..V, and row v of
    W = [g_v * 3/sqrt(H-1), -1.1*ln(rank_v)] with g_v ~ N(0, I) in H-1 dimensions; hidden
    states are [n, 1] with n ~ N(0, I), so that a logit is 3*N(0,1) - 1.1*ln(rank) as in
    step 2 of the chain recipe (the Zipf-like prior is the model's, shared by every row).
    Both are stored as bfloat16.  The draft sees the target's logits (float32 products of
    the rounded operands, in numpy) through noise as in step 3; its tokens and the
    verification uniforms follow steps 5 and 6."""
    rng0 = np.random.default_rng([config_id, seed, 1 << 30])
    rank = rng0.permutation(V) + 1
    bias = (-1.1 * np.log(rank.astype(np.float64))).astype(np.float32)
    weight = np.empty((V, H), dtype=np.uint16)
    rows = 8192
    scale = np.float32(3.0 / math.sqrt(H - 1))

    def wchunk(c: int) -> None:
        r = np.random.default_rng([config_id, seed, 1 << 30, c])
        v0, v1 = c * rows, min(V, (c + 1) * rows)
        g = r.standard_normal((v1 - v0, H - 1), dtype=np.float32) * scale
        weight[v0:v1, :H - 1] = f32_to_bf16_bits(g)
        weight[v0:v1, H - 1] = f32_to_bf16_bits(bias[v0:v1])

    with ThreadPoolExecutor(threads or _workers()) as ex:
        list(ex.map(wchunk, range((V + rows - 1) // rows)))
    hidden = np.empty((B, K + 1, H), dtype=np.uint16)
    q = np.empty((B, K, V), dtype=np.float32)
    x = np.empty((B, K), dtype=np.int32)
    u = np.empty((B, K + 1), dtype=np.float32)
    wf = bf16_bits_to_f32(weight)

    def one(b: int) -> None:
        rng = np.random.default_rng([config_id, seed, b])
        h = np.ones((K + 1, H), dtype=np.float32)
        h[:, :H - 1] = rng.standard_normal((K + 1, H - 1), dtype=np.float32)
        hb = f32_to_bf16_bits(h)
        hidden[b] = hb
        z = bf16_bits_to_f32(hb)[:K] @ wf.T
        nd = rng.standard_normal((K, V), dtype=np.float32)
        s = sigma(rng, b, B)
        zd = z.astype(np.float64) + s * nd.astype(np.float64)
        q[b] = _softmax64(zd).astype(np.float32)
        ud = rng.random(K)
        for k in range(K):
            cdf = _draft_sampler_cdf(zd[k], temperature, top_k)
            x[b, k] = min(int(np.searchsorted(cdf, ud[k] * cdf[-1], side="right")), V - 1)
        u[b] = rng.random(K + 1, dtype=np.float32)

    with ThreadPoolExecutor(threads or _workers()) as ex:
        list(ex.map(one, range(B)))
    return LMHeadInputs(B, K, V, H, float(temperature), int(top_k), hidden, weight, q, x, u)


# The workloads, by index.  Each entry builds inputs for a seed, with
# optional size overrides used by the smaller parity cases.
CONFIG_NAMES = {
    0: "chain B=1 K=4 V=1000 fp32 T=1",
    1: "chain B=8 K=5 V=32000 bf16 T=1",
    2: "chain B=64 K=7 V=128256 bf16 T=0.7 top_k=50",
    3: "tree-greedy B=32 N=27 V=32000 bf16",
    4: "chain B=512 K=8 V=128256 bf16 T=1",
    5: "tree-sample B=32 N=27 V=32000 bf16 T=1",
    6: "eagle2-expand B=64 E=10 V=128256 top_k=10 k_next=10",
    7: "kv-commit B=64 planes=64 row=2KiB N=27",
    8: "accept-rate B=512 K=8 V=128256 bf16 T=1 (the inputs of workload 4)",
    9: "lm-head-fused chain B=64 K=7 V=128256 H=4096 bf16 T=0.7 top_k=50",
}


def config(cid: int, seed: int = 0, *, B: Optional[int] = None, K: Optional[int] = None,
           V: Optional[int] = None, threads: Optional[int] = None):
    """Inputs for workload ``cid`` (0..10), optionally with smaller B/K/V (K: expanded nodes for 6)."""
    if cid == 0:
        return make_chain(B or 1, K or 4, V or 1000, dtype=DTYPE_F32, temperature=1.0, top_k=0,
                          sigma=sigma_const(0.5), config_id=0, seed=seed, threads=threads)
    if cid == 1:
        return make_chain(B or 8, K or 5, V or 32000, dtype=DTYPE_BF16, temperature=1.0, top_k=0,
                          sigma=sigma_const(0.5), config_id=1, seed=seed, threads=threads)
    if cid == 2:
        return make_chain(B or 64, K or 7, V or 128256, dtype=DTYPE_BF16, temperature=0.7, top_k=50,
                          sigma=sigma_halves(0.3, 1.0), config_id=2, seed=seed, threads=threads)
    if cid == 3:
        return make_tree(B or 32, V or 32000, dtype=DTYPE_BF16, sigma=0.5, config_id=3, seed=seed,
                         threads=threads)
    if cid in (4, 8):
        return make_chain(B or 512, K or 8, V or 128256, dtype=DTYPE_BF16, temperature=1.0, top_k=0,
                          sigma=sigma_uniform(0.2, 1.5), config_id=4, seed=seed, threads=threads)
    if cid == 5:
        return make_tree_sampled(B or 32, V or 32000, dtype=DTYPE_BF16, temperature=1.0, top_k=0,
                                 sigma=0.5, config_id=5, seed=seed, threads=threads)
    if cid == 10:
        # the benchmark's shape with the nucleus on whole rows: drafts from the draft's own nucleus
        return make_chain(B or 64, K or 7, V or 128256, dtype=DTYPE_BF16, temperature=0.7, top_k=0,
                          sigma=sigma_halves(0.3, 1.0), config_id=10, seed=seed, threads=threads, top_p=0.9)
    if cid == 9:
        return make_lm_head(B or 64, K or 7, V or 128256, 4096, temperature=0.7, top_k=50,
                            sigma=sigma_halves(0.3, 1.0), config_id=9, seed=seed, threads=threads)
    if cid == 7:
        return make_kv_commit(B or 64, planes=64, row=1024, max_prefix=16, config_id=7, seed=seed)
    if cid == 6:
        return make_expand(B or 64, K or 10, V or 128256, top_k=10, k_next=10, sigma=0.5, config_id=6, seed=seed,
                           threads=threads)
    raise ValueError(f"unknown workload {cid}")


def with_transform(ci: ChainInputs, *, temperature: float, top_k: int) -> ChainInputs:
    """Same arrays, different verification transform (draft tokens are kept)."""
    return dataclasses.replace(ci, temperature=float(temperature), top_k=int(top_k))


def draws_fixed_uniforms(B: int, K: int, values: Sequence[float]) -> np.ndarray:
    """A [B, K+1] float32 uniform array filled cyclically from ``values`` (edge-case helper)."""
    v = np.resize(np.asarray(values, dtype=np.float32), B * (K + 1))
    return v.reshape(B, K + 1)
