"""Exact output laws of a chain verifier, measured by treating it as a black box.

With the drafted tokens fixed, the verifier's output is a step function of the
uniforms: test k flips at u_k = min(1, ratio_k) and the final draw is a
non-decreasing step function of u_K.  Bisection over the float32 uniforms
therefore recovers every threshold and every cell of the final draw, and
summing over all drafted sequences (weighted by the proposal law) gives the
exact law of what the verifier emits -- to the float32 grid spacing (<= 6e-8).
Nothing here restates the verification arithmetic.
"""

from __future__ import annotations

import itertools

import numpy as np

_ONE_BITS = 0x3F800000  # float32 1.0


def bisect_first_false(pred, n: int) -> np.ndarray:
    """For n monotone predicates on float32 u in [0,1) (True below a threshold,
    False from it on), return the threshold as float64 (1.0 if never False)."""
    lo = np.zeros(n, np.int64)
    hi = np.full(n, _ONE_BITS, np.int64)
    while np.any(lo < hi):
        active = lo < hi
        mid = (lo + hi) // 2
        f = mid.astype(np.uint32).view(np.float32)
        ok = pred(f)
        lo = np.where(active & ok, mid + 1, lo)
        hi = np.where(active & ~ok, mid, hi)
    return lo.astype(np.uint32).view(np.float32).astype(np.float64)


def chain_law(run, K: int, V: int, proposal: np.ndarray):
    """Exact law of a K-position chain verifier.

    run(tokens[S,K], u[S,K+1]) -> (accept_len[S], out_tokens[S,K+1]) is the
    verifier on S copies of one input row.  proposal [K,V] is the law of the
    drafted token at each position.  Returns (emit [K+1,V], reach [K+2]) with
    emit[k,t] = P(accept_len >= k and the token at position k is t) and
    reach[k] = P(accept_len >= k) (reach[K+1] = 0).
    """
    seqs = np.array(list(itertools.product(range(V), repeat=K)), dtype=np.int32)
    w = np.prod(proposal[np.arange(K)[None, :], seqs], axis=1)
    seqs, w = seqs[w > 0], w[w > 0]
    S = len(seqs)
    rows = np.arange(S)

    def call(u):
        return run(seqs, u.astype(np.float32))

    thr = np.zeros((S, K))
    for k in range(K):
        def pred(f, k=k):
            u = np.zeros((S, K + 1), np.float32)
            u[:, k] = f
            al, _ = call(u)
            return al > k
        thr[:, k] = bisect_first_false(pred, S)

    def draw_law(k, u_base):
        law = np.zeros((S, V))
        prev = np.zeros(S)
        u = u_base.copy()
        u[:, K] = 0.0
        _, tok = call(u)
        cur = tok[:, k].copy()
        for _ in range(V + 1):
            def pred(f):
                uu = u_base.copy()
                uu[:, K] = f
                _, t = call(uu)
                return t[:, k] <= cur
            t = bisect_first_false(pred, S)
            valid = cur >= 0
            law[rows[valid], cur[valid]] += (t - prev)[valid]
            prev = t
            done = t >= 1.0
            if np.all(done):
                break
            uu = u_base.copy()
            uu[:, K] = np.where(done, 0.0, t)
            _, tt = call(uu)
            cur = np.where(done, cur, tt[:, k])
        return law

    emit = np.zeros((K + 1, V))
    reach = np.zeros(K + 2)
    prefix = np.ones(S)
    for k in range(K + 1):
        reach[k] = np.sum(w * prefix)
        u_base = np.zeros((S, K + 1), np.float32)
        if k < K:
            u_base[:, k] = np.nextafter(np.float32(1), np.float32(0))
            rej = draw_law(k, u_base)
            acc = np.zeros((S, V))
            acc[rows, seqs[:, k]] = thr[:, k]
            emit[k] = np.sum((w * prefix)[:, None] * (acc + (1.0 - thr[:, k])[:, None] * rej), axis=0)
            prefix = prefix * thr[:, k]
        else:
            emit[k] = np.sum((w * prefix)[:, None] * draw_law(k, u_base), axis=0)
    return emit, reach


def _step_law(tok_of, S: int, V: int) -> np.ndarray:
    """Law of a token that is a non-decreasing step function of one float32 uniform:
    tok_of(f[S]) -> tokens[S]; returns [S, V] cell lengths."""
    rows = np.arange(S)
    law = np.zeros((S, V))
    prev = np.zeros(S)
    cur = tok_of(np.zeros(S, np.float32)).copy()
    for _ in range(V + 1):
        t = bisect_first_false(lambda f: tok_of(f) <= cur, S)
        valid = cur >= 0
        law[rows[valid], cur[valid]] += (t - prev)[valid]
        prev = t
        done = t >= 1.0
        if np.all(done):
            break
        cur = np.where(done, cur, tok_of(np.where(done, 0.0, t).astype(np.float32)))
    return law


def tree_law(run, parents, V: int, proposal: np.ndarray):
    """Exact law of a sampling tree verifier, treated as a black box.

    run(tokens[S,N], u[S,N]) -> (accept_len[S], path[S,D+1], out_tokens[S,D+1]) is the
    verifier on S copies of one input row, u[:, n] (n >= 1) the uniform of node n's test
    and u[:, 0] that of the final draw.  The token of node n is drawn from
    proposal[parents[n]] independently of the others.  For fixed tokens the test of
    node n accepts below a threshold in u[:, n] and the final draw is a step function
    of u[:, 0]; bisection recovers both, node by node from the root, with the
    uniforms of earlier siblings set to reject and those of ancestors to accept.
    Returns (reach [N], law [N, V]): reach[n] = P(the accepted path passes node n),
    law[n, t] = P(it passes n and the token emitted after n is t).
    """
    par = np.asarray(parents)
    N = par.shape[0]
    depth = np.zeros(N, np.int64)
    for n in range(1, N):
        depth[n] = depth[par[n]] + 1
    free = list(range(1, N))
    seqs = np.zeros((V ** len(free), N), np.int32)
    if free:
        seqs[:, 1:] = np.array(list(itertools.product(range(V), repeat=len(free))), np.int32)
    w = np.ones(seqs.shape[0])
    for n in free:
        w = w * proposal[par[n], seqs[:, n]]
    keep = w > 0
    seqs, w = seqs[keep], w[keep]
    S = seqs.shape[0]
    rows = np.arange(S)
    reach = np.zeros(N)
    law = np.zeros((N, V))
    below_one = np.nextafter(np.float32(1), np.float32(0))

    def call(u):
        return run(seqs, u.astype(np.float32))

    def explore(c, ub, wc):
        reach[c] += wc.sum()
        ub = ub.copy()
        for n in [m for m in range(N) if par[m] == c]:
            def accepted(f, n=n):
                uu = ub.copy()
                uu[:, n] = f
                return call(uu)[1][:, depth[n]] == n
            thr = bisect_first_false(accepted, S)
            law[c] += np.bincount(seqs[:, n], weights=wc * thr, minlength=V)
            ua = ub.copy()
            ua[:, n] = 0.0
            explore(n, ua, wc * thr)
            ub[:, n] = np.minimum(thr, below_one)
            wc = wc * (1.0 - thr)

        def tok_of(f):
            uu = ub.copy()
            uu[:, 0] = f
            return call(uu)[2][:, depth[c]]
        law[c] += np.sum(wc[:, None] * _step_law(tok_of, S, V), axis=0)

    explore(0, np.zeros((S, N), np.float32), w)
    return reach, law
