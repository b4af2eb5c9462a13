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
