"""Pins of the oracle's decision margins, its draw diagnostics and its greedy acceptance rate.

The GPU parity rule admits a token or accept-length disagreement only where the
oracle's own margin is below 1e-5, so the margins must be right on their own:
- m_test[k] = |u_k - min(1, p'_k(x_k) / q'_k(x_k))| for every test performed;
- m_draw = the distance of u_K * S to the nearest edge of the chosen CDF cell, over S;
- py = r(y) / S, the drawn token's probability under the final-draw distribution.

Each is checked against a hand derivation from the two-token example of
"064 · 投机解码" section 二, and against a separate numpy walk (numpy's stable
sort and scipy's softmax for the transforms, numpy's cumsum and searchsorted for
the inverse CDF) on inputs whose residual mass S is far from 1 and whose CDF cells
differ in size by orders of magnitude.  Planted slips (a draw margin not divided
by S, a test margin measured against the ratio instead of min(1, ratio)) must fail
those checks.  The greedy acceptance rate (temperature 0: 1 if the two rows'
argmaxes agree) is checked against numpy's argmax (first occurrence) with ties.
"""

import math

import numpy as np
import pytest
import scipy.special

from test_oracle_pins import lib_draft, lib_target


def numpy_walk(z, q, x, u, T, top_k):
    """One batch row's chain verification from library routines: (tokens, accept_len,
    pk, qk, m_test, S, py, m_draw).  Follows 064 · 投机解码 section 三 (test left to right,
    stop at the first rejection, residual or bonus draw) with the repository's readings
    (u_k drives test k, u_K the draw; index-ascending inverse CDF, strict u*S < C_i)."""
    K1, V = z.shape
    K = K1 - 1
    pk = np.full(K, np.nan)
    qk = np.full(K, np.nan)
    m_test = np.full(K, np.nan)
    j = K
    for k in range(K):
        p = lib_target(z[k], T, top_k)
        qq = lib_draft(q[k], T, top_k)
        a, c = p[x[k]], qq[x[k]]
        ratio = a / c if c > 0 else (math.inf if a > 0 else 0.0)
        thr = min(1.0, ratio)
        pk[k], qk[k] = a, c
        m_test[k] = abs(float(u[k]) - thr)
        if not float(u[k]) < thr:
            j = k
            break
    pj = lib_target(z[j], T, top_k)
    if j < K:
        r = np.maximum(0.0, pj - lib_draft(q[j], T, top_k))
        if not r.sum() > 0:
            r = pj
    else:
        r = pj
    C = np.cumsum(r)               # sequential, index-ascending inclusive prefix sums
    S = C[-1]
    t = float(u[K]) * S
    y = int(np.searchsorted(C, t, side="right"))      # first i with t < C_i
    assert y < V, "rounding fallback not expected on these inputs"
    lo = C[y - 1] if y > 0 else 0.0
    m_draw = min(t - lo, C[y] - t) / S
    tokens = np.full(K + 1, -1)
    tokens[:j] = x[:j]
    tokens[j] = y
    return tokens, j, pk, qk, m_test, S, r[y] / S, m_draw


def _skewed_inputs(seed, B, K, V):
    """Logits with a wide spread (cells of the CDF from ~1e-9 to ~0.3) and a draft far
    enough from the target that the residual mass S = 1 - alpha lies well below 1."""
    rng = np.random.default_rng([91, seed])
    z = (4.0 * rng.standard_normal((B, K + 1, V))).astype(np.float32)
    q = scipy.special.softmax(z[:, :K].astype(np.float64) + 1.5 * rng.standard_normal((B, K, V)),
                              axis=2).astype(np.float32)
    return rng, z, q


def _draft_tokens(rng, q, T, top_k):
    B, K, V = q.shape
    return np.array([[rng.choice(V, p=lib_draft(q[b, k], T, top_k) / lib_draft(q[b, k], T, top_k).sum())
                      for k in range(K)] for b in range(B)], np.int32)


CASES = [(1.0, 0), (0.7, 0), (1.3, 0), (0.7, 20), (1.0, 5)]


@pytest.mark.parametrize("T,top_k", CASES)
def test_margins_match_a_numpy_walk(orc, T, top_k):
    B, K, V = 48, 4, 300
    rng, z, q = _skewed_inputs(int(T * 10) + top_k, B, K, V)
    x = _draft_tokens(rng, q, T, top_k)
    u = rng.random((B, K + 1), dtype=np.float32)
    o = orc.verify_chain(z, orc.F32, q, x, u, T, top_k)
    residual_rows = 0
    for b in range(B):
        tok, j, pk, qk, mt, S, py, md = numpy_walk(z[b], q[b], x[b], u[b], T, top_k)
        assert o["accept_len"][b] == j and np.array_equal(o["tokens"][b], tok), b
        np.testing.assert_allclose(o["pk"][b], pk, rtol=0, atol=1e-13)
        np.testing.assert_allclose(o["qk"][b], qk, rtol=0, atol=1e-13)
        np.testing.assert_allclose(o["m_test"][b], mt, rtol=0, atol=1e-13)
        assert o["S"][b] == pytest.approx(S, rel=1e-12, abs=0)
        assert o["py"][b] == pytest.approx(py, rel=1e-10, abs=1e-15)
        assert o["m_draw"][b] == pytest.approx(md, rel=1e-8, abs=1e-13)
        residual_rows += j < K
    assert residual_rows > 10          # the draws from a residual (S < 1) are exercised


def test_margin_inputs_have_unequal_cells_and_small_masses(orc):
    """The inputs above do what the comparison needs: residual masses well below 1 and
    CDF cells spanning many orders of magnitude (a margin slip by a factor S shows)."""
    B, K, V = 48, 4, 300
    rng, z, q = _skewed_inputs(10, B, K, V)
    x = _draft_tokens(rng, q, 1.0, 0)
    u = rng.random((B, K + 1), dtype=np.float32)
    o = orc.verify_chain(z, orc.F32, q, x, u, 1.0, 0)
    S = o["S"][o["accept_len"] < K]
    assert np.median(S) < 0.7 and S.min() < 0.4
    p = lib_target(z[0, 0], 1.0, 0)
    assert p.max() / p[p > 0].min() > 1e6


def test_margins_two_token_example():
    """Hand derivation on 064 · 投机解码 section 二's example, p = (0.6, 0.4), q = (0.8, 0.2):

    - draft token A (index 0), u_0 = 0.8: ratio 0.6/0.8 = 0.75 < u_0, so the test rejects
      with margin |0.8 - 0.75| = 0.05; the residual is (0, 0.2), S = 0.2; u_1 = 0.3 puts
      u_1*S = 0.06 in token B's cell [0, 0.2): margin min(0.06, 0.14)/0.2 = 0.3, py = 1;
    - draft token B (index 1), u_0 = 0.25: ratio 2, min(1, 2) = 1, margin 0.75, accepted;
      the bonus is drawn from p with S = 1; u_1 = 0.5 falls in A's cell [0, 0.6): margin
      min(0.5, 0.1) = 0.1, py = 0.6.
    The float32 inputs (log p as float32 logits, q and u as float32) move these values by
    at most a few 1e-8."""
    import oracle as orc
    z = np.log(np.array([[0.6, 0.4], [0.6, 0.4]])).astype(np.float32)
    q = np.array([[[0.8, 0.2]]], np.float32)
    cases = [(0, (0.8, 0.3), dict(accept_len=0, tok=[1, -1], m_test=0.05, S=0.2, py=1.0, m_draw=0.3)),
             (1, (0.25, 0.5), dict(accept_len=1, tok=[1, 0], m_test=0.75, S=1.0, py=0.6, m_draw=0.1))]
    for x, u, e in cases:
        o = orc.verify_chain(z[None], orc.F32, q, np.array([[x]], np.int32), np.array([u], np.float32), 1.0, 0)
        assert o["accept_len"][0] == e["accept_len"]
        assert o["tokens"][0].tolist() == e["tok"]
        assert o["m_test"][0, 0] == pytest.approx(e["m_test"], abs=1e-7)
        assert o["S"][0] == pytest.approx(e["S"], abs=1e-7)
        assert o["py"][0] == pytest.approx(e["py"], abs=1e-7)
        assert o["m_draw"][0] == pytest.approx(e["m_draw"], abs=1e-6)


@pytest.mark.parametrize("variant,field", [(5, "m_draw"), (6, "m_test")])
def test_planted_margin_slips_are_caught(orc, variant, field):
    """A draw margin left undivided by S (5), or a test margin measured against the raw
    ratio (6), disagrees with the numpy walk."""
    B, K, V = 48, 4, 300
    rng, z, q = _skewed_inputs(17, B, K, V)
    x = _draft_tokens(rng, q, 1.0, 0)
    u = rng.random((B, K + 1), dtype=np.float32)
    orc.set_variant(variant)
    try:
        o = orc.verify_chain(z, orc.F32, q, x, u, 1.0, 0)
    finally:
        orc.set_variant(0)
    worst = 0.0
    for b in range(B):
        _, _, _, _, mt, _, _, md = numpy_walk(z[b], q[b], x[b], u[b], 1.0, 0)
        want = md if field == "m_draw" else mt
        got = o[field][b]
        ok = ~np.isnan(np.atleast_1d(want))
        worst = max(worst, float(np.max(np.abs(np.atleast_1d(got)[ok] - np.atleast_1d(want)[ok]))))
    assert worst > 1e-3


def test_greedy_accept_rate_matches_numpy_argmax(orc):
    """Temperature 0: alpha = 1 when the first-occurrence argmaxes of the target and draft
    rows agree, else 0; NaN in either row gives NaN."""
    rng = np.random.default_rng(93)
    B, K, V = 40, 3, 64
    z = np.round(2 * rng.standard_normal((B, K + 1, V))).astype(np.float32)   # many exact ties
    q = (np.round(4 * rng.random((B, K, V))) / 8).astype(np.float32)            # ties in the draft too
    # rows where both maxima are tied and the first occurrences agree or differ
    for b in range(0, B, 4):
        z[b, 0, :] = 0.0
        z[b, 0, [5, 9]] = 3.0
        q[b, 0, :] = 0.0
        q[b, 0, [5 if b % 8 == 0 else 9, 12]] = 0.5
    z[1, 1, 7] = np.nan
    q[2, 2, 3] = np.nan
    a = orc.accept_rate(z, orc.F32, q, 0.0, 0)
    matches = 0
    for b in range(B):
        for k in range(K):
            if np.isnan(z[b, k]).any() or np.isnan(q[b, k]).any():
                assert np.isnan(a[b, k])
                continue
            want = 1.0 if int(np.argmax(z[b, k])) == int(np.argmax(q[b, k])) else 0.0
            assert a[b, k] == want, (b, k)
            matches += want == 1.0
    assert 0 < matches < B * K - 2
    # the top-k setting does not change the greedy rule
    assert np.array_equal(orc.accept_rate(z, orc.F32, q, 0.0, 5), a, equal_nan=True)
