"""GPU-vs-oracle comparison rules shared by the parity tests.

Sampled tokens and accept lengths must match the oracle exactly, except
where the oracle's own decision margin is below MARGIN (|u - min(1, ratio)|
for a test, distance of u*S to the chosen cell's edge over S for the draw);
such admissible disagreements are counted and must stay below 1e-4 of the
decisions made.  Probabilities reported by the kernels must agree within
PROB_TOL.  Greedy, tree and index work is bit-exact.
"""

from __future__ import annotations

import dataclasses
import math

import numpy as np

MARGIN = 1e-5
PROB_TOL = 1e-5
ADMISSIBLE_RATE = 1e-4


@dataclasses.dataclass
class Tally:
    decisions: int = 0
    admissible: int = 0
    rows: int = 0

    def add(self, other: "Tally") -> None:
        self.decisions += other.decisions
        self.admissible += other.admissible
        self.rows += other.rows

    def check(self) -> None:
        assert self.admissible <= ADMISSIBLE_RATE * self.decisions, \
            f"{self.admissible} admissible disagreements in {self.decisions} decisions"


def to_torch(arr, device="cuda"):
    import torch
    if arr.dtype == np.uint16:
        return torch.from_numpy(np.ascontiguousarray(arr).view(np.int16)).to(device).view(torch.bfloat16)
    return torch.from_numpy(np.ascontiguousarray(arr)).to(device)


def compare_chain(orc: dict, tokens: np.ndarray, alen: np.ndarray, diag, K: int, greedy: bool = False,
                  rows=None, V=None, draft_tokens=None) -> Tally:
    """Compare GPU outputs (numpy) with an oracle result dict for the given batch rows.
    V and draft_tokens ([B, K], GPU row order), when given, let a row admitted on a
    small margin be checked for range and for the draft tokens it accepted."""
    t = Tally()
    B = alen.shape[0]
    rows = range(B) if rows is None else rows
    for i, b in enumerate(rows):
        oa = int(orc["accept_len"][i])
        ga = int(alen[b])
        t.rows += 1
        if oa < 0 or ga < 0:
            assert oa == ga == -1, f"row {b}: error flag mismatch (oracle {oa}, gpu {ga})"
            assert np.all(tokens[b] == -1)
            continue
        t.decisions += min(oa + 1, K) + 1
        ot = orc["tokens"][i]
        if greedy:
            assert ga == oa and np.array_equal(tokens[b], ot), f"row {b}: greedy mismatch"
            continue
        if diag is not None:
            np.testing.assert_allclose(diag[b, :K], orc["pk"][i], rtol=0, atol=PROB_TOL, err_msg=f"row {b} p'(x)")
            np.testing.assert_allclose(diag[b, K:2 * K], orc["qk"][i], rtol=0, atol=PROB_TOL,
                                       err_msg=f"row {b} q'(x)")
        if ga == oa:
            if np.array_equal(tokens[b], ot):
                if diag is not None:
                    assert abs(diag[b, 2 * K] - orc["S"][i]) <= PROB_TOL, f"row {b} S"
                    assert abs(diag[b, 2 * K + 1] - orc["py"][i]) <= PROB_TOL, f"row {b} p(y)"
                continue
            m = orc["m_draw"][i]
            assert m < MARGIN, f"row {b}: draw differs (gpu {tokens[b, oa]}, oracle {ot[oa]}) at margin {m}"
            t.admissible += 1
        else:
            k = min(ga, oa)
            m = orc["m_test"][i, k]
            assert m < MARGIN, f"row {b}: test {k} differs (gpu len {ga}, oracle {oa}) at margin {m}"
            t.admissible += 1
        _check_admitted_row(tokens[b], ot, ga, oa, V, None if draft_tokens is None else draft_tokens[b], b)
    return t


def _check_admitted_row(gt: np.ndarray, ot: np.ndarray, ga: int, oa: int, V, xb, b: int) -> None:
    """A row whose last decision differs within the margin must still be well formed: the
    accepted draft tokens (those both sides accepted equal the oracle's; all of them equal
    the row's draft tokens when given), one emitted token in [0, V), then -1 padding."""
    k = min(ga, oa)
    assert np.array_equal(gt[:k], ot[:k]), f"row {b}: accepted draft tokens differ"
    if xb is not None:
        assert np.array_equal(gt[:ga], np.asarray(xb)[:ga]), f"row {b}: accepted tokens are not the draft's"
    y = int(gt[ga])
    assert 0 <= y and (V is None or y < V), f"row {b}: emitted token {y} out of range"
    assert np.all(gt[ga + 1:] == -1), f"row {b}: padding after the emitted token"


def oracle_rows(ci, rows):
    """Slice a ChainInputs to the given batch rows (for running the oracle on a sample)."""
    rows = np.asarray(rows)
    return dict(logits=ci.logits[rows], q=ci.draft_probs[rows], x=ci.draft_tokens[rows], u=ci.uniforms[rows])


def run_oracle_chain(orc, ci, rows=None):
    if rows is None:
        return orc.verify_chain(ci.logits, ci.dtype, ci.draft_probs, ci.draft_tokens, ci.uniforms,
                                ci.temperature, ci.top_k)
    s = oracle_rows(ci, rows)
    return orc.verify_chain(s["logits"], ci.dtype, s["q"], s["x"], s["u"], ci.temperature, ci.top_k)


def run_gpu_chain(R, ci, diag=True):
    import torch
    z = to_torch(ci.logits)
    q = to_torch(ci.draft_probs)
    x = to_torch(ci.draft_tokens)
    u = to_torch(ci.uniforms)
    out = R.verify_chain(z, q, x, u, ci.temperature, ci.top_k, diag=diag)
    torch.cuda.synchronize()
    return [o.cpu().numpy() if o is not None else None for o in out] + ([None] if not diag else [])


def nan_equal_close(a, b, tol):
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    assert np.array_equal(np.isnan(a), np.isnan(b)), "NaN pattern differs"
    m = ~np.isnan(a)
    if m.any():
        assert np.max(np.abs(a[m] - b[m])) <= tol, f"max |diff| {np.max(np.abs(a[m] - b[m]))}"


def log_tally(name: str, t: Tally) -> None:
    rate = t.admissible / t.decisions if t.decisions else math.nan
    print(f"[parity] {name}: rows={t.rows} decisions={t.decisions} admissible={t.admissible} rate={rate:.2e}",
          flush=True)
