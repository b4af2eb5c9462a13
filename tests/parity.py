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
                  rows=None) -> Tally:
    """Compare GPU outputs (numpy) with an oracle result dict for the given batch rows."""
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
            assert np.array_equal(tokens[b, :oa], ot[:oa])
            m = orc["m_draw"][i]
            assert m < MARGIN, f"row {b}: draw differs (gpu {tokens[b, oa]}, oracle {ot[oa]}) at margin {m}"
            t.admissible += 1
        else:
            k = min(ga, oa)
            m = orc["m_test"][i, k]
            assert m < MARGIN, f"row {b}: test {k} differs (gpu len {ga}, oracle {oa}) at margin {m}"
            t.admissible += 1
    return t


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
