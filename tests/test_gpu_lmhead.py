"""Parity of spec_verify_chain_fused (the LM head and the verification in one pass, the
logits kept on the chip) with the oracle, which forms the logits exactly in fp64
(oracle.lm_head_logits) and then verifies as for any chain.

The GPU's logits carry the rounding of fp32 accumulation on the matrix cores: H/16
accumulation steps, each rounding a partial sum of size up to |z|.  Modelled as a
random walk of 2^-24-relative errors, that is about 16 * 6e-8 * 20 = 2e-5 for H = 4096
and |z| <= 20 at six standard deviations, so the tests take EPS_Z = 5e-5 as the logit
tolerance (a CPU emulation of the same accumulation on these inputs stays below 1e-5).
It moves a probability p' = softmax(z/T) by at most 2 * EPS_Z / T relative, which sets:
- a row whose exact top-k boundary (the k-th and (k+1)-th logits; greedy: the first two)
  lies within 2 * EPS_Z may legitimately keep another set: such rows are admitted and
  counted instead of compared;
- p'(x_k) and the draw's mass agree within 1e-5 + 4 * EPS_Z / T (relative to p');
- a differing accept length or token is admitted only where the oracle's decision margin
  is below the same bound, and admitted decisions stay below 1e-3 of all.
"""

import dataclasses

import numpy as np
import pytest

from parity import to_torch
from rejection_sampling_verify_10_amd import workloads as W

pytestmark = pytest.mark.gpu

EPS_Z = 5e-5
ADMIT_RATE = 1e-3


@pytest.fixture(scope="module")
def R():
    import torch
    import rejection_sampling_verify_10_amd as R
    assert torch.cuda.is_available(), "GPU test without a GPU"
    R.lib()
    return R


def boundary_gap(z64_row, kk):
    """Gap between the kk-th and (kk+1)-th largest exact logits of a row."""
    s = np.sort(z64_row)[::-1]
    return s[kk - 1] - s[kk] if kk < s.shape[0] else np.inf


def run_fused(R, li, rows=None):
    import torch
    z, w = to_torch(li.hidden), to_torch(li.weight)
    q, x, u = to_torch(li.draft_probs), to_torch(li.draft_tokens), to_torch(li.uniforms)
    tok, alen, dg = R.verify_chain_fused(z, w, q, x, u, li.temperature, li.top_k, diag=True)
    torch.cuda.synchronize()
    return tok.cpu().numpy(), alen.cpu().numpy(), dg.cpu().numpy()


def check(R, orc, li, name, rows=None):
    print(f"[case] fused {name}: B={li.B} K={li.K} V={li.V} H={li.H} T={li.temperature} top_k={li.top_k}",
          flush=True)
    tok, alen, dg = run_fused(R, li)
    rows = np.arange(li.B) if rows is None else np.asarray(rows)
    z64 = orc.lm_head_logits(li.hidden[rows], li.weight)
    o = orc.verify_chain(z64, orc.F64, li.draft_probs[rows], li.draft_tokens[rows], li.uniforms[rows],
                         li.temperature, li.top_k)
    T, K = li.temperature, li.K
    greedy = T == 0.0
    kk = 1 if greedy else li.top_k
    tol = 1e-5 + (0.0 if greedy else 4 * EPS_Z / T)
    decisions = admitted = near_rows = 0
    for i, b in enumerate(rows):
        oa, ga = int(o["accept_len"][i]), int(alen[b])
        if oa < 0 or ga < 0:
            assert oa == ga == -1, f"{name} row {b}: error flag (oracle {oa}, gpu {ga})"
            assert np.all(tok[b] == -1)
            continue
        used = range(0, min(max(oa, ga), K) + 1)
        if min(boundary_gap(z64[i, k], kk) for k in used) < 2 * EPS_Z:
            near_rows += 1                  # the kept set may differ: a legitimate other answer
            continue
        decisions += min(oa + 1, K) + 1
        if greedy:
            assert ga == oa and np.array_equal(tok[b], o["tokens"][i]), f"{name} row {b}: greedy"
            continue
        both = min(ga, oa, K - 1) + 1           # positions both sides tested
        pk, gp = o["pk"][i][:both], dg[b, :both]
        assert np.all(np.abs(gp - pk) <= 1e-5 + 4 * EPS_Z / T * pk), f"{name} row {b}: p'(x)"
        assert np.all(np.abs(dg[b, K:K + both] - o["qk"][i][:both]) <= 1e-5), f"{name} row {b}: q'(x)"
        if ga == oa and np.array_equal(tok[b], o["tokens"][i]):
            assert abs(dg[b, 2 * K] - o["S"][i]) <= tol, f"{name} row {b}: S"
            continue
        if ga == oa:
            m = o["m_draw"][i]
        else:
            m = o["m_test"][i, min(ga, oa)]
        assert m < tol, f"{name} row {b}: differs (gpu {ga}, oracle {oa}) at margin {m}"
        assert np.array_equal(tok[b, :min(ga, oa)], o["tokens"][i, :min(ga, oa)])
        assert 0 <= tok[b, ga] < li.V and np.all(tok[b, ga + 1:] == -1)
        admitted += 1
    print(f"[fused] {name}: rows={len(rows)} decisions={decisions} admitted={admitted} near-boundary rows={near_rows}",
          flush=True)
    assert admitted <= ADMIT_RATE * max(decisions, 1) + (1 if decisions < 1000 else 0)
    assert near_rows <= max(1, len(rows) // 20)
    return alen


@pytest.mark.parametrize("B,K,V,H,T,top_k", [
    (6, 3, 2000, 256, 0.7, 50),      # one partial tile of rows (R = 24) and a ragged last unit
    (40, 3, 5000, 512, 1.0, 10),     # two tiles of rows (R = 160)
    (8, 2, 1000, 128, 0.0, 0),       # greedy
    (3, 5, 33000, 1024, 1.3, 64),
    (33, 1, 777, 64, 0.0, 0),
])
def test_fused_small(R, orc, B, K, V, H, T, top_k):
    li = W.make_lm_head(B, K, V, H, temperature=T, top_k=top_k, sigma=W.sigma_const(0.5), config_id=97,
                        seed=V % 1000 + H)
    alen = check(R, orc, li, f"V={V} H={H}")
    assert np.all(alen >= 0)


def test_fused_units_that_hold_many_of_the_top_k(R, orc):
    """A head that puts most of every row's top-k into the first 128 columns: the unit's
    four candidates cannot hold them, so the merge recomputes that unit (same bits) and
    still returns the exact top-k."""
    li = W.make_lm_head(8, 3, 3000, 256, temperature=0.7, top_k=50, sigma=W.sigma_const(0.5), config_id=98,
                        seed=0)
    wt = li.weight.copy()
    bias = W.bf16_bits_to_f32(wt[:, -1]).copy()
    bias[:100] += 12.0                     # 100 logits far above the rest, all in unit 0
    wt[:, -1] = W.f32_to_bf16_bits(bias)
    li = dataclasses.replace(li, weight=wt)
    check(R, orc, li, "saturated unit")


def test_fused_nan_inputs(R, orc):
    """A NaN in a hidden state makes that target row's logits NaN (E1); a NaN in a head row
    makes one logit of every row NaN, so every row is an error row."""
    li = W.make_lm_head(6, 3, 1500, 128, temperature=0.7, top_k=20, sigma=W.sigma_const(0.5), config_id=99,
                        seed=1)
    hid = li.hidden.copy()
    hid[1, 0, 5] = 0x7FC0                   # row 0 of batch 1: always consulted
    hid[2, 3, 7] = 0x7FC0                   # the last row of batch 2: consulted only if all accepted
    alen = check(R, orc, dataclasses.replace(li, hidden=hid), "NaN hidden")
    assert alen[1] == -1
    wt = li.weight.copy()
    wt[700, 3] = 0x7FC0
    alen = check(R, orc, dataclasses.replace(li, weight=wt), "NaN head row")
    assert np.all(alen == -1)
    lg = dataclasses.replace(li, temperature=0.0, top_k=0, hidden=hid)
    alen = check(R, orc, lg, "NaN hidden, greedy")
    assert alen[1] == -1


@pytest.mark.slow
def test_fused_workload9_sampled_rows(R, orc):
    """The benchmark's launch (B=64, K=7, V=128256, H=4096, T=0.7, top-k 50), checked on 8
    batch rows (64 logit rows formed by the oracle)."""
    li = W.config(9, 1)
    check(R, orc, li, "workload 9", rows=np.arange(0, 64, 8))
