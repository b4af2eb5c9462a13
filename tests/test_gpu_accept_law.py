"""The accept-length law on the GPU, across the sampling workloads.

For one batch row with draft tokens x_k drawn independently from q'_k and
uniforms independent of everything, position k is reached with probability
prod_{i<k} alpha_i, alpha_i = sum min(p'_i, q'_i) ("064 · 投机解码", section 二:
the chance that one drafted token survives is the overlap of the two
distributions).  So E[accept_len] = sum_{k=1..K} prod_{i<k} alpha_i and
Var[accept_len] = sum_k (2k - 1) prod_{i<k} alpha_i - E^2.  The test takes
accept_len from spec_verify_chain and alpha from spec_accept_rate (the GPU's
two entry points, no oracle) over every batch row of a workload recipe and
checks the total with a z-test.  Rows differ in alpha (different logits and
draft noise), so this is the non-iid form of the closed formula
E[tokens] = (1 - alpha^(K+1)) / (1 - alpha) of "投机解码与 EAGLE" section 二.
"""

import numpy as np
import pytest

from parity import to_torch
from rejection_sampling_verify_10_amd import workloads as W

Z_LIMIT = 4.5


@pytest.fixture(scope="module")
def R():
    import torch
    import rejection_sampling_verify_10_amd as R
    assert torch.cuda.is_available(), "GPU test without a GPU"
    R.lib()
    return R


def law_moments(alpha: np.ndarray):
    """Per-row mean and variance of accept_len for independent positions with pass
    probabilities alpha [B, K]."""
    reach = np.cumprod(alpha.astype(np.float64), axis=1)       # P(accept_len >= k), k = 1..K
    K = alpha.shape[1]
    w = 2.0 * np.arange(1, K + 1) - 1.0
    mean = reach.sum(axis=1)
    var = (reach * w).sum(axis=1) - mean ** 2
    return mean, var


def z_score(R, ci) -> float:
    import torch
    z, q, x, u = (to_torch(a) for a in (ci.logits, ci.draft_probs, ci.draft_tokens, ci.uniforms))
    _, alen = R.verify_chain(z, q, x, u, ci.temperature, ci.top_k)
    alpha = R.accept_rate(z, q, ci.temperature, ci.top_k)
    torch.cuda.synchronize()
    alen = alen.cpu().numpy().astype(np.float64)
    alpha = alpha.cpu().numpy()
    assert np.all(alen >= 0) and np.all(np.isfinite(alpha))
    mean, var = law_moments(alpha)
    zs = (alen.sum() - mean.sum()) / np.sqrt(var.sum())
    print(f"[law] B={ci.B} K={ci.K} V={ci.V} T={ci.temperature} top_k={ci.top_k}: mean accept_len "
          f"{alen.mean():.4f} vs {mean.mean():.4f} (z = {zs:+.2f})", flush=True)
    return zs


def test_law_moments_closed_form():
    """With every alpha equal the moments reduce to the closed form of the pages."""
    a = 0.8
    mean, var = law_moments(np.full((1, 4), a))
    assert mean[0] + 1 == pytest.approx((1 - a ** 5) / (1 - a))
    # direct enumeration of P(accept_len = j)
    pj = np.array([a ** j * (1 - a) for j in range(4)] + [a ** 4])
    j = np.arange(5)
    assert var[0] == pytest.approx((pj * j ** 2).sum() - (pj * j).sum() ** 2)


@pytest.mark.gpu
@pytest.mark.parametrize("cid,B,seed", [(1, 1024, 31), (2, 512, 32), (4, 512, 33)])
def test_mean_accept_len_per_workload(R, cid, B, seed):
    """Workload 1 (V = 32000, T = 1), workload 2 (V = 128256, T = 0.7, top-k 50, two
    noise levels) and workload 4 (V = 128256, per-row noise), each over B batch rows."""
    ci = W.config(cid, seed, B=B)
    assert abs(z_score(R, ci)) < Z_LIMIT
