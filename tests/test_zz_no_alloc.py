"""spec_verify_chain_noalloc (the chain call on the library's own device scratch, for callers
that cannot allocate) against spec_verify_chain with a caller workspace: the same kernels,
so the outputs must be identical, element for element.  Each mode is called twice in a
row, the second time with a smaller input, and the modes follow one another so that the
scratch is reused across kinds of calls (a top-k call after a dense one needs it zeroed).
"""

import ctypes

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


def both(R, ci, name):
    import torch
    print(f"[case] noalloc {name}: B={ci.B} K={ci.K} V={ci.V} T={ci.temperature} top_k={ci.top_k}", flush=True)
    z, q, x, u = (to_torch(a) for a in (ci.logits, ci.draft_probs, ci.draft_tokens, ci.uniforms))
    dev = z.device
    B, K = ci.B, ci.K
    outs = []
    for fn in ("noalloc", "workspace"):
        tok = torch.full((B, K + 1), -7, dtype=torch.int32, device=dev)
        alen = torch.full((B,), -7, dtype=torch.int32, device=dev)
        dg = torch.full((B, 2 * K + 2), -7.0, dtype=torch.float32, device=dev)
        if fn == "noalloc":
            R.verify_chain_noalloc(z, q, x, u, ci.temperature, ci.top_k, diag=True, out=(tok, alen, dg))
        else:
            R.verify_chain(z, q, x, u, ci.temperature, ci.top_k, diag=True, out=(tok, alen, dg))
        torch.cuda.synchronize()
        outs.append((tok.cpu().numpy(), alen.cpu().numpy(), dg.cpu().numpy()))
    (t1, a1, d1), (t2, a2, d2) = outs
    assert np.array_equal(a1, a2), name
    assert np.array_equal(t1, t2), name
    assert np.array_equal(d1, d2, equal_nan=True), name
    assert np.all(a1 >= 0), name
    return a1


@pytest.mark.parametrize("mode", ["topk", "walk", "greedy", "transformed", "topk-after-all"])
def test_noalloc_matches_the_workspace_call(R, mode):
    if mode in ("topk", "topk-after-all"):
        both(R, W.config(2, 61), "top-k, full c2")
        both(R, W.config(2, 62, B=8), "top-k, B=8")
    elif mode == "walk":
        both(R, W.config(4, 63, B=64), "dense walk B=64")
        both(R, W.config(4, 64, B=16), "dense walk B=16")
    elif mode == "greedy":
        both(R, W.with_transform(W.config(1, 65, B=32), temperature=0.0, top_k=0), "greedy B=32")
        both(R, W.with_transform(W.config(1, 66, B=4), temperature=0.0, top_k=0), "greedy B=4")
    else:
        both(R, W.with_transform(W.config(1, 67, B=16), temperature=0.7, top_k=0), "T=0.7 B=16")
        both(R, W.with_transform(W.config(1, 68, B=3), temperature=0.7, top_k=0), "T=0.7 B=3")


def test_noalloc_rejects_calls_beyond_its_scratch(R):
    """A top-k chain whose workspace exceeds SPEC_NOALLOC_SCRATCH_BYTES returns SPEC_ESCRATCH
    (-5) and launches nothing."""
    L = R.lib()
    B, K, V, T, k = 1024, 8, 128256, 0.7, 50
    assert R.chain_workspace_bytes(B, K, V, 1, T, k) > (32 << 20)
    fake = ctypes.c_void_p(0x7F0000000000)
    rc = L.spec_verify_chain_noalloc(fake, 1, fake, fake, fake, B, K, V, T, k, fake, fake, None, None)
    assert rc == -5
    assert b"scratch" in L.spec_error_string(-5)
