"""Verification step of speculative decoding on MI355X (gfx950).

Thin ctypes binding over ``libspecverify.so`` (see ``include/spec_verify.h``):
it checks tensor placement and dtypes, allocates outputs and the workspace
with torch, and passes raw device pointers plus torch's current HIP stream.
Every step of the computation runs in the library's HIP kernels; there is no
CPU path.  If the library is missing the first call raises.
"""

from __future__ import annotations

import ctypes
import os
from typing import Optional, Sequence, Tuple

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libspecverify.so")

SPEC_F32 = 0
SPEC_BF16 = 1
SPEC_TOPK_MAX = 64
SPEC_MAX_K = 63
SPEC_MAX_NODES = 64

_lib: Optional[ctypes.CDLL] = None


class SpecError(RuntimeError):
    pass


def lib() -> ctypes.CDLL:
    """Load the HIP library (raises if it has not been built).  SPEC_VERIFY_LIBRARY names
    another build of the same sources to load instead (e.g. a host-sanitizer build)."""
    global _lib
    if _lib is None:
        path = os.environ.get("SPEC_VERIFY_LIBRARY") or LIB_PATH
        if not os.path.exists(path):
            raise SpecError(f"{path} is missing: build it with "
                            "`python -m rejection_sampling_verify_10_amd.build`")
        L = ctypes.CDLL(path)
        P, I, F, Z = ctypes.c_void_p, ctypes.c_int, ctypes.c_float, ctypes.c_size_t
        L.spec_error_string.argtypes = [I]
        L.spec_error_string.restype = ctypes.c_char_p
        L.spec_workspace_bytes.argtypes = [I, I, I, I]
        L.spec_workspace_bytes.restype = Z
        L.spec_chain_workspace_bytes.argtypes = [I, I, I, I, F, I]
        L.spec_chain_workspace_bytes.restype = Z
        L.spec_tree_workspace_bytes.argtypes = [I, I, I, I]
        L.spec_tree_workspace_bytes.restype = Z
        L.spec_accept_rate_workspace_bytes.argtypes = [I, I, I, I, F, I]
        L.spec_accept_rate_workspace_bytes.restype = Z
        L.spec_verify_chain.argtypes = [P, I, P, P, P, I, I, I, F, I, P, P, P, P, Z, P]
        L.spec_verify_chain.restype = I
        L.spec_chain_fused_workspace_bytes.argtypes = [I, I, I, I, F, I]
        L.spec_chain_fused_workspace_bytes.restype = Z
        L.spec_verify_chain_fused.argtypes = [P, P, P, P, P, I, I, I, I, F, I, P, P, P, P, Z, P]
        L.spec_verify_chain_fused.restype = I
        L.spec_verify_chain_noalloc.argtypes = [P, I, P, P, P, I, I, I, F, I, P, P, P, P]
        L.spec_verify_chain_noalloc.restype = I
        L.spec_verify_chain_topp.argtypes = [P, I, P, P, P, I, I, I, F, I, F, P, P, P, P, Z, P]
        L.spec_verify_chain_topp.restype = I
        L.spec_verify_tree_greedy.argtypes = [P, I, P, P, I, I, I, P, P, P, P, Z, P]
        L.spec_verify_tree_greedy.restype = I
        L.spec_verify_tree_sample.argtypes = [P, I, P, P, P, P, I, I, I, F, I, P, P, P, P]
        L.spec_verify_tree_sample.restype = I
        L.spec_verify_tree_sample_rows.argtypes = [P, I, P, P, P, P, I, I, I, F, I, P, P, P, P]
        L.spec_verify_tree_sample_rows.restype = I
        L.spec_tree_sample_workspace_bytes.argtypes = [I, I]
        L.spec_tree_sample_workspace_bytes.restype = Z
        L.spec_verify_tree_sample_ws.argtypes = [P, I, P, P, P, P, I, I, I, F, I, P, P, P, P, Z, P]
        L.spec_verify_tree_sample_ws.restype = I
        L.spec_verify_tree_sample_rows_ws.argtypes = [P, I, P, P, P, P, I, I, I, F, I, P, P, P, P, Z, P]
        L.spec_verify_tree_sample_rows_ws.restype = I
        L.spec_verify_tree_greedy_rows.argtypes = [P, I, P, P, I, I, I, P, P, P, P, Z, P]
        L.spec_verify_tree_greedy_rows.restype = I
        L.spec_tree_expand_workspace_bytes.argtypes = [I, I, I, I]
        L.spec_tree_expand_workspace_bytes.restype = Z
        L.spec_tree_expand.argtypes = [P, P, I, I, I, I, I, P, P, P, P, Z, P]
        L.spec_tree_expand.restype = I
        L.spec_tree_rerank.argtypes = [P, P, I, I, I, P, P, P, P]
        L.spec_tree_rerank.restype = I
        LL = ctypes.c_longlong
        L.spec_kv_commit.argtypes = [P, I, LL, I, LL, LL, I, I, P, P, I, I, P, P, P]
        L.spec_kv_commit.restype = I
        L.spec_accept_rate.argtypes = [P, I, P, I, I, I, F, I, P, P, Z, P]
        L.spec_accept_rate.restype = I
        L.spec_profile_events.argtypes = [P, P]
        L.spec_profile_events.restype = I
        L.spec_workspace_init.argtypes = [P, Z, P]
        L.spec_workspace_init.restype = I
        L.spec_copy_probe.argtypes = [P, P, Z, P]
        L.spec_copy_probe.restype = I
        L.spec_read_probe.argtypes = [P, Z, P, P]
        L.spec_read_probe.restype = I
        _lib = L
    return _lib


def _check(rc: int, what: str) -> None:
    if rc != 0:
        raise SpecError(f"{what}: {lib().spec_error_string(rc).decode()} ({rc})")


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return SPEC_BF16
    if t.dtype == torch.float32:
        return SPEC_F32
    raise TypeError(f"logits must be bfloat16 or float32, got {t.dtype}")


def _dev(t: torch.Tensor, name: str, dtype=None) -> int:
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    return t.data_ptr()


def _shape(t: Optional[torch.Tensor], name: str, shape: Tuple[int, ...]) -> None:
    if t is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")


def _stream(device: torch.device) -> int:
    return torch.cuda.current_stream(device).cuda_stream


def _workspace(nbytes: int, device: torch.device,
               given: Optional[torch.Tensor] = None) -> Tuple[int, Optional[torch.Tensor]]:
    if nbytes == 0:
        return 0, None
    if given is not None:
        _dev(given, "workspace", torch.uint8)
        if given.numel() < nbytes + 256:
            raise ValueError(f"workspace needs {nbytes + 256} bytes, got {given.numel()}")
        return (given.data_ptr() + 255) // 256 * 256, given
    ws = torch.zeros(nbytes + 256, dtype=torch.uint8, device=device)
    p = ws.data_ptr()
    return (p + 255) // 256 * 256, ws


def workspace_bytes(B: int, K_or_N: int, V: int, top_k: int = 0) -> int:
    """One workspace size for every chain, acceptance-rate and greedy-tree call of this shape."""
    return int(lib().spec_workspace_bytes(B, K_or_N, V, int(top_k)))


def chain_workspace_bytes(B: int, K: int, V: int, dtype: int, temperature: float, top_k: int) -> int:
    return int(lib().spec_chain_workspace_bytes(B, K, V, dtype, float(temperature), int(top_k)))


def tree_workspace_bytes(B: int, N: int, V: int, dtype: int) -> int:
    return int(lib().spec_tree_workspace_bytes(B, N, V, dtype))


def accept_rate_workspace_bytes(B: int, K: int, V: int, dtype: int, temperature: float, top_k: int) -> int:
    return int(lib().spec_accept_rate_workspace_bytes(B, K, V, dtype, float(temperature), int(top_k)))


def verify_chain(target_logits: torch.Tensor, draft_probs: Optional[torch.Tensor],
                 draft_tokens: torch.Tensor, uniforms: Optional[torch.Tensor],
                 temperature: float = 1.0, top_k: int = 0, top_p: float = 1.0, *, diag: bool = False,
                 out: Optional[Tuple[torch.Tensor, ...]] = None, workspace: Optional[torch.Tensor] = None):
    """Batched chain verification (``spec_verify_chain``).

    target_logits [B, K+1, V] bf16/f32, draft_probs [B, K, V] f32, draft_tokens [B, K] int32,
    uniforms [B, K+1] f32; top_p < 1 adds the nucleus cut (top-k on, temperature > 0).
    Returns (tokens [B, K+1] int32, accept_len [B] int32) and, with
    ``diag=True``, a third tensor [B, 2K+2] f32.  Asynchronous on the current stream.
    ``out`` reuses output tensors; ``workspace`` (uint8, zero-filled before its first
    use, at least the size reported by :func:`chain_workspace_bytes` + 256) avoids the
    per-call allocation; calls leave it reusable.
    """
    B, K1, V = target_logits.shape
    K = K1 - 1
    dev = target_logits.device
    code = _dtype_code(target_logits)
    _shape(draft_probs, "draft_probs", (B, K, V))
    _shape(draft_tokens, "draft_tokens", (B, K))
    _shape(uniforms, "uniforms", (B, K + 1))
    if float(temperature) != 0.0 and (draft_probs is None or uniforms is None):
        raise ValueError("sampling verification needs draft_probs and uniforms")
    z = _dev(target_logits, "target_logits")
    q = _dev(draft_probs, "draft_probs", torch.float32) if draft_probs is not None else None
    x = _dev(draft_tokens, "draft_tokens", torch.int32)
    u = _dev(uniforms, "uniforms", torch.float32) if uniforms is not None else None
    if out is not None:
        _shape(out[0], "out tokens", (B, K + 1))
        _shape(out[1], "out accept_len", (B,))
        if diag:
            _shape(out[2], "out diag", (B, 2 * K + 2))
        _dev(out[0], "out tokens", torch.int32)
        _dev(out[1], "out accept_len", torch.int32)
        if diag:
            _dev(out[2], "out diag", torch.float32)
    if out is None:
        tokens = torch.empty((B, K + 1), dtype=torch.int32, device=dev)
        alen = torch.empty((B,), dtype=torch.int32, device=dev)
        dg = torch.empty((B, 2 * K + 2), dtype=torch.float32, device=dev) if diag else None
    else:
        tokens, alen = out[0], out[1]
        dg = out[2] if diag else None
    need = chain_workspace_bytes(B, K, V, code, temperature, top_k)
    wp, ws = _workspace(need, dev, workspace)
    if float(top_p) != 1.0:
        rc = lib().spec_verify_chain_topp(z, code, q, x, u, B, K, V, float(temperature), int(top_k), float(top_p),
                                          tokens.data_ptr(), alen.data_ptr(),
                                          dg.data_ptr() if dg is not None else None, wp, need, _stream(dev))
        _check(rc, "spec_verify_chain_topp")
    else:
        rc = lib().spec_verify_chain(z, code, q, x, u, B, K, V, float(temperature), int(top_k),
                                     tokens.data_ptr(), alen.data_ptr(), dg.data_ptr() if dg is not None else None,
                                     wp, need, _stream(dev))
        _check(rc, "spec_verify_chain")
    return (tokens, alen, dg) if diag else (tokens, alen)


def chain_fused_workspace_bytes(B: int, K: int, V: int, H: int, temperature: float, top_k: int) -> int:
    return int(lib().spec_chain_fused_workspace_bytes(B, K, V, H, float(temperature), int(top_k)))


def verify_chain_fused(hidden: torch.Tensor, head_weight: torch.Tensor, draft_probs: Optional[torch.Tensor],
                       draft_tokens: torch.Tensor, uniforms: Optional[torch.Tensor], temperature: float = 1.0,
                       top_k: int = 0, *, diag: bool = False, out: Optional[Tuple[torch.Tensor, ...]] = None,
                       workspace: Optional[torch.Tensor] = None):
    """``spec_verify_chain_fused``: the chain verification fed by the target's last hidden
    states and LM head instead of logits (the logits stay on the chip).

    hidden [B, K+1, H] bf16, head_weight [V, H] bf16, draft_probs [B, K, V] f32,
    draft_tokens [B, K] int32, uniforms [B, K+1] f32; greedy (temperature 0) or top-k.
    Returns what :func:`verify_chain` returns."""
    B, K1, H = hidden.shape
    K = K1 - 1
    V = head_weight.shape[0]
    dev = hidden.device
    if hidden.dtype != torch.bfloat16 or head_weight.dtype != torch.bfloat16:
        raise TypeError("hidden and head_weight must be bfloat16")
    _shape(head_weight, "head_weight", (V, H))
    _shape(draft_probs, "draft_probs", (B, K, V))
    _shape(draft_tokens, "draft_tokens", (B, K))
    _shape(uniforms, "uniforms", (B, K + 1))
    if float(temperature) != 0.0 and (draft_probs is None or uniforms is None):
        raise ValueError("sampling verification needs draft_probs and uniforms")
    if out is None:
        tokens = torch.empty((B, K + 1), dtype=torch.int32, device=dev)
        alen = torch.empty((B,), dtype=torch.int32, device=dev)
        dg = torch.empty((B, 2 * K + 2), dtype=torch.float32, device=dev) if diag else None
    else:
        tokens, alen = out[0], out[1]
        dg = out[2] if diag else None
        _shape(tokens, "out tokens", (B, K + 1))
        _shape(alen, "out accept_len", (B,))
        if diag:
            _shape(dg, "out diag", (B, 2 * K + 2))
    need = chain_fused_workspace_bytes(B, K, V, H, temperature, top_k)
    wp, ws = _workspace(need, dev, workspace)
    rc = lib().spec_verify_chain_fused(
        _dev(hidden, "hidden"), _dev(head_weight, "head_weight"),
        _dev(draft_probs, "draft_probs", torch.float32) if draft_probs is not None else None,
        _dev(draft_tokens, "draft_tokens", torch.int32),
        _dev(uniforms, "uniforms", torch.float32) if uniforms is not None else None,
        B, K, V, H, float(temperature), int(top_k), _dev(tokens, "out tokens", torch.int32),
        _dev(alen, "out accept_len", torch.int32), _dev(dg, "out diag", torch.float32) if dg is not None else None,
        wp, need, _stream(dev))
    _check(rc, "spec_verify_chain_fused")
    return (tokens, alen, dg) if diag else (tokens, alen)


def verify_chain_noalloc(target_logits: torch.Tensor, draft_probs: Optional[torch.Tensor],
                         draft_tokens: torch.Tensor, uniforms: Optional[torch.Tensor],
                         temperature: float = 1.0, top_k: int = 0, *, diag: bool = False,
                         out: Optional[Tuple[torch.Tensor, ...]] = None):
    """``spec_verify_chain_noalloc``: :func:`verify_chain` on the library's own device
    scratch (no workspace; with ``out`` given the call allocates nothing at all).
    Calls that may overlap on one GPU race."""
    B, K1, V = target_logits.shape
    K = K1 - 1
    dev = target_logits.device
    code = _dtype_code(target_logits)
    _shape(draft_probs, "draft_probs", (B, K, V))
    _shape(draft_tokens, "draft_tokens", (B, K))
    _shape(uniforms, "uniforms", (B, K + 1))
    if float(temperature) != 0.0 and (draft_probs is None or uniforms is None):
        raise ValueError("sampling verification needs draft_probs and uniforms")
    if out is None:
        tokens = torch.empty((B, K + 1), dtype=torch.int32, device=dev)
        alen = torch.empty((B,), dtype=torch.int32, device=dev)
        dg = torch.empty((B, 2 * K + 2), dtype=torch.float32, device=dev) if diag else None
    else:
        tokens, alen = out[0], out[1]
        dg = out[2] if diag else None
        _shape(tokens, "out tokens", (B, K + 1))
        _shape(alen, "out accept_len", (B,))
        if diag:
            _shape(dg, "out diag", (B, 2 * K + 2))
    rc = lib().spec_verify_chain_noalloc(
        _dev(target_logits, "target_logits"), code,
        _dev(draft_probs, "draft_probs", torch.float32) if draft_probs is not None else None,
        _dev(draft_tokens, "draft_tokens", torch.int32),
        _dev(uniforms, "uniforms", torch.float32) if uniforms is not None else None,
        B, K, V, float(temperature), int(top_k), _dev(tokens, "out tokens", torch.int32),
        _dev(alen, "out accept_len", torch.int32), _dev(dg, "out diag", torch.float32) if dg is not None else None,
        _stream(dev))
    _check(rc, "spec_verify_chain_noalloc")
    return (tokens, alen, dg) if diag else (tokens, alen)


def verify_tree_greedy(target_logits: torch.Tensor, node_tokens: torch.Tensor, parents: Sequence[int], *,
                       out: Optional[Tuple[torch.Tensor, ...]] = None, workspace: Optional[torch.Tensor] = None):
    """Greedy static-tree verification (``spec_verify_tree_greedy``).

    target_logits [B, N, V], node_tokens [B, N] int32, parents: N host ints (one static tree)
    or a [B, N] int32 GPU tensor (a tree per batch row; then D = N - 1).
    Returns (path [B, D+1], tokens [B, D+1], accept_len [B]) int32 tensors.  ``out`` reuses
    output tensors and ``workspace`` a workspace, as for :func:`verify_chain`.
    """
    B, N, V = target_logits.shape
    dev = target_logits.device
    code = _dtype_code(target_logits)
    _shape(node_tokens, "node_tokens", (B, N))
    rows = isinstance(parents, torch.Tensor)
    par, D = _tree_parents(parents, B, N)
    path, toks, alen = _tree_outputs(out, B, D, dev)
    need = tree_workspace_bytes(B, N, V, code)
    wp, ws = _workspace(need, dev, workspace)
    fn = lib().spec_verify_tree_greedy_rows if rows else lib().spec_verify_tree_greedy
    rc = fn(_dev(target_logits, "target_logits"), code, _dev(node_tokens, "node_tokens", torch.int32), par, B, N, V,
            path.data_ptr(), toks.data_ptr(), alen.data_ptr(), wp, need, _stream(dev))
    _check(rc, "spec_verify_tree_greedy" + ("_rows" if rows else ""))
    return path, toks, alen


def _tree_parents(parents, B: int, N: int):
    """A static tree (N host ints) -> (ctypes array, max depth); a tree per batch row
    ([B, N] int32 GPU tensor) -> (its pointer, N - 1)."""
    if isinstance(parents, torch.Tensor):
        _shape(parents, "parents", (B, N))
        return _dev(parents, "parents", torch.int32), N - 1
    if len(parents) != N:
        raise ValueError(f"parents must have {N} entries")
    par = (ctypes.c_int32 * N)(*[int(p) for p in parents])
    depth = [0] * N
    for n in range(1, N):
        depth[n] = depth[int(parents[n])] + 1 if 0 <= int(parents[n]) < n else 0
    return par, max(depth)


def _tree_outputs(out, B: int, D: int, dev):
    if out is None:
        return (torch.empty((B, D + 1), dtype=torch.int32, device=dev),
                torch.empty((B, D + 1), dtype=torch.int32, device=dev),
                torch.empty((B,), dtype=torch.int32, device=dev))
    path, toks, alen = out
    _shape(path, "out path", (B, D + 1))
    _shape(toks, "out tokens", (B, D + 1))
    _shape(alen, "out accept_len", (B,))
    for o, n in ((path, "out path"), (toks, "out tokens"), (alen, "out accept_len")):
        _dev(o, n, torch.int32)
    return path, toks, alen


def tree_sample_workspace_bytes(B: int, N: int) -> int:
    return int(lib().spec_tree_sample_workspace_bytes(B, N))


def verify_tree_sample(target_logits: torch.Tensor, draft_probs: torch.Tensor, node_tokens: torch.Tensor,
                       uniforms: torch.Tensor, parents: Sequence[int], temperature: float = 1.0, top_k: int = 0,
                       *, out: Optional[Tuple[torch.Tensor, ...]] = None, workspace=None):
    """Sampling static-tree verification (``spec_verify_tree_sample_ws``).

    target_logits [B, N, V] bf16/f32, draft_probs [B, N, V] f32 (row n: the draft
    distribution at node n), node_tokens [B, N] int32, uniforms [B, N] f32 (u[n] tests
    node n, u[0] drives the final draw), parents: N host ints (one static tree) or a [B, N]
    int32 GPU tensor (a tree per batch row; then D = N - 1).  Returns (path [B, D+1],
    tokens [B, D+1], accept_len [B]) int32 tensors; ``out`` reuses output tensors.
    ``workspace``: a zeroed uint8 tensor of at least tree_sample_workspace_bytes(B, N)
    (left zero by the call), None for a fresh one, or False for the call without a
    workspace (``spec_verify_tree_sample``: one workgroup per batch row).
    """
    B, N, V = target_logits.shape
    dev = target_logits.device
    code = _dtype_code(target_logits)
    _shape(draft_probs, "draft_probs", (B, N, V))
    _shape(node_tokens, "node_tokens", (B, N))
    _shape(uniforms, "uniforms", (B, N))
    rows = isinstance(parents, torch.Tensor)
    par, D = _tree_parents(parents, B, N)
    path, toks, alen = _tree_outputs(out, B, D, dev)
    args = (_dev(target_logits, "target_logits"), code, _dev(draft_probs, "draft_probs", torch.float32),
            _dev(node_tokens, "node_tokens", torch.int32), _dev(uniforms, "uniforms", torch.float32), par, B, N, V,
            float(temperature), int(top_k), path.data_ptr(), toks.data_ptr(), alen.data_ptr())
    name = "spec_verify_tree_sample" + ("_rows" if rows else "")
    if workspace is False:
        rc = getattr(lib(), name)(*args, _stream(dev))
    else:
        need = tree_sample_workspace_bytes(B, N)
        wp, _ws = _workspace(need, dev, workspace)
        name += "_ws"
        rc = getattr(lib(), name)(*args, wp, need, _stream(dev))
    _check(rc, name)
    return path, toks, alen


def tree_expand_workspace_bytes(B: int, E: int, V: int, top_k: int) -> int:
    return int(lib().spec_tree_expand_workspace_bytes(B, E, V, top_k))


def tree_expand(draft_probs: torch.Tensor, node_values: torch.Tensor, top_k: int, k_next: int, *,
                out: Optional[Tuple[torch.Tensor, ...]] = None, workspace: Optional[torch.Tensor] = None):
    """One EAGLE-2 expansion layer (``spec_tree_expand``).

    draft_probs [B, E, V] f32, node_values [B, E] f32.  Returns (child tokens [B, E, top_k]
    int32, child values [B, E, top_k] f32, next [B, k_next] int32 flat child indices).
    """
    B, E, V = draft_probs.shape
    dev = draft_probs.device
    _shape(node_values, "node_values", (B, E))
    if out is None:
        toks = torch.empty((B, E, top_k), dtype=torch.int32, device=dev)
        vals = torch.empty((B, E, top_k), dtype=torch.float32, device=dev)
        nxt = torch.empty((B, k_next), dtype=torch.int32, device=dev)
    else:
        toks, vals, nxt = out
        _shape(toks, "out tokens", (B, E, top_k))
        _shape(vals, "out values", (B, E, top_k))
        _shape(nxt, "out next", (B, k_next))
        _dev(toks, "out tokens", torch.int32)
        _dev(vals, "out values", torch.float32)
        _dev(nxt, "out next", torch.int32)
    need = tree_expand_workspace_bytes(B, E, V, top_k)
    wp, ws = _workspace(need, dev, workspace)
    rc = lib().spec_tree_expand(_dev(draft_probs, "draft_probs", torch.float32),
                                _dev(node_values, "node_values", torch.float32), B, E, V, int(top_k), int(k_next),
                                toks.data_ptr(), vals.data_ptr(), nxt.data_ptr(), wp, need, _stream(dev))
    _check(rc, "spec_tree_expand")
    return toks, vals, nxt


def tree_rerank(parents: torch.Tensor, values: torch.Tensor, m: int):
    """EAGLE-2 reranking (``spec_tree_rerank``).

    parents [B, M] int32 (-1 = child of the root), values [B, M] f32.  Returns (nodes [B, m],
    parent positions [B, m]) int32 and the ancestor mask [B, m+1, m+1] uint8.
    """
    B, M = parents.shape
    dev = parents.device
    _shape(values, "values", (B, M))
    nodes = torch.empty((B, m), dtype=torch.int32, device=dev)
    ppos = torch.empty((B, m), dtype=torch.int32, device=dev)
    mask = torch.empty((B, m + 1, m + 1), dtype=torch.uint8, device=dev)
    rc = lib().spec_tree_rerank(_dev(parents, "parents", torch.int32), _dev(values, "values", torch.float32), B, M,
                                int(m), nodes.data_ptr(), ppos.data_ptr(), mask.data_ptr(), _stream(dev))
    _check(rc, "spec_tree_rerank")
    return nodes, ppos, mask


def kv_commit(kv: torch.Tensor, prefix: torch.Tensor, path: torch.Tensor, accept_len: torch.Tensor, N: int,
              *, out_len: Optional[torch.Tensor] = None, capacity: Optional[int] = None) -> torch.Tensor:
    """KV commit of accepted tree paths (``spec_kv_commit``), in place.

    kv [planes, B, S, ...] on the GPU, rows = the trailing dimensions (contiguous within a
    row; planes, batch and positions may be strided); prefix [B], path [B, D+1] and
    accept_len [B] int32.  capacity (positions per (plane, b) row, at most S) defaults to S;
    a batch row whose path would reach past it moves nothing.  Returns the new lengths [B]
    int32 (-1 for such rows and malformed ones).
    """
    planes, B, S = kv.shape[:3]
    cap = S if capacity is None else int(capacity)
    if not 1 <= cap <= S:
        raise ValueError(f"capacity must lie in [1, {S}]")
    if not kv.is_cuda:
        raise ValueError("kv must be a GPU tensor")
    row = kv[0, 0, 0]
    if not row.is_contiguous():
        raise ValueError("a KV row must be contiguous")
    if any(kv.stride(d) == 0 and kv.shape[d] > 1 for d in range(3)):
        raise ValueError("kv planes, batch rows and positions must not share memory (an expanded view)")
    es = kv.element_size()
    _shape(prefix, "prefix", (B,))
    _shape(accept_len, "accept_len", (B,))
    if path.dim() != 2 or path.shape[0] != B:
        raise ValueError("path must be [B, D+1]")
    nl = out_len if out_len is not None else torch.empty((B,), dtype=torch.int32, device=kv.device)
    rc = lib().spec_kv_commit(kv.data_ptr(), planes, kv.stride(0) * es, B, kv.stride(1) * es, kv.stride(2) * es,
                              row.numel() * es, cap, _dev(prefix, "prefix", torch.int32),
                              _dev(path, "path", torch.int32),
                              path.shape[1], int(N), _dev(accept_len, "accept_len", torch.int32),
                              _dev(nl, "out_len", torch.int32), _stream(kv.device))
    _check(rc, "spec_kv_commit")
    return nl


def accept_rate(target_logits: torch.Tensor, draft_probs: torch.Tensor, temperature: float = 1.0,
                top_k: int = 0, *, out: Optional[torch.Tensor] = None,
                workspace: Optional[torch.Tensor] = None) -> torch.Tensor:
    """alpha[b, k] = sum min(p'_k, q'_k) (``spec_accept_rate``); returns [B, K] f32.
    ``out`` reuses the output tensor and ``workspace`` a workspace, as for :func:`verify_chain`."""
    B, K1, V = target_logits.shape
    K = K1 - 1
    dev = target_logits.device
    code = _dtype_code(target_logits)
    _shape(draft_probs, "draft_probs", (B, K, V))
    if out is None:
        alpha = torch.empty((B, K), dtype=torch.float32, device=dev)
    else:
        _shape(out, "out alpha", (B, K))
        _dev(out, "out alpha", torch.float32)
        alpha = out
    need = accept_rate_workspace_bytes(B, K, V, code, temperature, top_k)
    wp, ws = _workspace(need, dev, workspace)
    rc = lib().spec_accept_rate(_dev(target_logits, "target_logits"), code,
                                _dev(draft_probs, "draft_probs", torch.float32), B, K, V,
                                float(temperature), int(top_k), alpha.data_ptr(), wp, need, _stream(dev))
    _check(rc, "spec_accept_rate")
    return alpha


def new_workspace(nbytes: int, device: torch.device) -> torch.Tensor:
    """A zero-filled workspace tensor for the ``workspace=`` argument."""
    return torch.zeros(nbytes + 256, dtype=torch.uint8, device=device)


def profile_next_call(start: torch.cuda.Event, stop: torch.cuda.Event) -> None:
    """Bracket the dominant kernel of this thread's next verification call with two events."""
    _check(lib().spec_profile_events(ctypes.c_void_p(start.cuda_event), ctypes.c_void_p(stop.cuda_event)),
           "spec_profile_events")


def copy_probe(src: torch.Tensor, dst: torch.Tensor) -> None:
    """Plain streaming copy kernel (for calibrating hardware byte counters)."""
    n = src.numel() * src.element_size()
    if dst.numel() * dst.element_size() < n:
        raise ValueError("dst is smaller than src")
    _check(lib().spec_copy_probe(_dev(src, "src"), _dev(dst, "dst"), n, _stream(src.device)), "spec_copy_probe")


def read_probe(src: torch.Tensor, sink: torch.Tensor) -> None:
    """Read-only streaming kernel over src (achievable HBM read bandwidth)."""
    n = src.numel() * src.element_size()
    _check(lib().spec_read_probe(_dev(src, "src"), n, _dev(sink, "sink"), _stream(src.device)), "spec_read_probe")
