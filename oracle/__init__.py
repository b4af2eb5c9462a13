"""CPU oracle for the speculative-decoding verification step (test infrastructure).

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  It wraps ``liboracle.so`` (built from
``spec_oracle.c`` by :func:`build`) with ctypes and numpy; it shares no code
with the HIP library.

Every function is a plain fp64 restatement of the method; see the header of
``spec_oracle.c`` for the passages followed, the readings taken and the error
rules.
"""

from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Optional

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "spec_oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")
_lib: Optional[ctypes.CDLL] = None

F32 = 0
BF16 = 1
F64 = 2      # fp64 logit rows (the logits lm_head_logits forms)


def build(force: bool = True) -> str:
    """Compile liboracle.so with gcc (fp64, IEEE semantics, OpenMP over batch rows)."""
    if force or not os.path.exists(_LIB):
        tmp = _LIB + ".tmp"
        subprocess.check_call(["gcc", "-O2", "-std=c11", "-fopenmp", "-fPIC", "-shared",
                               "-Wall", "-Wno-unknown-pragmas", "-o", tmp, _SRC, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


def lib() -> ctypes.CDLL:
    """The oracle library; ORACLE_LIBRARY names another build of the same source (the
    sanitizer build of the host-side tests)."""
    global _lib
    if _lib is None:
        path = os.environ.get("ORACLE_LIBRARY") or _LIB
        if path == _LIB and not os.path.exists(_LIB):
            build()
        L = ctypes.CDLL(path)
        P, I, D = ctypes.c_void_p, ctypes.c_int, ctypes.c_double
        L.oracle_verify_chain.argtypes = [P, I, P, P, P, I, I, I, D, I, P, P, P, P, P, P, P, P]
        L.oracle_verify_chain_p.argtypes = [P, I, P, P, P, I, I, I, D, I, D, P, P, P, P, P, P, P, P]
        L.oracle_target_dist_p.argtypes = [P, I, I, D, I, D, P]
        L.oracle_draft_dist_p.argtypes = [P, I, D, I, D, P]
        L.oracle_verify_tree_greedy.argtypes = [P, I, P, P, I, I, I, P, P, P]
        L.oracle_accept_rate.argtypes = [P, I, P, I, I, I, D, I, P]
        L.oracle_verify_tree_sample.argtypes = [P, I, P, P, P, P, I, I, I, D, I, P, P, P, P, P]
        L.oracle_tree_expand.argtypes = [P, P, I, I, I, I, I, P, P, P]
        L.oracle_tree_rerank.argtypes = [P, P, I, I, I, P, P, P]
        LL = ctypes.c_longlong
        L.oracle_kv_commit.argtypes = [P, I, LL, I, LL, LL, I, I, P, P, I, I, P, P]
        L.oracle_target_dist.argtypes = [P, I, I, D, I, P]
        L.oracle_lm_head_logits.argtypes = [P, P, I, I, I, P]
        L.oracle_draft_dist.argtypes = [P, I, D, I, P]
        L.oracle_argmax_row.argtypes = [P, I, I]
        L.oracle_set_variant.argtypes = [I]
        L.oracle_set_threads.argtypes = [I]
        L.oracle_set_threads.restype = None
        for f in ("oracle_verify_chain", "oracle_verify_chain_p", "oracle_target_dist_p", "oracle_draft_dist_p",
                  "oracle_verify_tree_greedy", "oracle_accept_rate",
                  "oracle_verify_tree_sample", "oracle_tree_expand", "oracle_tree_rerank", "oracle_kv_commit",
                  "oracle_target_dist", "oracle_draft_dist", "oracle_argmax_row", "oracle_lm_head_logits",
                  "oracle_max_threads"):
            getattr(L, f).restype = I
        L.oracle_set_variant.restype = None
        _lib = L
    return _lib


def _p(a: np.ndarray) -> int:
    assert a.flags.c_contiguous
    return a.ctypes.data


def _logits_arr(logits: np.ndarray, dtype: int) -> np.ndarray:
    want = np.uint16 if dtype == BF16 else np.float64 if dtype == F64 else np.float32
    return np.ascontiguousarray(logits, dtype=want)


def set_variant(v: int) -> None:
    """Plant a deliberate mistake (tests of the pins only); 0 restores the method."""
    lib().oracle_set_variant(int(v))


def set_threads(n: int) -> None:
    """Threads of the oracle's loops over batch rows."""
    lib().oracle_set_threads(int(n))


def max_threads() -> int:
    return int(lib().oracle_max_threads())


def verify_chain(logits, dtype, draft_probs, draft_tokens, uniforms, temperature, top_k, top_p=1.0):
    """Chain verification (a nucleus cut at top_p < 1 after temperature and top-k); returns a
    dict of numpy arrays (see spec_oracle.c)."""
    z = _logits_arr(logits, dtype)
    B, K1, V = z.shape
    K = K1 - 1
    q = np.ascontiguousarray(draft_probs, dtype=np.float32).reshape(B, K, V)
    x = np.ascontiguousarray(draft_tokens, dtype=np.int32).reshape(B, K)
    u = np.ascontiguousarray(uniforms, dtype=np.float32).reshape(B, K + 1)
    out = dict(tokens=np.empty((B, K + 1), np.int32), accept_len=np.empty(B, np.int32),
               pk=np.empty((B, K)), qk=np.empty((B, K)), S=np.empty(B), py=np.empty(B),
               m_test=np.empty((B, K)), m_draw=np.empty(B))
    rc = lib().oracle_verify_chain_p(_p(z), dtype, _p(q), _p(x), _p(u), B, K, V, float(temperature),
                                   int(top_k), float(top_p), _p(out["tokens"]), _p(out["accept_len"]),
                                   _p(out["pk"]), _p(out["qk"]), _p(out["S"]), _p(out["py"]),
                                   _p(out["m_test"]), _p(out["m_draw"]))
    if rc != 0:
        raise ValueError(f"oracle_verify_chain rejected its arguments ({rc})")
    return out


def verify_tree_greedy(logits, dtype, node_tokens, parents):
    z = _logits_arr(logits, dtype)
    B, N, V = z.shape
    par = np.ascontiguousarray(parents, dtype=np.int32)
    tok = np.ascontiguousarray(node_tokens, dtype=np.int32).reshape(B, N)
    depth = np.zeros(N, dtype=np.int64)
    for n in range(1, N):
        depth[n] = depth[par[n]] + 1
    D = int(depth.max())
    out = dict(path=np.empty((B, D + 1), np.int32), tokens=np.empty((B, D + 1), np.int32),
               accept_len=np.empty(B, np.int32))
    rc = lib().oracle_verify_tree_greedy(_p(z), dtype, _p(tok), _p(par), B, N, V, _p(out["path"]),
                                         _p(out["tokens"]), _p(out["accept_len"]))
    if rc != 0:
        raise ValueError(f"oracle_verify_tree_greedy rejected its arguments ({rc})")
    return out


def tree_depths(parents) -> np.ndarray:
    par = np.asarray(parents, dtype=np.int64)
    depth = np.zeros(par.shape[0], dtype=np.int64)
    for n in range(1, par.shape[0]):
        depth[n] = depth[par[n]] + 1
    return depth


def verify_tree_sample(logits, dtype, draft_probs, node_tokens, uniforms, parents, temperature, top_k):
    """Sampling verification of a static tree (T > 0); returns path, tokens, accept_len,
    m_test [B, N] and m_draw [B] (see spec_oracle.c)."""
    z = _logits_arr(logits, dtype)
    B, N, V = z.shape
    par = np.ascontiguousarray(parents, dtype=np.int32)
    q = np.ascontiguousarray(draft_probs, dtype=np.float32).reshape(B, N, V)
    tok = np.ascontiguousarray(node_tokens, dtype=np.int32).reshape(B, N)
    u = np.ascontiguousarray(uniforms, dtype=np.float32).reshape(B, N)
    D = int(tree_depths(par).max())
    out = dict(path=np.empty((B, D + 1), np.int32), tokens=np.empty((B, D + 1), np.int32),
               accept_len=np.empty(B, np.int32), m_test=np.empty((B, N)), m_draw=np.empty(B))
    rc = lib().oracle_verify_tree_sample(_p(z), dtype, _p(q), _p(tok), _p(u), _p(par), B, N, V,
                                         float(temperature), int(top_k), _p(out["path"]),
                                         _p(out["tokens"]), _p(out["accept_len"]), _p(out["m_test"]),
                                         _p(out["m_draw"]))
    if rc != 0:
        raise ValueError(f"oracle_verify_tree_sample rejected its arguments ({rc})")
    return out


def tree_expand(draft_probs, node_values, top_k, k_next):
    """One EAGLE-2 expansion layer: child tokens [B,E,K], child values [B,E,K] (float32) and
    the k_next flat child indices of highest value [B,k_next]."""
    q = np.ascontiguousarray(draft_probs, dtype=np.float32)
    B, E, V = q.shape
    nv = np.ascontiguousarray(node_values, dtype=np.float32).reshape(B, E)
    out = dict(tokens=np.empty((B, E, top_k), np.int32), values=np.empty((B, E, top_k), np.float32),
               next=np.empty((B, k_next), np.int32))
    rc = lib().oracle_tree_expand(_p(q), _p(nv), B, E, V, int(top_k), int(k_next), _p(out["tokens"]),
                                  _p(out["values"]), _p(out["next"]))
    if rc != 0:
        raise ValueError(f"oracle_tree_expand rejected its arguments ({rc})")
    return out


def tree_rerank(parents, values, m):
    """EAGLE-2 reranking: kept nodes in flattened order [B,m], their parents' flattened
    positions [B,m] (0 = root) and the ancestor mask [B,m+1,m+1] (uint8)."""
    par = np.ascontiguousarray(parents, dtype=np.int32)
    B, M = par.shape
    v = np.ascontiguousarray(values, dtype=np.float32).reshape(B, M)
    out = dict(nodes=np.empty((B, m), np.int32), parent_pos=np.empty((B, m), np.int32),
               mask=np.empty((B, m + 1, m + 1), np.uint8))
    rc = lib().oracle_tree_rerank(_p(par), _p(v), B, M, int(m), _p(out["nodes"]), _p(out["parent_pos"]),
                                  _p(out["mask"]))
    if rc != 0:
        raise ValueError(f"oracle_tree_rerank rejected its arguments ({rc})")
    return out


def kv_commit(kv, prefix, path, N, accept_len, capacity=None):
    """KV commit on a copy of kv [planes, B, S, row] (any dtype): returns (new kv, new lengths).
    capacity (positions per (plane, b) row) defaults to S."""
    out = np.ascontiguousarray(kv).copy()
    planes, B, S = out.shape[:3]
    cap = S if capacity is None else int(capacity)
    row_bytes = out[0, 0, 0].nbytes
    pre = np.ascontiguousarray(prefix, dtype=np.int32)
    pth = np.ascontiguousarray(path, dtype=np.int32)
    al = np.ascontiguousarray(accept_len, dtype=np.int32)
    nl = np.empty(B, np.int32)
    rc = lib().oracle_kv_commit(_p(out), planes, out[0].nbytes, B, out[0, 0].nbytes, row_bytes, row_bytes, cap,
                                _p(pre), _p(pth), pth.shape[1], int(N), _p(al), _p(nl))
    if rc != 0:
        raise ValueError(f"oracle_kv_commit rejected its arguments ({rc})")
    return out, nl


def lm_head_logits(hidden_bits, weight_bits) -> np.ndarray:
    """fp64 logits hidden @ W^T of bf16 hidden states [..., H] and head weights [V, H] (raw
    bits, uint16); shape [..., V]."""
    h = np.ascontiguousarray(hidden_bits, dtype=np.uint16)
    w = np.ascontiguousarray(weight_bits, dtype=np.uint16)
    H = h.shape[-1]
    V = w.shape[0]
    assert w.shape[1] == H
    R = h.size // H
    z = np.empty((R, V))
    if lib().oracle_lm_head_logits(_p(h), _p(w), R, V, H, _p(z)) != 0:
        raise ValueError("oracle_lm_head_logits rejected its arguments")
    return z.reshape(h.shape[:-1] + (V,))


def accept_rate(logits, dtype, draft_probs, temperature, top_k):
    z = _logits_arr(logits, dtype)
    B, K1, V = z.shape
    K = K1 - 1
    q = np.ascontiguousarray(draft_probs, dtype=np.float32).reshape(B, K, V)
    a = np.empty((B, K))
    rc = lib().oracle_accept_rate(_p(z), dtype, _p(q), B, K, V, float(temperature), int(top_k), _p(a))
    if rc != 0:
        raise ValueError(f"oracle_accept_rate rejected its arguments ({rc})")
    return a


def target_dist(row, dtype, temperature, top_k, top_p=1.0):
    """p' of one logit row (fp64, length V); None if the row is invalid."""
    z = _logits_arr(row, dtype).reshape(-1)
    p = np.empty(z.shape[0])
    bad = lib().oracle_target_dist_p(_p(z), dtype, z.shape[0], float(temperature), int(top_k), float(top_p), _p(p))
    return None if bad else p


def draft_dist(row, temperature, top_k, top_p=1.0):
    """q' of one row of draft probabilities (fp64); None if invalid."""
    q = np.ascontiguousarray(row, dtype=np.float32).reshape(-1)
    out = np.empty(q.shape[0])
    bad = lib().oracle_draft_dist_p(_p(q), q.shape[0], float(temperature), int(top_k), float(top_p), _p(out))
    return None if bad else out


def argmax_row(row, dtype) -> int:
    z = _logits_arr(row, dtype).reshape(-1)
    return int(lib().oracle_argmax_row(_p(z), dtype, z.shape[0]))
