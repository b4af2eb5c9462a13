#!/usr/bin/env python3
"""Throughput of the speculative-decoding verification step on one MI355X.

A step is one call of the workload's entry point over one batch of synthetic
inputs that already sit in HBM: spec_verify_chain (workloads 0, 1, 2, 4, and 10
with the nucleus on whole rows), spec_verify_tree_greedy (3),
spec_verify_tree_sample (5), one EAGLE-2 expansion layer, spec_tree_expand (6),
spec_kv_commit (7), spec_accept_rate on the inputs of workload 4 (8), or
spec_verify_chain_fused, the LM head with the verification in its epilogue (9).  The default
workload is the chain verification with B=64, K=7, V=128256 (bf16 target
logits, fp32 draft probabilities, temperature 0.7, top-k 50 on both
distributions).  Several copies of the inputs are rotated so that the working
set exceeds the 256 MB Infinity Cache.

Prints ONE JSON line: the workload's rows per second (verified token rows
B*(K+1) for a chain, node rows B*N for a tree, expanded draft rows B*E,
committed paths B) and the step time from K timed steps with nothing else on
the stream; the dominant kernel's achieved HBM bandwidth against the 8 TB/s
peak, timed live with HIP events that the library attaches to that kernel's
dispatch on the call's stream during a second pass of K steps (events between
kernels add several microseconds of queue latency, so they stay out of the
step timing); the hardware-counter traffic recorded under profiles/ when it
matches the current kernel source; and the CPU oracle's throughput on the host
cores.

    python bench.py [--gpus 1] [--steps 400] [--warmup 40] [--workload 0..10] [--no-c4]

The default line (workload 2) also carries, under "c4", the step time, rows/s and
walk-kernel roofline of workload 4, measured in a child process.
"""

from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
PEAK_HBM_GBS = 8000.0
PEAK_BF16_TFLOPS = 2500.0     # dense bf16 matrix-core peak
METRIC = "verified token-rows/s and achieved HBM GB/s (% of peak), V=128256, B=64, K=7"

# The default is the headline workload (2); 0, 1 and 3 are the small configurations, bound by
# launch latency and reported without a bandwidth bar.  copies: input sets rotated so that
# the working set exceeds the 256 MB Infinity Cache where it can.
WORKLOADS = {
    0: dict(name="chain verify B=1 K=4 V=1000, fp32 target logits, fp32 draft probs, T=1, no top-k",
            kernel="dense_walk_kernel", copies=1, oracle_rows=1, dtype="f32 in, f32 exp, f64 draw"),
    1: dict(name="chain verify B=8 K=5 V=32000, bf16 target logits, fp32 draft probs, T=1, no top-k",
            kernel="draw_part_kernel", copies=64, oracle_rows=8, dtype="bf16 in, f32 exp, f64 draw"),
    2: dict(name="chain verify B=64 K=7 V=128256, bf16 target logits, fp32 draft probs, T=0.7, top_k=50",
            kernel="topk_chunk_kernel", copies=4, oracle_rows=64, single_kernel=True,
            dtype="bf16/f32 in, f32 select, f32 probabilities"),
    3: dict(name="greedy static-tree verify B=32 N=27 (depth 5) V=32000, bf16 target logits",
            kernel="rowstats_kernel", copies=10, oracle_rows=32, dtype="bf16 in, exact argmax"),
    4: dict(name="chain verify B=512 K=8 V=128256, bf16 target logits, fp32 draft probs, T=1, no top-k",
            kernel="dense_walk_kernel", copies=1, oracle_rows=32, single_kernel=True,
            dtype="bf16 in, f32 exp, f64 draw"),
    5: dict(name="sampled static-tree verify B=32 N=27 (depth 5) V=32000, bf16 target logits, fp32 draft probs, "
                 "T=1, no top-k",
            kernel="tree_cluster_kernel", copies=4, oracle_rows=32, dtype="bf16 in, f64 probabilities"),
    7: dict(name="KV commit of accepted tree paths B=64, 64 planes (32 layers x K/V), 2 KiB rows (8 heads x 128 "
                 "x bf16), 27-node tree, prefix <= 16",
            kernel="kv_commit_kernel", copies=8, oracle_rows=64, dtype="bytes (bf16 rows)"),
    9: dict(name="LM head fused with chain verify B=64 K=7 V=128256 H=4096, bf16 hidden states and head, fp32 draft "
                 "probs, T=0.7, top_k=50",
            kernel="lmhead_tile_kernel", copies=1, oracle_rows=4, bound="mfma",
            dtype="bf16 MFMA with f32 accumulation, f32 select, f32 probabilities"),
    8: dict(name="acceptance rate B=512 K=8 V=128256, bf16 target logits, fp32 draft probs, T=1, no top-k",
            kernel="alpha_row_kernel", copies=1, oracle_rows=32, single_kernel=True,
            dtype="bf16 in, f32 exp and terms, f64 sums"),
    10: dict(name="chain verify with the nucleus on whole rows B=64 K=7 V=128256, bf16 target logits, fp32 draft "
                  "probs, T=0.7, top_p=0.9, no top-k",
             kernel="nucleus_row_kernel", copies=4, oracle_rows=16, top_p=0.9,
             dtype="bf16/f32 in, f64 probabilities, fixed-point cut masses"),
    6: dict(name="EAGLE-2 expansion layer B=64 E=10 V=128256, fp32 draft probs, top_k=10 children per node, "
                 "k_next=10 kept",
            kernel="topk_chunk_kernel", copies=2, oracle_rows=8, dtype="f32 in, f32 select and value products"),
}


def log(msg: str) -> None:
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def kernel_source_digest() -> str:
    """Digest of every kernel source (csrc/*.hip, *.hpp): counter figures taken on other
    sources are stale."""
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "rejection_sampling_verify_10_amd", "csrc")
    for f in sorted(os.listdir(csrc)):
        if f.endswith((".hip", ".hpp")):
            with open(os.path.join(csrc, f), "rb") as fh:
                h.update(f.encode() + b"\0" + fh.read())
    return h.hexdigest()[:16]


def counter_traffic(workload: int):
    """HBM bytes per launch of the dominant kernel from the committed counter summary,
    or None when the summary is absent or was taken on another kernel source."""
    path = os.path.join(ROOT, "profiles", f"{WORKLOADS[workload]['kernel']}_workload{workload}_counters.md")
    if not os.path.exists(path):
        return None
    text = open(path).read()
    m_sha = re.search(r"kernel_source_digest:\s*([0-9a-f]+)", text)
    m_b = re.search(r"traffic_bytes_per_launch:\s*([0-9.eE+]+)", text)
    if not (m_sha and m_b) or m_sha.group(1) != kernel_source_digest():
        return None
    return float(m_b.group(1))


SELECT_CHUNK_BYTES = 112 * 1024    # largest chunk of a row in the top-k selection kernel


def select_chunks(V: int, esz: int) -> int:
    """Chunks per row in the top-k selection: the fewest equal chunks of whole 16-byte
    vectors that each fit SELECT_CHUNK_BYTES."""
    per_vec = 16 // esz
    c = max(1, -(-V * esz // SELECT_CHUNK_BYTES))
    while True:
        e = -(-V // c)
        e = -(-e // per_vec) * per_vec
        if e * esz <= SELECT_CHUNK_BYTES:
            return -(-V // e)
        c += 1


def tree_walk_rows(path, parents):
    """Rows the sampled-tree walk reads from memory: per batch row, the target rows of the
    nodes it visits and the draft rows of the visited nodes where a residual was formed (a
    child other than the first accepted, or every child rejected)."""
    first = {}
    for n in range(1, len(parents)):
        first.setdefault(int(parents[n]), n)
    targets = drafts = tests = 0
    for row in path:
        nodes = [int(n) for n in row if n >= 0]
        if not nodes:
            continue
        targets += len(nodes)
        for i, c in enumerate(nodes):
            if c not in first:
                continue
            nxt = nodes[i + 1] if i + 1 < len(nodes) else None
            drafts += nxt != first[c]
            kids = [n for n in range(1, len(parents)) if parents[n] == c]
            tests += len(kids) if nxt is None else kids.index(nxt) + 1
    return targets, drafts, tests


def algorithmic_bytes(workload: int, B: int, K: int, V: int, top_k: int, accept_len=None, esz: int = 2,
                      tree_path=None, parents=None) -> float:
    """Bytes the dominant kernel must move per launch (see the design notes).  For the trees,
    K is the node count N."""
    if workload == 8:
        # target rows 0..K-1 and every draft row once, alpha written
        return B * K * V * (esz + 4) + B * K * 4
    if workload == 7:
        # every row that moves read and written once (rows t = 1..d of each path with
        # path[t] != t, in every plane), the path, prefix and length read and the new length
        # written; tree_path is the committed path array [B, D+1]
        import numpy as np
        planes, rb = K, top_k
        moved = sum(int(np.count_nonzero(tree_path[b, 1:d + 1] != np.arange(1, d + 1)))
                    for b, d in enumerate(accept_len) if d > 0)
        return 2 * planes * moved * rb + B * (8 + 4) + B * tree_path.shape[1] * 4
    if workload == 6:
        # every draft row once; per chunk a sorted list of top_k (value, index) pairs plus count
        # and flags written; the children (token, value) and the kept indices written
        # (K is the number of expanded nodes E; the workload keeps k_next = top_k)
        chunks = B * K * select_chunks(V, 4)
        return B * K * V * 4 + chunks * (top_k * 8 + 8) + B * K * top_k * 8 + B * top_k * 4
    if workload == 5:
        # the walk: each visited node's target row once, the draft row of each visited node
        # where a residual was formed, z[x] and q[x] of every child tested, the tokens and
        # uniforms read and the outputs written
        targets, drafts, tests = tree_walk_rows(tree_path, parents)
        D1 = tree_path.shape[1]
        return targets * V * esz + drafts * V * 4 + tests * (esz + 4) + B * (K * 8 + D1 * 8 + 4)
    if workload == 3:
        # the row statistics: every node row once, argmax and flags written
        return B * K * V * esz + B * K * 12
    if workload == 10:
        # the cut of every row needs every target row (bf16) and every draft row (fp32): each
        # once, and the cuts written
        return B * (K + 1) * V * 2 + B * K * V * 4 + B * (2 * K + 1) * 32
    if workload == 2:
        # every target row (bf16) and every draft row (fp32) once.  The chunk lists the
        # selection hands to the finishers (64 words of 8 bytes per chunk) are written and
        # read back within the launch while they sit in L2, and cleared there: they are
        # not counted (list_word_bytes gives their size)
        return B * (K + 1) * V * 2 + B * K * V * 4
    j = [K] * B if accept_len is None else [int(a) for a in accept_len]
    if workload == 1:
        # the all-rows route's draw, split over several workgroups per batch row: target row j
        # of each batch row and the draft row j when j < K, plus the row statistics of rows
        # 0..j and the tokens and uniforms read (the slices' partial sums, a few KB per batch
        # row written and read back by the finishing launch, are not counted)
        drafts = sum(1 for a in j if 0 <= a < K)
        return sum(1 for a in j if a >= 0) * V * esz + drafts * V * 4 + B * ((K + 1) * 24 + K * 8 + (K + 1) * 4)
    # the walk: target rows 0..j of each batch row once, the draft row j when j < K, the
    # gathered q[x_k], tokens and uniforms read, the outputs written
    rows = sum(a + 1 for a in j if a >= 0)
    drafts = sum(1 for a in j if 0 <= a < K)
    return rows * V * esz + drafts * V * 4 + B * (K * 12 + (K + 1) * 4 + (K + 2) * 4)


def list_word_bytes(B: int, K: int, V: int, esz: int = 2) -> int:
    """Hand-over words of a top-k chain launch: 64 words of 8 bytes per selection chunk."""
    chunks = B * (K + 1) * select_chunks(V, esz) + B * K * select_chunks(V, 4)
    return chunks * 64 * 8


def copy_probe(R, torch, args) -> int:
    """Plain device copy of 512 MiB per launch (bytes read = bytes written = 512 MiB)."""
    n = 512 << 20
    src = torch.empty(n, dtype=torch.uint8, device="cuda").fill_(7)
    dst = torch.empty(n, dtype=torch.uint8, device="cuda")
    for _ in range(args.warmup):
        R.copy_probe(src, dst)
    torch.cuda.synchronize()
    a = torch.cuda.Event(enable_timing=True)
    b = torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(args.steps):
        R.copy_probe(src, dst)
    b.record()
    torch.cuda.synchronize()
    us = a.elapsed_time(b) * 1e3 / args.steps
    print(json.dumps({"probe": "copy", "bytes_read": n, "bytes_written": n, "us_per_launch": us,
                      "GBps_read_plus_write": 2 * n / us / 1e3}), flush=True)
    return 0


def unfused_baseline(R, torch, ci, inputs, T, top_k, args) -> dict:
    """The same step without the fusion, for context: the library GEMM of torch (F.linear,
    bf16 logits written to memory), then spec_verify_chain on those logits."""
    h, w, q, x, u = inputs
    B, K1, H = h.shape
    K = K1 - 1
    dev = h.device
    tok = torch.empty((B, K1), dtype=torch.int32, device=dev)
    alen = torch.empty((B,), dtype=torch.int32, device=dev)
    ws = R.new_workspace(R.chain_workspace_bytes(B, K, w.shape[0], 1, T, top_k), dev)
    h2 = h.reshape(B * K1, H)

    def one():
        z = torch.nn.functional.linear(h2, w).reshape(B, K1, -1)
        R.verify_chain(z, q, x, u, T, top_k, out=(tok, alen), workspace=ws)

    n = max(10, args.steps // 4)
    for _ in range(5):
        one()
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(n):
        one()
    b.record()
    torch.cuda.synchronize()
    return {"ms_per_step": a.elapsed_time(b) / n, "steps": n,
            "what": "torch F.linear (bf16 logits [B, K+1, V] written to HBM) + spec_verify_chain"}


def read_probe_gbps(R, torch, dev) -> float:
    """Achievable streaming-read bandwidth: the library's read-only probe over 1 GiB
    (four times the Infinity Cache), 20 launches timed together."""
    n = 1 << 30
    src = torch.empty(n, dtype=torch.uint8, device=dev)
    sink = torch.zeros(1, dtype=torch.int32, device=dev)
    for _ in range(3):
        R.read_probe(src, sink)
    torch.cuda.synchronize()
    a = torch.cuda.Event(enable_timing=True)
    b = torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(20):
        R.read_probe(src, sink)
    b.record()
    torch.cuda.synchronize()
    return n / (a.elapsed_time(b) * 1e-3 / 20) / 1e9


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=400)
    ap.add_argument("--warmup", type=int, default=40)
    ap.add_argument("--workload", type=int, default=2, choices=sorted(WORKLOADS))
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-c4", action="store_true",
                    help="skip the B=512 K=8 chain (workload 4) that the default line carries under \"c4\"")
    ap.add_argument("--copy-probe", action="store_true",
                    help="time the library's plain copy kernel on 512 MiB instead (counter calibration)")
    args = ap.parse_args()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU only: the verification step shards over the batch with no "
              "exchange, so there is no multi-GPU path to time (run with --gpus 1).", file=sys.stderr)
        return 2

    import numpy as np
    import torch

    import rejection_sampling_verify_10_amd as R
    from rejection_sampling_verify_10_amd import workloads as W

    R.lib()                                   # fails loudly without the HIP library
    if args.copy_probe:
        return copy_probe(R, torch, args)
    wl = WORKLOADS[args.workload]
    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)

    t0 = time.time()
    ci = W.config(args.workload, seed=args.seed)
    top_p = wl.get("top_p", 1.0)
    tree = args.workload == 3
    arate = args.workload == 8
    sampled_tree = args.workload == 5
    expand = args.workload == 6
    kvc = args.workload == 7
    fused = args.workload == 9
    log(f"workload {args.workload}: {wl['name']} (inputs drawn in {time.time() - t0:.1f} s)")

    def to_dev(a):
        if a.dtype == np.uint16:
            return torch.from_numpy(a.view(np.int16)).to(dev).view(torch.bfloat16)
        return torch.from_numpy(a).to(dev)

    esz = 2 if getattr(ci, "dtype", W.DTYPE_F32) == W.DTYPE_BF16 else 4
    if tree:
        B, K, V, T, top_k = ci.B, ci.N, ci.V, 0.0, 0
        depth = [0] * K
        for n in range(1, K):
            depth[n] = depth[int(ci.parents[n])] + 1
        D = max(depth)
        base = [to_dev(ci.logits), to_dev(ci.node_tokens)]
        tok = torch.empty((B, D + 1), dtype=torch.int32, device=dev)
        path = torch.empty((B, D + 1), dtype=torch.int32, device=dev)
        alen = torch.empty((B,), dtype=torch.int32, device=dev)
        ws = R.new_workspace(R.tree_workspace_bytes(B, K, V, ci.dtype), dev)
        parents = ci.parents.tolist()
        rows_per_step = B * K                  # node rows verified
    elif kvc:
        # K: planes, top_k: bytes per row (for the algorithmic byte count)
        B, K, V, T, top_k = ci.B, ci.planes, ci.S, 1.0, ci.row * 2
        kv0 = torch.from_numpy(ci.kv.view(np.int16)).to(dev)
        base = [kv0, to_dev(ci.prefix), to_dev(ci.path), to_dev(ci.accept_len)]
        alen = to_dev(ci.accept_len)
        xn = torch.empty((B,), dtype=torch.int32, device=dev)
        rows_per_step = B                      # accepted paths committed
    elif expand:
        B, K, V, T, top_k = ci.B, ci.E, ci.V, 1.0, ci.top_k
        base = [to_dev(ci.draft_probs), to_dev(ci.node_values)]
        xt = torch.empty((B, K, top_k), dtype=torch.int32, device=dev)
        xv = torch.empty((B, K, top_k), dtype=torch.float32, device=dev)
        xn = torch.empty((B, ci.k_next), dtype=torch.int32, device=dev)
        alen = torch.zeros((B,), dtype=torch.int32, device=dev)
        ws = R.new_workspace(R.tree_expand_workspace_bytes(B, K, V, top_k), dev)
        rows_per_step = B * K                  # draft rows expanded
    elif sampled_tree:
        B, K, V, T, top_k = ci.B, ci.N, ci.V, ci.temperature, ci.top_k
        depth = [0] * K
        for n in range(1, K):
            depth[n] = depth[int(ci.parents[n])] + 1
        D = max(depth)
        base = [to_dev(ci.logits), to_dev(ci.draft_probs), to_dev(ci.node_tokens), to_dev(ci.uniforms)]
        tok = torch.empty((B, D + 1), dtype=torch.int32, device=dev)
        path = torch.empty((B, D + 1), dtype=torch.int32, device=dev)
        alen = torch.empty((B,), dtype=torch.int32, device=dev)
        parents = ci.parents.tolist()
        rows_per_step = B * K                  # node rows verified
        ws = R.new_workspace(R.tree_sample_workspace_bytes(B, K), dev)
    elif fused:
        B, K, V, T, top_k = ci.B, ci.K, ci.V, ci.temperature, ci.top_k
        Hd = ci.H
        base = [to_dev(ci.hidden), to_dev(ci.weight), to_dev(ci.draft_probs), to_dev(ci.draft_tokens),
                to_dev(ci.uniforms)]
        tok = torch.empty((B, K + 1), dtype=torch.int32, device=dev)
        alen = torch.empty((B,), dtype=torch.int32, device=dev)
        ws = R.new_workspace(R.chain_fused_workspace_bytes(B, K, V, Hd, T, top_k), dev)
        rows_per_step = B * (K + 1)            # token rows verified
    elif arate:
        B, K, V, T, top_k = ci.B, ci.K, ci.V, ci.temperature, ci.top_k
        base = [to_dev(ci.logits), to_dev(ci.draft_probs)]
        alpha_out = torch.empty((B, K), dtype=torch.float32, device=dev)
        alen = torch.zeros((B,), dtype=torch.int32, device=dev)
        ws = R.new_workspace(R.accept_rate_workspace_bytes(B, K, V, ci.dtype, T, top_k), dev)
        rows_per_step = B * K                  # (target, draft) row pairs compared
    else:
        B, K, V, T, top_k = ci.B, ci.K, ci.V, ci.temperature, ci.top_k
        base = [to_dev(ci.logits), to_dev(ci.draft_probs), to_dev(ci.draft_tokens), to_dev(ci.uniforms)]
        tok = torch.empty((B, K + 1), dtype=torch.int32, device=dev)
        alen = torch.empty((B,), dtype=torch.int32, device=dev)
        ws = R.new_workspace(R.chain_workspace_bytes(B, K, V, ci.dtype, T, top_k), dev)
        rows_per_step = B * (K + 1)            # token rows verified
    sets = [base] + [[t.clone() for t in base] for _ in range(wl["copies"] - 1)]
    in_bytes = sum(t.numel() * t.element_size() for t in base)
    log(f"{wl['copies']} input copies x {in_bytes / 1e6:.1f} MB resident")

    def step(i: int) -> None:
        if tree:
            z, nt = sets[i % len(sets)]
            R.verify_tree_greedy(z, nt, parents, out=(path, tok, alen), workspace=ws)
        elif kvc:
            kv, pre, pth, al = sets[i % len(sets)]
            R.kv_commit(kv, pre, pth, al, ci.N, out_len=xn)
        elif expand:
            q, nv = sets[i % len(sets)]
            R.tree_expand(q, nv, top_k, ci.k_next, out=(xt, xv, xn), workspace=ws)
        elif sampled_tree:
            z, q, nt, u = sets[i % len(sets)]
            R.verify_tree_sample(z, q, nt, u, parents, T, top_k, out=(path, tok, alen), workspace=ws)
        elif arate:
            z, q = sets[i % len(sets)]
            R.accept_rate(z, q, T, top_k, out=alpha_out, workspace=ws)
        elif fused:
            h, w, q, x, u = sets[i % len(sets)]
            R.verify_chain_fused(h, w, q, x, u, T, top_k, out=(tok, alen), workspace=ws)
        else:
            z, q, x, u = sets[i % len(sets)]
            R.verify_chain(z, q, x, u, T, top_k, top_p, out=(tok, alen), workspace=ws)

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()

    # Timed region: K steps back to back, events only around the whole region.
    t_begin = torch.cuda.Event(enable_timing=True)
    t_end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t_begin.record()
    for i in range(args.steps):
        step(args.warmup + i)
    t_end.record()
    torch.cuda.synchronize()
    ms_step = t_begin.elapsed_time(t_end) / args.steps

    # Kernel pass: K more steps, the library attaching events to the dispatch of the
    # dominant kernel of each on the call's stream.
    kstart = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps)]
    kstop = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps)]
    for e in kstart + kstop:
        e.record()
    torch.cuda.synchronize()
    for i in range(args.steps):
        R.profile_next_call(kstart[i], kstop[i])
        step(args.warmup + args.steps + i)
    torch.cuda.synchronize()
    k_ms = sum(a.elapsed_time(b) for a, b in zip(kstart, kstop)) / args.steps
    single_kernel = wl.get("single_kernel", False)
    if single_kernel:
        # the kernel is the whole call: its time cannot exceed the step time of the timed pass
        k_ms = min(k_ms, ms_step)
    value = rows_per_step / (ms_step * 1e-3)
    unit = {3: "node-rows/s", 5: "node-rows/s", 6: "expanded draft rows/s", 7: "committed paths/s",
            8: "row pairs/s"}.get(args.workload, "token-rows/s")
    al = alen.cpu().numpy()
    extra = {}
    if fused:
        # the dominant kernel is the GEMM: 2*R*V*H flops on the matrix cores; the bytes
        # every step must read are the head, the hidden states and the draft rows
        flops = 2.0 * B * (K + 1) * V * Hd
        alg = V * Hd * 2 + B * (K + 1) * Hd * 2 + B * K * V * 4
        achieved = flops / (k_ms * 1e-3) / 1e12
        log(f"step {ms_step * 1e3:.1f} us, {wl['kernel']} {k_ms * 1e3:.1f} us -> {achieved:.0f} TFLOP/s "
            f"({100 * achieved / PEAK_BF16_TFLOPS:.1f}% of the bf16 peak); accept_len histogram "
            f"{np.bincount(al[al >= 0], minlength=K + 1).tolist()}")
        extra["unfused"] = unfused_baseline(R, torch, ci, sets[0], T, top_k, args)
        log(f"unfused (library GEMM to bf16 logits, then spec_verify_chain): "
            f"{extra['unfused']['ms_per_step'] * 1e3:.1f} us per step")
        probe = None
    else:
        alg = algorithmic_bytes(args.workload, B, K, V, top_k, al, esz,
                                path.cpu().numpy() if sampled_tree else ci.path if kvc else None,
                                ci.parents if sampled_tree else None)
        achieved = alg / (k_ms * 1e-3) / 1e9
        log(f"step {ms_step * 1e3:.1f} us, {wl['kernel']} {k_ms * 1e3:.1f} us -> {achieved:.0f} GB/s "
            f"({100 * achieved / PEAK_HBM_GBS:.1f}% of peak)"
            + ("" if (expand or kvc or arate) else "; accept_len histogram "
               f"{np.bincount(al[al >= 0], minlength=(K + 1) if not (tree or sampled_tree) else 1).tolist()}"))
        probe = read_probe_gbps(R, torch, dev)
        log(f"read probe {probe:.0f} GB/s; {wl['kernel']} at {100 * achieved / probe:.1f}% of it")
    step_alg_gbs = alg / (ms_step * 1e-3) / 1e9
    traffic = counter_traffic(args.workload)

    cpu = None
    if not args.no_cpu_baseline:
        import oracle

        def oracle_rate(rows: int, budget_s: float):
            """The oracle over the first `rows` batch rows, repeated until about budget_s of
            wall time so that the rate is stable; data generation is not timed."""
            reps = 0
            t0 = time.perf_counter()
            while True:
                if tree:
                    oracle.verify_tree_greedy(ci.logits[:rows], ci.dtype, ci.node_tokens[:rows], ci.parents)
                elif kvc:
                    oracle.kv_commit(ci.kv[:, :rows], ci.prefix[:rows], ci.path[:rows], ci.N, ci.accept_len[:rows])
                elif expand:
                    oracle.tree_expand(ci.draft_probs[:rows], ci.node_values[:rows], top_k, ci.k_next)
                elif sampled_tree:
                    oracle.verify_tree_sample(ci.logits[:rows], ci.dtype, ci.draft_probs[:rows],
                                              ci.node_tokens[:rows], ci.uniforms[:rows], ci.parents, T, top_k)
                elif arate:
                    oracle.accept_rate(ci.logits[:rows], ci.dtype, ci.draft_probs[:rows], T, top_k)
                elif fused:
                    z64 = oracle.lm_head_logits(ci.hidden[:rows], ci.weight)
                    oracle.verify_chain(z64, oracle.F64, ci.draft_probs[:rows], ci.draft_tokens[:rows],
                                        ci.uniforms[:rows], T, top_k)
                else:
                    oracle.verify_chain(ci.logits[:rows], ci.dtype, ci.draft_probs[:rows], ci.draft_tokens[:rows],
                                        ci.uniforms[:rows], T, top_k, top_p)
                reps += 1
                dt = time.perf_counter() - t0
                if dt >= budget_s or reps >= 200:
                    return reps * rows * rows_per_step / B / dt, reps, dt

        rows = min(wl["oracle_rows"], B)
        threads = oracle.max_threads()
        rate, reps, dt = oracle_rate(rows, 1.5)
        # one thread: a smaller sample of the same rows (about a second of work)
        oracle.set_threads(1)
        try:
            rows1 = max(1, min(rows, rows // threads if rows >= threads else rows))
            rate1, reps1, dt1 = oracle_rate(rows1, 1.0)
        finally:
            oracle.set_threads(threads)
        cpu = {"value": rate, "unit": unit, "cores": threads, "kind": "oracle",
               "sample": f"first {rows} of {B} batch rows ({rows * rows_per_step // B} {unit[:-2]}) of the same workload, "
                         f"{reps} passes, fp64 C oracle, OpenMP over batch rows, {dt:.2f} s wall",
               "single_thread": {"value": rate1, "unit": unit, "cores": 1,
                                 "sample": f"first {rows1} batch rows, {reps1} passes, {dt1:.2f} s"}}
        log(f"oracle: {rate:.0f} {unit} on {threads} threads, {rate1:.0f} on one")

    line = {
        "metric": METRIC if args.workload == 2 else f"{unit} and achieved HBM GB/s (% of peak), {wl['name']}",
        "value": value,
        "unit": unit,
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": wl["dtype"],
        "data": "synthetic",
        "config": ({"workload": wl["name"], "B": B, "N": K, "V": V, "input_copies": wl["copies"],
                    "parallelism": "single GPU"} if tree else
                   {"workload": wl["name"], "B": B, "N": K, "V": V, "temperature": T, "top_k": top_k,
                    "input_copies": wl["copies"], "parallelism": "single GPU"} if sampled_tree else
                   {"workload": wl["name"], "B": B, "E": K, "V": V, "top_k": top_k, "k_next": ci.k_next,
                    "rows": "expanded draft rows", "input_copies": wl["copies"], "parallelism": "single GPU"}
                   if expand else
                   {"workload": wl["name"], "B": B, "planes": K, "S": V, "row_bytes": top_k, "tree_nodes": ci.N,
                    "rows": "committed paths", "input_copies": wl["copies"], "parallelism": "single GPU"}
                   if kvc else
                   {"workload": wl["name"], "B": B, "K": K, "V": V, "temperature": T, "top_k": top_k,
                    "rows": "(target, draft) row pairs", "input_copies": wl["copies"], "parallelism": "single GPU"}
                   if arate else
                   {"workload": wl["name"], "B": B, "K": K, "V": V, "H": Hd, "temperature": T, "top_k": top_k,
                    "input_copies": wl["copies"], "parallelism": "single GPU"}
                   if fused else
                   {"workload": wl["name"], "B": B, "K": K, "V": V, "temperature": T, "top_k": top_k,
                    **({"top_p": top_p} if top_p < 1.0 else {}),
                    "input_copies": wl["copies"], "parallelism": "single GPU"}),
        "step_algorithmic_GBps": step_alg_gbs,
        "emitted_tokens_per_s": None if arate else float(np.sum(al[al >= 0] + 1)) / (ms_step * 1e-3),
        "roofline": ({"bound": "mfma", "kernel": wl["kernel"], "achieved": achieved, "peak": PEAK_BF16_TFLOPS,
                      "unit": "TFLOP/s", "frac": achieved / PEAK_BF16_TFLOPS, "traffic": traffic,
                      "kernel_us": k_ms * 1e3, "flops": 2.0 * B * (K + 1) * V * Hd,
                      "kernel_timing": "HIP events attached to the GEMM kernel's dispatch on the call's stream, "
                                       "second pass of the same number of steps"} if fused else
                     {"bound": "hbm", "kernel": wl["kernel"], "achieved": achieved, "peak": PEAK_HBM_GBS,
                      "unit": "GB/s", "frac": achieved / PEAK_HBM_GBS, "traffic": traffic,
                      "kernel_us": k_ms * 1e3, "algorithmic_bytes": alg,
                      "kernel_timing": "HIP events attached to the kernel's dispatch (hipExtLaunchKernel) on "
                                       "the call's stream, second pass of the same number of steps"
                                       + (", capped by the timed pass's step time (the kernel is the whole call)"
                                          if single_kernel else ""),
                      "read_probe_GBps": probe, "frac_of_read_probe": achieved / probe}),
        "cpu_baseline": cpu,
    }
    if args.workload == 4:
        # The walk reads target rows only up to the first rejection.  The bytes of the
        # route that reduces every row first (every target row once, plus the draft row of
        # each residual draw) put its step time beside a full read of the batch.
        drafts = int(np.sum((al >= 0) & (al < K)))
        all_rows = B * (K + 1) * V * esz + drafts * V * 4
        line["roofline"]["all_rows_bytes"] = all_rows
        line["roofline"]["all_rows_equivalent_frac"] = all_rows / (ms_step * 1e-3) / 1e9 / PEAK_HBM_GBS
    line.update(extra)
    if args.workload == 2 and not args.no_c4:
        line["c4"] = c4_line(args)
    print(json.dumps(line), flush=True)
    return 0


def c4_line(args) -> dict | None:
    """Workload 4 (the dense chain B=512 K=8 V=128256, T=1) in a child process with the
    same steps and warmup: its step time, rows/s and the walk kernel's roofline, so the
    default line carries the large dense batch beside the headline top-k chain."""
    import subprocess
    cmd = [sys.executable, os.path.abspath(__file__), "--workload", "4", "--no-cpu-baseline",
           "--steps", str(args.steps), "--warmup", str(args.warmup), "--seed", str(args.seed)]
    log("workload 4 in a child process for the c4 keys")
    r = subprocess.run(cmd, stdout=subprocess.PIPE, text=True, timeout=600)
    if r.returncode != 0:
        log(f"workload 4 failed with status {r.returncode}")
        return None
    c4 = json.loads(r.stdout.strip().splitlines()[-1])
    keep = ("workload", "B", "K", "V", "temperature", "top_k")
    return {"workload": {k: c4["config"][k] for k in keep}, "value": c4["value"], "unit": c4["unit"],
            "ms_per_step": c4["ms_per_step"], "emitted_tokens_per_s": c4["emitted_tokens_per_s"],
            "roofline": {k: c4["roofline"][k] for k in
                         ("bound", "kernel", "achieved", "peak", "unit", "frac", "traffic", "kernel_us",
                          "algorithmic_bytes", "all_rows_bytes", "all_rows_equivalent_frac")}}


if __name__ == "__main__":
    sys.exit(main())
