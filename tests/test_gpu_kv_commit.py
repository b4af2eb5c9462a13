"""Parity of spec_kv_commit with the CPU oracle (bit-exact: it moves bytes)."""

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


def run(R, orc, k, name, kv=None, path=None, alen=None, layout="planes-first", prefix=None, capacity=None):
    import torch
    kv = k.kv if kv is None else kv
    path = k.path if path is None else path
    alen = k.accept_len if alen is None else alen
    prefix = k.prefix if prefix is None else prefix
    print(f"[case] kv commit {name}: B={k.B} planes={kv.shape[0]} S={kv.shape[2]} row={kv.shape[3:]} {layout}",
          flush=True)
    want, want_len = orc.kv_commit(kv, prefix, path, k.N, alen, capacity=capacity)
    if layout == "batch-first":                      # planes strided over the batch: [B, planes, S, row] memory
        dev = torch.from_numpy(np.ascontiguousarray(kv.swapaxes(0, 1))).cuda().transpose(0, 1)
    else:
        dev = torch.from_numpy(np.ascontiguousarray(kv)).cuda()
    nl = R.kv_commit(dev, to_torch(prefix), to_torch(path), to_torch(alen), k.N, capacity=capacity)
    torch.cuda.synchronize()
    assert np.array_equal(nl.cpu().numpy(), want_len), name
    assert np.array_equal(dev.cpu().numpy(), want), name
    return want_len


@pytest.mark.parametrize("row", [1024, 10])
def test_rows_past_the_capacity(R, orc, row):
    """Batch rows whose path reaches past the cache (prefix + path[d] >= capacity, or a prefix
    beyond it) are error rows that move nothing; the check runs before any load, so the
    kernel never touches memory past the cache.  A path ending on the last position moves."""
    k = W.make_kv_commit(16, planes=3, row=row, max_prefix=6, config_id=77, seed=row)
    S = k.kv.shape[2]
    pre = k.prefix.copy()
    last = k.path[np.arange(k.B), k.accept_len]
    pre[0] = S - 1 - last[0]                          # exactly fits
    pre[1] = S - last[1]                              # one row past the end
    pre[2] = 2 ** 30                                  # far past the end
    pre[3] = S - 1 - last[3]
    nl = run(R, orc, k, f"capacity row={row}", prefix=pre)
    assert nl[0] >= 0 and nl[1] == -1 and nl[2] == -1
    cap = S - 3
    nl = run(R, orc, k, f"capacity {cap} row={row}", prefix=pre, capacity=cap)
    assert nl[0] == -1 and nl[3] == -1


def test_workload7_full(R, orc):
    """64 planes (32 layers x K, V), B=64, 2 KiB rows (8 heads x 128 x bf16): the launch bench.py times."""
    run(R, orc, W.config(7, 0), "workload 7")


@pytest.mark.parametrize("row,dtype", [(8, np.uint16), (10, np.uint16), (3, np.uint8), (8192, np.uint16)])
def test_row_shapes(R, orc, row, dtype):
    """16-byte rows (vectors), 20-byte rows (4-byte words), 3-byte rows (bytes), and 16 KiB
    rows (more than a block stages: one row at a time)."""
    k = W.make_kv_commit(12, planes=3, row=row, max_prefix=9, config_id=73, seed=row)
    kv = k.kv.astype(dtype) if dtype != np.uint16 else k.kv
    run(R, orc, k, f"row={row}", kv=kv)


def test_strided_planes_overlapping_paths_and_errors(R, orc):
    k = W.make_kv_commit(10, planes=4, row=64, max_prefix=6, config_id=74, seed=0)
    path, alen = k.path.copy(), k.accept_len.copy()
    path[0, :4] = [0, 2, 3, 7]                       # destinations that are other moves' sources
    path[0, 4:] = -1
    alen[0] = 3
    alen[1] = -1                                     # error rows: nothing moves
    path[2, 0] = 5
    path[3, 1] = k.N
    alen[3] = max(alen[3], 1)
    run(R, orc, k, "strided, overlapping, errors", path=path, alen=alen, layout="batch-first")


@pytest.mark.parametrize("row", [8, 1024])
def test_longest_paths(R, orc, row):
    """A 64-node path tree (the most nodes a tree has): paths of every depth up to 63, so the
    path check uses every lane; 16-byte rows are staged whole, 2 KiB rows past 8 moving rows
    move one at a time."""
    k = W.make_kv_commit(96, planes=2, row=row, parents=np.arange(-1, 63, dtype=np.int32), max_prefix=3,
                         config_id=75, seed=row)
    assert k.path.shape[1] == 64 and k.accept_len.max() >= 60
    alen = k.accept_len.copy()
    path = k.path.copy()
    alen[0] = 63
    path[0] = np.arange(64, dtype=np.int32)          # the whole tree accepted: nothing moves
    run(R, orc, k, f"longest paths row={row}", path=path, alen=alen)
