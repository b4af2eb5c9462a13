"""Builds libspecverify.so (the C-ABI HIP library) for gfx950, in-tree.

    python -m rejection_sampling_verify_10_amd.build
"""

from __future__ import annotations

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
ROOT = os.path.dirname(HERE)
LIB = os.path.join(HERE, "libspecverify.so")
SOURCES = ["alpha.hip", "api.hip", "dense_tr.hip", "dense_walk.hip", "eagle2.hip", "kv_commit.hip", "lmhead.hip", "nucleus.hip", "rowstats.hip",
           "topk.hip", "tree_cluster.hip", "tree_sample.hip", "verify.hip"]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-Wall",
    # packed fp32 VALU forms stay off: plain float code only
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", os.path.join(ROOT, "include"),
]


def build(verbose: bool = False) -> str:
    """Compile every source and link the shared library; returns its path."""
    objdir = os.path.join(HERE, "_build")
    os.makedirs(objdir, exist_ok=True)

    def compile_one(src: str) -> str:
        obj = os.path.join(objdir, src.replace(".hip", ".o"))
        cmd = [HIPCC, *FLAGS, "-c", os.path.join(CSRC, src), "-o", obj]
        r = subprocess.run(cmd, capture_output=True, text=True)
        msg = "\n".join(l for l in (r.stdout + r.stderr).splitlines()
                        if "packed-fp32-ops" not in l and l.strip())
        if r.returncode != 0:
            raise RuntimeError(f"hipcc failed for {src}:\n{msg}")
        if verbose and msg:
            print(msg, file=sys.stderr)
        return obj

    with ThreadPoolExecutor(len(SOURCES)) as ex:
        objs = list(ex.map(compile_one, SOURCES))
    tmp = LIB + ".tmp"
    r = subprocess.run([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp, *objs],
                       capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}{r.stderr}")
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
