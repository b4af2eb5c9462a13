"""Host-side sanitizer builds: the oracle and the C-ABI library's host code under
AddressSanitizer and UndefinedBehaviorSanitizer.

- The oracle (plain C) is rebuilt with gcc and -fsanitize=address,undefined, and the oracle
  pins run against it in a child process (ORACLE_LIBRARY points the wrapper at it).
- The library's entry points (argument checks, workspace sizing and carving) are rebuilt
  with the sanitizers on the host side only, linked with the ordinary kernel objects, and
  the ABI tests run against it (SPEC_VERIFY_LIBRARY).  No GPU code is instrumented and no
  kernel is launched.
Each child preloads its compiler's sanitizer runtime; any report aborts the child.
"""

import glob
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")


def _child(env_extra, tests, tmp_path):
    env = dict(os.environ)
    env.update(env_extra)
    env["OMP_NUM_THREADS"] = "4"
    r = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider", "-m", "not gpu",
                        *tests], cwd=ROOT, env=env, capture_output=True, text=True, timeout=900)
    assert r.returncode == 0, (r.stdout[-4000:] + "\n" + r.stderr[-4000:])
    return r.stdout


@pytest.mark.slow
def test_oracle_pins_under_asan_ubsan(tmp_path):
    lib = str(tmp_path / "liboracle_san.so")
    subprocess.check_call(["gcc", "-O1", "-g", "-std=c11", "-fopenmp", "-fPIC", "-shared", "-fno-omit-frame-pointer",
                           "-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-o", lib,
                           os.path.join(ROOT, "oracle", "spec_oracle.c"), "-lm"])
    runtime = ":".join(subprocess.check_output(["gcc", f"-print-file-name={n}"], text=True).strip()
                       for n in ("libasan.so", "libubsan.so"))
    out = _child({"ORACLE_LIBRARY": lib, "LD_PRELOAD": runtime,
                  "ASAN_OPTIONS": "detect_leaks=0:abort_on_error=1",
                  "UBSAN_OPTIONS": "halt_on_error=1:print_stacktrace=1"},
                 ["tests/test_oracle_pins.py", "tests/test_oracle_margins.py", "tests/test_oracle_tree_sample.py",
                  "tests/test_oracle_eagle2.py"], tmp_path)
    assert "passed" in out


@pytest.mark.slow
def test_abi_host_code_under_asan_ubsan(tmp_path):
    from rejection_sampling_verify_10_amd import build
    objdir = os.path.join(ROOT, "rejection_sampling_verify_10_amd", "_build")
    others = [os.path.join(objdir, s.replace(".hip", ".o")) for s in build.SOURCES if s != "api.hip"]
    if not all(os.path.exists(o) for o in others):
        build.build()
    api_o = str(tmp_path / "api_san.o")
    lib = str(tmp_path / "libspecverify_san.so")
    flags = [f for f in build.FLAGS if f != "-O3"]
    subprocess.check_call([HIPCC, *flags, "-O1", "-g", "-Xarch_host", "-fsanitize=address",
                           "-Xarch_host", "-fsanitize=undefined", "-Xarch_host", "-fno-sanitize-recover=all",
                           "-c", os.path.join(ROOT, "rejection_sampling_verify_10_amd", "csrc", "api.hip"),
                           "-o", api_o])
    subprocess.check_call([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-Xarch_host", "-fsanitize=address",
                           "-Xarch_host", "-fsanitize=undefined", "-shared-libasan", "-o", lib, api_o, *others])
    rt = glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so")
    assert rt, "clang's AddressSanitizer runtime is missing"
    out = _child({"SPEC_VERIFY_LIBRARY": lib, "LD_PRELOAD": rt[0],
                  "ASAN_OPTIONS": "detect_leaks=0:abort_on_error=1",
                  "UBSAN_OPTIONS": "halt_on_error=1:print_stacktrace=1"},
                 ["tests/test_abi.py"], tmp_path)
    assert "passed" in out
