"""The host side of the library (argument checks, planning, the error
channel) under AddressSanitizer and UndefinedBehaviorSanitizer.

Every source is rebuilt with the sanitizers on its host pass only (device
code is built as usual and never runs here), into a temporary directory, and
the C-ABI tests (tests/test_abi.py, which call every entry point with bad,
edge and valid arguments that stop before any GPU work) run against that
library in a child process with the ASan runtime preloaded.  A sanitizer
report aborts the child (no recovery), which fails this test."""

import glob
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "transformer_attention_query_amd", "csrc")
SOURCES = ["api.cpp", "prefill.hip", "decode.hip", "rel_logits.hip", "prologue.hip", "mx.hip", "backward.hip"]
HOST_SANITIZE = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
                 "-Xarch_host", "-fno-sanitize-recover=all", "-Xarch_host", "-fno-omit-frame-pointer"]


def _hipcc():
    return shutil.which("hipcc") or ("/opt/rocm/bin/hipcc" if os.path.exists("/opt/rocm/bin/hipcc") else None)


def _asan_runtime(hipcc):
    out = subprocess.run([hipcc, "-print-file-name=libclang_rt.asan-x86_64.so"], capture_output=True, text=True)
    path = out.stdout.strip()
    if os.path.isabs(path) and os.path.exists(path):
        return path
    hits = glob.glob("/opt/rocm/lib/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so")
    return hits[0] if hits else None


def test_abi_tests_pass_under_host_sanitizers(tmp_path):
    hipcc = _hipcc()
    if hipcc is None:
        pytest.skip("hipcc not found")
    runtime = _asan_runtime(hipcc)
    if runtime is None:
        pytest.skip("ASan runtime not found")
    procs = []
    objs = []
    for src in SOURCES:
        obj = str(tmp_path / (os.path.splitext(src)[0] + ".o"))
        cmd = [hipcc, "-O1", "-g", "-std=c++17", "-fPIC", "--offload-arch=gfx950",
               "-I", os.path.join(ROOT, "include"), "-I", CSRC,
               "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", "-mllvm", "-amdgpu-mfma-vgpr-form",
               *HOST_SANITIZE, "-x", "hip", "-c", os.path.join(CSRC, src), "-o", obj]
        procs.append((src, subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)))
        objs.append(obj)
    for src, p in procs:
        out, _ = p.communicate()
        assert p.returncode == 0, f"sanitizer build of {src} failed:\n{out}"
    lib = str(tmp_path / "librelattn_sanitized.so")
    # the sanitizer runtime is preloaded in the child, so the link needs no runtime of its own
    link = subprocess.run([hipcc, "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", lib],
                          capture_output=True, text=True)
    assert link.returncode == 0, link.stdout + link.stderr
    env = dict(os.environ, RELATTN_LIBRARY=lib, LD_PRELOAD=runtime,
               ASAN_OPTIONS="detect_leaks=0:abort_on_error=1", UBSAN_OPTIONS="print_stacktrace=1")
    run = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider",
                          os.path.join(ROOT, "tests", "test_abi.py")],
                         cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    assert run.returncode == 0, f"ABI tests under ASan/UBSan failed:\n{run.stdout[-4000:]}\n{run.stderr[-4000:]}"
    assert " passed" in run.stdout
