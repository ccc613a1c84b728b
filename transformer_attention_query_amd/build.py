"""Build ``librelattn.so`` in-tree with hipcc for gfx950.

Usage: ``python -m transformer_attention_query_amd.build`` (or
``__graft_entry__.build()``).  Each source is compiled to an object under
``_build/`` in parallel, then linked into the package directory, where the
binding loads it from.
"""

from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD_DIR = os.path.join(ROOT, "_build")
LIB = os.path.join(HERE, "librelattn.so")
# yardstick kernels for bench.py (streaming read, MFMA, exp, LDS, clock; not part of the ABI)
PROBE_SOURCE = "ceilings.hip"
PROBE_LIB = os.path.join(HERE, "libceilings.so")

SOURCES = ["api.cpp", "prefill.hip", "decode.hip", "rel_logits.hip", "prologue.hip", "mx.hip", "backward.hip"]
ARCH = "gfx950"

# Packed fp32 VALU ops are switched off for every device pass (the compiler
# would otherwise form v_pk_* from ordinary float code).  MFMAs are kept in
# their VGPR form: the kernels fit in 256 VGPRs, and the AGPR form would cost
# accumulator copies on every VALU touch.
DEVICE_FLAGS = ["-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", "-mllvm", "-amdgpu-mfma-vgpr-form"]
COMMON_FLAGS = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}", "-I", INCLUDE, "-I", CSRC,
                "-Wall", "-Wno-unused-function"]


def hipcc() -> str:
    path = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(path):
        raise RuntimeError("hipcc not found")
    return path


def _compile(src: str) -> str:
    obj = os.path.join(BUILD_DIR, os.path.splitext(src)[0] + ".o")
    lang = ["-x", "hip"]
    cmd = [hipcc(), *COMMON_FLAGS, *DEVICE_FLAGS, *lang, "-c", os.path.join(CSRC, src), "-o", obj]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"compile of {src} failed:\n{' '.join(cmd)}\n{res.stdout}\n{res.stderr}")
    warn = "\n".join(l for l in res.stderr.splitlines() if "packed-fp32-ops" not in l and l.strip())
    if warn:
        print(warn, file=sys.stderr)
    return obj


def build(verbose: bool = True) -> str:
    """Compile every source and link the shared library; returns its path."""
    os.makedirs(BUILD_DIR, exist_ok=True)
    with cf.ThreadPoolExecutor(max_workers=min(len(SOURCES), os.cpu_count() or 4)) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = LIB + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"link failed:\n{' '.join(cmd)}\n{res.stdout}\n{res.stderr}")
    os.replace(tmp, LIB)
    probe_obj = _compile(PROBE_SOURCE)
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", probe_obj, "-o", PROBE_LIB + ".tmp"]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"link failed:\n{' '.join(cmd)}\n{res.stdout}\n{res.stderr}")
    os.replace(PROBE_LIB + ".tmp", PROBE_LIB)
    if verbose:
        print(f"built {LIB} and {PROBE_LIB}")
    return LIB


if __name__ == "__main__":
    build()
