"""Build libpkv.so (the HIP kernels and the C ABI) in-tree for gfx950.

Usage: ``python -m paged_kv_gqa_mapping_amd.build`` or ``build()`` from Python.
Every call recompiles; sources compile in parallel, then link into
``paged_kv_gqa_mapping_amd/libpkv.so``.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD_DIR = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libpkv.so")

SOURCES = ["api.cpp", "block_manager.cpp", "copy_kernels.hip", "row_attn.hip", "prefill_mfma.hip", "prefill_plan.hip", "rope_store.hip", "checks.hip"]

# gfx950 only.  Packed fp32 vector instructions are disabled for device code;
# the host pass does not know the feature and warns, which is harmless.
FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-Wall",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", os.path.join(ROOT, "include"),
]


def _hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build libpkv.so)")


def _run(cmd):
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    out = "\n".join(line for line in r.stdout.splitlines()
                    if "packed-fp32-ops" not in line and "ignoring feature" not in line)
    if r.returncode != 0:
        raise RuntimeError(f"command failed ({r.returncode}): {' '.join(cmd)}\n{out}")
    return out


def build(verbose: bool = False) -> str:
    hipcc = _hipcc()
    os.makedirs(BUILD_DIR, exist_ok=True)
    objs = []
    cmds = []
    for src in SOURCES:
        obj = os.path.join(BUILD_DIR, os.path.splitext(src)[0] + ".o")
        lang = ["-x", "hip"]
        cmds.append([hipcc, *FLAGS, *lang, "-c", os.path.join(CSRC, src), "-o", obj])
        objs.append(obj)
    workers = max(1, min(len(cmds), os.cpu_count() or 1, 16))
    with ThreadPoolExecutor(workers) as ex:
        for out in ex.map(_run, cmds):
            if verbose and out.strip():
                print(out)
    tmp = LIB + ".tmp"
    _run([hipcc, "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", tmp])
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
