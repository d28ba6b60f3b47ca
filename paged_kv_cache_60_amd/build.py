"""Build libpagedkv.so in-tree for gfx950.

    python -m paged_kv_cache_60_amd.build

HIP sources are compiled with hipcc for gfx950 only, with packed fp32 vector
instructions disabled; the host-only block manager is compiled with g++.
Objects go to ``_build/`` at the repository root; the library is written next
to this file, where the Python binding loads it.
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
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libpagedkv.so")

HIP_SOURCES = ["kv_write.hip", "block_copy.hip", "attn_decode.hip", "attn_prefill.hip", "step_meta.hip"]
CXX_SOURCES = ["block_manager.cpp"]

ARCH = "gfx950"
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
HIP_FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-Wall", "-Wno-unused-function",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", os.path.join(ROOT, "include"),
]
# per-source extra flags: the matrix-core kernels (prefill, grouped-head decode)
# keep their accumulators in ordinary VGPRs; in the accumulator-register form the
# compiler copied every output accumulator out and back on each iteration of
# the token loop (64 per step in prefill, 32 per unit in decode)
VGPR_FORM = ["-mllvm", "-amdgpu-mfma-vgpr-form"]
HIP_EXTRA = {"attn_prefill.hip": VGPR_FORM, "attn_decode.hip": VGPR_FORM}
CXX_FLAGS = ["-O2", "-std=c++17", "-fPIC", "-Wall", "-I", os.path.join(ROOT, "include")]


def _run(cmd):
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"command failed ({r.returncode}): {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    return r


def build(verbose: bool = False) -> str:
    """Compile every source and link libpagedkv.so; returns its path."""
    if not os.path.exists(HIPCC):
        raise RuntimeError(f"hipcc not found at {HIPCC}")
    os.makedirs(BUILD, exist_ok=True)
    jobs = []
    for src in HIP_SOURCES:
        obj = os.path.join(BUILD, src.replace(".hip", ".o"))
        jobs.append([HIPCC, *HIP_FLAGS, *HIP_EXTRA.get(src, []), "-c", os.path.join(CSRC, src), "-o", obj])
    for src in CXX_SOURCES:
        obj = os.path.join(BUILD, src.replace(".cpp", ".o"))
        jobs.append([shutil.which("g++") or "g++", *CXX_FLAGS, "-c", os.path.join(CSRC, src), "-o", obj])
    with ThreadPoolExecutor(max_workers=min(8, len(jobs))) as ex:
        for r in ex.map(_run, jobs):
            if verbose and (r.stdout or r.stderr):
                print(r.stdout, r.stderr, file=sys.stderr)
    objs = [j[-1] for j in jobs]
    tmp = LIB + ".tmp"
    _run([HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs])
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
