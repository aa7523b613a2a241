"""Builds librkv.so (host radix tree + gfx950 HIP kernels) in-tree.

    python -m prefix_shared_kv_host_amd.build

Host C++ files are compiled with g++, HIP files with hipcc for gfx950, and
everything is linked by hipcc into prefix_shared_kv_host_amd/librkv.so.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
OUT = os.path.join(PKG, "librkv.so")
BUILD = os.path.join(PKG, "_build")

ARCH = os.environ.get("RKV_OFFLOAD_ARCH", "gfx950")
HIPCC = os.environ.get("HIPCC", shutil.which("hipcc") or "/opt/rocm/bin/hipcc")
CXX = os.environ.get("CXX", "g++")

HIP_FLAGS = [
    "-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
    # packed fp32 instructions are kept out of every kernel
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # kernels run with the IEEE mode bit off and never test for NaN, so max
    # and min need no quieting of their inputs (NaN still propagates through
    # arithmetic, which is how a gather of a poisoned slot shows up)
    "-mno-amdgpu-ieee", "-fno-honor-nans",
    "-Wno-unused-command-line-argument",
    f"-I{INCLUDE}", f"-I{CSRC}",
]
CXX_FLAGS = ["-O2", "-std=c++17", "-fPIC", "-Wall", "-Wextra", f"-I{INCLUDE}", f"-I{CSRC}"]


def _run(cmd):
    p = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    # the host pass of hipcc does not know the packed-fp32 feature; drop that note
    noise = "is not a recognized feature for this target"
    lines = [ln for ln in p.stdout.splitlines() if noise not in ln]
    if p.returncode != 0:
        raise RuntimeError("command failed:\n  " + " ".join(cmd) + "\n" + "\n".join(lines))
    return "\n".join(lines)


def sources():
    cpp = sorted(f for f in os.listdir(CSRC) if f.endswith(".cpp"))
    hip = sorted(f for f in os.listdir(CSRC) if f.endswith(".hip"))
    return cpp, hip


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    cpp, hip = sources()
    jobs = []
    for f in cpp:
        obj = os.path.join(BUILD, f + ".o")
        jobs.append([CXX, *CXX_FLAGS, "-c", os.path.join(CSRC, f), "-o", obj])
    for f in hip:
        obj = os.path.join(BUILD, f + ".o")
        jobs.append([HIPCC, *HIP_FLAGS, "-c", os.path.join(CSRC, f), "-o", obj])
    workers = min(len(jobs), int(os.environ.get("MAX_JOBS", "8")))
    with cf.ThreadPoolExecutor(max_workers=max(1, workers)) as ex:
        for out in ex.map(_run, jobs):
            if verbose and out.strip():
                print(out)
    objs = [os.path.join(BUILD, f + ".o") for f in cpp + hip]
    tmp = OUT + ".tmp"
    _run([HIPCC, "-shared", "-fPIC", f"--offload-arch={ARCH}", *objs, "-o", tmp])
    os.replace(tmp, OUT)
    return OUT


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
