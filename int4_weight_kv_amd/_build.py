"""Builds libfutx.so (HIP for gfx950 + host C++) in the package directory.

Usage: python -m int4_weight_kv_amd._build [--changed]   (or __graft_entry__.build()).
Recompiles every source; with --changed, only sources whose object is older
than the source or any header.
"""

import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libfutx.so")

HIP_SOURCES = ["kernels.hip", "gemm.hip", "head.hip", "abi.hip", "noalloc.hip", "measure.hip", "fp8.hip"]
CPP_SOURCES = ["pack.cpp"]
ARCH = "gfx950"

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
HIP_FLAGS = [
    f"--offload-arch={ARCH}",
    "-O3",
    "-std=c++17",
    "-fPIC",
    # packed fp32 VALU forms are kept out of the generated code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", INCLUDE,
    "-I", CSRC,
]
CXX_FLAGS = ["-O2", "-std=c++17", "-fPIC", "-pthread", "-I", INCLUDE, "-I", CSRC]


def _run(cmd):
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        sys.stderr.write(r.stdout + r.stderr)
        raise RuntimeError("build step failed: " + " ".join(cmd))
    return r


def _stale(src, obj):
    if not os.path.exists(obj):
        return True
    heads = [os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith(".h")]
    heads += [os.path.join(INCLUDE, f) for f in os.listdir(INCLUDE) if f.endswith(".h")]
    newest = max(os.path.getmtime(f) for f in [src] + heads)
    return os.path.getmtime(obj) < newest


def build(verbose=False, changed_only=False):
    os.makedirs(BUILD, exist_ok=True)
    jobs, objs = [], []
    for src in HIP_SOURCES + CPP_SOURCES:
        path = os.path.join(CSRC, src)
        obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
        objs.append(obj)
        if changed_only and not _stale(path, obj):
            continue
        if src.endswith(".hip"):
            jobs.append([HIPCC, *HIP_FLAGS, "-c", path, "-o", obj])
        else:
            jobs.append([shutil.which("g++") or "g++", *CXX_FLAGS, "-c", path, "-o", obj])
    if jobs:
        with ThreadPoolExecutor(max_workers=min(8, len(jobs))) as ex:
            list(ex.map(_run, jobs))
    tmp = LIB + ".tmp"
    _run([HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-pthread", "-o", tmp, *objs])
    os.replace(tmp, LIB)
    if verbose:
        print("built", LIB)
    return LIB


if __name__ == "__main__":
    build(verbose=True, changed_only="--changed" in sys.argv[1:])
