"""Builds libpkv.so in-tree for gfx950.

Host files (allocator, errors) are plain C++17 built with g++; the kernels
and their launchers are HIP built with hipcc for --offload-arch=gfx950; the
shared library is linked by hipcc against the HIP runtime. Run as
``python -m paged_kv_cache_392_amd.build`` or through
``__graft_entry__.build()``.
"""

import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libpkv.so")

HOST_SOURCES = ["errors.cpp", "pool.cpp", "sched.cpp"]
HIP_SOURCES = ["kernels.hip"]

ARCH = "gfx950"
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
CXX = os.environ.get("CXX", "g++")

# Packed fp32 instructions are kept out of every code object. MFMA results
# go to ordinary VGPRs: with accumulation registers the compiler copied the
# multi-row attention's accumulators between the two files on every step.
HIP_FLAGS = [
    f"--offload-arch={ARCH}", "-mcode-object-version=5", "-O3", "-std=c++17", "-fPIC",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", "-mllvm", "-amdgpu-mfma-vgpr-form",
    "-Wall", "-Wno-unused-function",
]
HOST_FLAGS = ["-O2", "-std=c++17", "-fPIC", "-Wall", "-Wextra"]


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    if res.returncode != 0:
        sys.stderr.write(res.stdout)
        raise RuntimeError(f"build step failed: {' '.join(cmd)}")
    # hipcc's host pass warns about the gfx-only target feature: not an error
    out = "\n".join(l for l in res.stdout.splitlines() if "packed-fp32-ops" not in l)
    if verbose and out.strip():
        print(out)


def build(verbose=False):
    os.makedirs(BUILD, exist_ok=True)
    objs = []
    for src in HOST_SOURCES:
        obj = os.path.join(BUILD, src + ".o")
        _run([CXX, *HOST_FLAGS, "-I", INCLUDE, "-c", os.path.join(CSRC, src), "-o", obj], verbose)
        objs.append(obj)
    for src in HIP_SOURCES:
        obj = os.path.join(BUILD, src + ".o")
        _run([HIPCC, *HIP_FLAGS, "-I", INCLUDE, "-c", os.path.join(CSRC, src), "-o", obj], verbose)
        objs.append(obj)
    tmp = LIB + ".tmp"
    _run([HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp], verbose)
    os.replace(tmp, LIB)
    return LIB


def clean():
    shutil.rmtree(BUILD, ignore_errors=True)


if __name__ == "__main__":
    print(build(verbose=True))
