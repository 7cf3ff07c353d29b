"""Builds libpkv.so in-tree for gfx950.

Host files (allocator, errors) are plain C++17 built with g++; the kernels
and their launchers are HIP built with hipcc for --offload-arch=gfx950; the
shared library is linked by hipcc against the HIP runtime. Run as a script,
``python paged_kv_cache_392_amd/build.py`` (importing the package opens the
library, so ``python -m`` cannot build it the first time), or through
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
    # hipcc's host pass warns about the gfx-only target feature: not an error;
    # resource remarks are parsed by the caller, not echoed
    out = "\n".join(l for l in res.stdout.splitlines() if "packed-fp32-ops" not in l)
    shown = "\n".join(l for l in out.splitlines() if "kernel-resource-usage" not in l and l.strip()
                      and not l.lstrip()[:1].isdigit() and l.strip() != "| ^" and "|" not in l[:8])
    if verbose and shown.strip():
        print(shown)
    return out


RESOURCES = os.path.join(BUILD, "kernel_resources.txt")
_FIELDS = {"VGPRs": "vgprs", "AGPRs": "agprs", "ScratchSize [bytes/lane]": "scratch", "VGPRs Spill": "vgpr_spill",
           "SGPRs Spill": "sgpr_spill", "Occupancy [waves/SIMD]": "occupancy", "LDS Size [bytes/block]": "lds"}


def parse_resources(text):
    """Per-kernel register, scratch, occupancy and LDS figures from the
    compiler's kernel-resource-usage remarks."""
    kernels, cur = [], None
    for line in text.splitlines():
        if "kernel-resource-usage" not in line or "remark:" not in line:
            continue
        body = line.split("remark:", 1)[1].rsplit("[-Rpass-analysis", 1)[0].strip()
        if body.startswith("Function Name:"):
            cur = {"name": body.split(":", 1)[1].strip()}
            kernels.append(cur)
        elif cur is not None and ":" in body:
            key, val = body.rsplit(":", 1)
            if key.strip() in _FIELDS:
                cur[_FIELDS[key.strip()]] = int(val.strip())
    return kernels


def write_resources(kernels, path=RESOURCES):
    with open(path, "w") as f:
        f.write("# kernel\tvgprs\tagprs\tscratch_bytes_per_lane\tvgpr_spill\tsgpr_spill\twaves_per_simd\tlds_bytes\n")
        for k in kernels:
            f.write("\t".join([k["name"]] + [str(k.get(x, -1)) for x in
                                             ("vgprs", "agprs", "scratch", "vgpr_spill", "sgpr_spill", "occupancy",
                                              "lds")]) + "\n")


def build(verbose=False):
    os.makedirs(BUILD, exist_ok=True)
    objs = []
    for src in HOST_SOURCES:
        obj = os.path.join(BUILD, src + ".o")
        _run([CXX, *HOST_FLAGS, "-I", INCLUDE, "-c", os.path.join(CSRC, src), "-o", obj], verbose)
        objs.append(obj)
    kernels = []
    for src in HIP_SOURCES:
        obj = os.path.join(BUILD, src + ".o")
        out = _run([HIPCC, *HIP_FLAGS, "-Rpass-analysis=kernel-resource-usage", "-I", INCLUDE, "-c",
                    os.path.join(CSRC, src), "-o", obj], verbose)
        kernels += parse_resources(out)
        objs.append(obj)
    write_resources(kernels)
    # every kernel keeps its state in registers and LDS: scratch memory in a
    # hot loop costs more than the occupancy it buys. Scalar registers
    # spilled into vector-register lanes (the shared-prefix plan kernels'
    # launch state) touch no memory and are allowed; a scratch size of zero
    # shows that every spill went there.
    bad = [k["name"] for k in kernels if k.get("scratch", 0) or k.get("vgpr_spill", 0)]
    if not kernels:
        raise RuntimeError("no kernel-resource-usage remarks from hipcc")
    if bad:
        raise RuntimeError(f"kernels using scratch memory or spilling registers: {bad} (see {RESOURCES})")
    tmp = LIB + ".tmp"
    _run([HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp], verbose)
    os.replace(tmp, LIB)
    return LIB


def clean():
    shutil.rmtree(BUILD, ignore_errors=True)


if __name__ == "__main__":
    print(build(verbose=True))
