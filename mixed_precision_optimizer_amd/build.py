"""Build libhpo.so in-tree with hipcc for gfx950.

    python -m mixed_precision_optimizer_amd.build

Device code: -O3, no floating-point contraction (each multiply and add of the
update rounds on its own), HIP's default correctly rounded fp32 division and
square root, fp32 denormals kept, and packed-fp32 instruction selection
switched off.  Host code is plain C++ against the HIP runtime API.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD_DIR = os.path.join(ROOT, "_build")
LIB_PATH = os.path.join(PKG, "libhpo.so")
ARCH = "gfx950"


# gfx950 kernel files and host files of libhpo
DEVICE_SOURCES = ("hpo_kernels.hip", "hpo_muon.hip", "hpo_static.hip")
HOST_SOURCES = ("hpo_api.cpp", "hpo_muon_api.cpp")


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build libhpo.so)")


DEVICE_FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    "-ffp-contract=off", "-fno-fast-math", "-fhip-fp32-correctly-rounded-divide-sqrt",
    "-fno-gpu-flush-denormals-to-zero",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-command-line-argument",
]
HOST_FLAGS = ["-x", "c++", "-O2", "-std=c++17", "-fPIC", "-Wall", "-Wextra", "-D__HIP_PLATFORM_AMD__"]


def rocm_include() -> str:
    return os.path.join(os.path.dirname(os.path.dirname(os.path.realpath(hipcc()))), "include")


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)


def build(verbose: bool = False) -> str:
    """Compile the kernels and the host API, link libhpo.so (always rebuilds)."""
    os.makedirs(BUILD_DIR, exist_ok=True)
    cc = hipcc()
    inc = ["-I", INCLUDE, "-I", CSRC]
    objs = []
    for src in DEVICE_SOURCES:
        obj = os.path.join(BUILD_DIR, os.path.splitext(src)[0] + ".o")
        _run([cc, *DEVICE_FLAGS, *inc, "-c", os.path.join(CSRC, src), "-o", obj], verbose)
        objs.append(obj)
    for src in HOST_SOURCES:
        obj = os.path.join(BUILD_DIR, os.path.splitext(src)[0] + ".o")
        _run([cc, *HOST_FLAGS, *inc, "-I", rocm_include(), "-c", os.path.join(CSRC, src), "-o", obj], verbose)
        objs.append(obj)
    tmp = LIB_PATH + ".tmp"
    _run([cc, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp], verbose)
    os.replace(tmp, LIB_PATH)
    return LIB_PATH


if __name__ == "__main__":
    print(build(verbose=True))
    sys.exit(0)
