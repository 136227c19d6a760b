"""Build the package's libraries in-tree: HIP for gfx950 with hipcc, and the
host library with g++.

``libzero_shard.so``     the C ABI of include/zero_shard.h (the optimizer step)
``libzero_testkit.so``   seeded synthetic inputs and plain streaming
                         reference kernels (csrc/zero_testkit.h), used by
                         tests and benchmarks
``libzero_probes.so``    device probes of the optimizer library's own code
                         (csrc/zero_probes.h), used by tests and benchmarks
``libzero_host_adam.so`` the multi-core SIMD host step (include/zero_host_adam.h)

Flags: no FMA contraction, no fast-math (IEEE division and square root stay
correctly rounded), and packed-fp32 instructions disabled on the GPU.
"""
from __future__ import annotations

import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
INCLUDE = os.path.join(ROOT, "include")
CSRC = os.path.join(PKG, "csrc")

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"

HIP_FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-shared",
    "-ffp-contract=off", "-fno-fast-math",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wextra", "-Wno-unused-command-line-argument",
    "-I", INCLUDE, "-I", CSRC,
]

LIBS = {
    "libzero_shard.so": ["zero_shard.hip"],
    "libzero_testkit.so": ["testkit.hip"],
    "libzero_probes.so": ["probes.hip"],
}

CXX = os.environ.get("CXX_HOST", "g++")
HOST_FLAGS = [
    "-O3", "-std=c++17", "-fPIC", "-shared", "-fopenmp",
    "-ffp-contract=off", "-fno-fast-math", "-fno-math-errno",
    "-Wall", "-Wextra", "-I", INCLUDE,
]
HOST_LIBS = {
    "libzero_host_adam.so": ["host_adam.cpp"],
}


def library_path(name: str) -> str:
    return os.path.join(PKG, name)


def build_library(name: str, extra_flags=(), out_path: str | None = None, verbose=False) -> str:
    host = name in HOST_LIBS
    srcs = [os.path.join(CSRC, s) for s in (HOST_LIBS if host else LIBS)[name]]
    out = out_path or library_path(name)
    tmp = out + ".tmp"
    cmd = [CXX, *HOST_FLAGS] if host else [HIPCC, *HIP_FLAGS]
    cmd += [*extra_flags, "-o", tmp, *srcs]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        sys.stderr.write(r.stdout + r.stderr)
        raise RuntimeError(f"{cmd[0]} failed building {name}")
    os.replace(tmp, out)
    return out


def build_all(verbose=False) -> list[str]:
    return [build_library(name, verbose=verbose) for name in (*LIBS, *HOST_LIBS)]


if __name__ == "__main__":
    for p in build_all(verbose=True):
        print("built", p)
