"""Compile libbs.so (HIP kernels + C ABI + host tables) for gfx950, in-tree."""
from __future__ import annotations

import os
import subprocess

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libbs.so")

SOURCES = [os.path.join(CSRC, "bs_kernels.hip"), os.path.join(CSRC, "bs_host.cpp"),
           os.path.join(CSRC, "bs_bench.cpp")]

HIPCC_FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
    "-ffp-contract=off",
    # the leading kernel arguments arrive in SGPRs at wave launch
    "-mllvm", "-amdgpu-kernarg-preload-count=16",
    # no packed fp32 instructions anywhere in the device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-command-line-argument",
    "-I", INCLUDE,
]


def hipcc() -> str:
    return os.path.join(os.environ.get("ROCM_PATH", "/opt/rocm"), "bin", "hipcc")


def build(extra_flags=(), out: str = LIB, verbose: bool = False) -> str:
    """Compile every source into one shared library; returns its path."""
    tmp = out + ".tmp"
    cmd = [hipcc(), *HIPCC_FLAGS, *extra_flags, "-o", tmp, *SOURCES]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True, capture_output=not verbose)
    os.replace(tmp, out)
    return out


def resource_report(out: str) -> str:
    """The compiler's per-kernel register, spill, LDS and occupancy report for
    the device code, built with the library's own flags, written to `out`."""
    cmd = [hipcc(), *[f for f in HIPCC_FLAGS if f not in ("-shared", "-fPIC")],
           "-Rpass-analysis=kernel-resource-usage", "-c", SOURCES[0], "-o", os.devnull]
    r = subprocess.run(cmd, check=True, capture_output=True, text=True)
    with open(out, "w") as f:
        f.write(r.stderr)
    return out


if __name__ == "__main__":
    import sys
    if len(sys.argv) == 3 and sys.argv[1] == "--resource-report":
        print(resource_report(sys.argv[2]))
    else:
        print(build(verbose=True))
