"""Builds the HIP/C++ library libdash_mi355x.so in this package directory (gfx950 only)."""
from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
LIB_NAME = "libdash_mi355x.so"
LIB_PATH = os.path.join(HERE, LIB_NAME)
SOURCES = [
    os.path.join(HERE, "csrc", "bwd_kernels.hip"),
    os.path.join(HERE, "csrc", "dash_api.cpp"),
    os.path.join(HERE, "csrc", "schedule.cpp"),
]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

# Packed fp32 instructions are kept out of the generated code (the leading '-'
# disables the target feature).
FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I" + os.path.join(ROOT, "include"), "-I" + os.path.join(HERE, "csrc"),
]


def build(verbose: bool = False, resource_usage: bool = False) -> str:
    """Compile every source into LIB_PATH (always recompiles); returns the library path."""
    tmp = LIB_PATH + ".tmp"
    cmd = [HIPCC] + FLAGS + (["-Rpass-analysis=kernel-resource-usage"] if resource_usage else [])
    cmd += ["-x", "hip"] + SOURCES + ["-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        sys.stderr.write(res.stdout + res.stderr)
        raise RuntimeError(f"hipcc failed with exit code {res.returncode}")
    if verbose or resource_usage:
        sys.stderr.write(res.stderr)
    os.replace(tmp, LIB_PATH)
    return LIB_PATH


if __name__ == "__main__":
    build(verbose=True, resource_usage="--resource-usage" in sys.argv)
