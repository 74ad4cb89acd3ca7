"""Builds the HIP/C++ library libdash_mi355x.so in this package directory (gfx950 only)."""
from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
LIB_NAME = "libdash_mi355x.so"
LIB_PATH = os.path.join(HERE, LIB_NAME)
# Profiling build (-DDASH_PROFILE): the main kernel also records per-wave phase cycle
# counters, exported through dash_profile_attach. Not used by the default path.
PROF_LIB_PATH = os.path.join(HERE, "libdash_mi355x_prof.so")
# Replay build (-DDASH_REPLAY): every ordered dQ partial is dumped (dash_replay_attach),
# for the exact check of the reduction order. Not used by the default path.
REPLAY_LIB_PATH = os.path.join(HERE, "libdash_mi355x_replay.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
BUILD_DIR = os.path.join(ROOT, "_build")

# Packed fp32 instructions are kept out of the generated code (the leading '-'
# disables the target feature).
COMMON = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I" + os.path.join(ROOT, "include"), "-I" + os.path.join(HERE, "csrc"),
]
# MFMA results of the 4-wave main kernel are allocated in VGPRs (-amdgpu-mfma-vgpr-form):
# the softmax reads them with VALU instructions, which cannot read AGPRs, so AGPR
# results would need a copy each. (The 2-wave kernel keeps the default: this LLVM
# crashes on it with the option.)
VGPR_FORM = ["-mllvm", "-amdgpu-mfma-vgpr-form"]
# (source, extra flags, object name)
MAIN_FLAGS = {(64, 4): VGPR_FORM, (128, 4): VGPR_FORM, (64, 2): [], (128, 2): []}
# The two-waves-per-SIMD kernel (d = 128): MFMA results in VGPRs for the same reason.
PAIR_FLAGS = VGPR_FORM
UNITS = [
    ("bwd_main.hip", [f"-DDASH_MAIN_D={d}", f"-DDASH_MAIN_NW={nw}"] + fl, f"bwd_main_d{d}_nw{nw}.o")
    for (d, nw), fl in MAIN_FLAGS.items()
] + [
    ("bwd_pair.hip", PAIR_FLAGS, "bwd_pair.o"),
    ("aux_kernels.hip", [], "aux_kernels.o"),
    ("fwd_main.hip", [], "fwd_main.o"),
    ("dq_pass.hip", [], "dq_pass.o"),
    ("dash_api.cpp", [], "dash_api.o"),
    ("schedule.cpp", [], "schedule.o"),
]


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        sys.stderr.write(res.stdout + res.stderr)
        raise RuntimeError(f"hipcc failed with exit code {res.returncode}: {' '.join(cmd)}")
    return res


def build(verbose: bool = False, resource_usage: bool = False, profile: bool = False, replay: bool = False) -> str:
    """Compile every source and link LIB_PATH (PROF_LIB_PATH with profile=True,
    REPLAY_LIB_PATH with replay=True; always recompiles); returns the library path."""
    assert not (profile and replay)
    out = PROF_LIB_PATH if profile else (REPLAY_LIB_PATH if replay else LIB_PATH)
    tag = "prof" if profile else ("replay" if replay else "rel")
    os.makedirs(BUILD_DIR, exist_ok=True)
    extra = (["-DDASH_PROFILE"] if profile else []) + (["-DDASH_REPLAY"] if replay else []) + \
        (["-Rpass-analysis=kernel-resource-usage"] if resource_usage else [])
    objs = []
    for src, flags, obj in UNITS:
        o = os.path.join(BUILD_DIR, tag + "_" + obj)
        res = _run([HIPCC] + COMMON + flags + extra + ["-c", "-x", "hip", os.path.join(HERE, "csrc", src), "-o", o],
                   verbose)
        if resource_usage:
            sys.stderr.write(res.stderr)
        objs.append(o)
    tmp = out + ".tmp"
    _run([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC"] + objs + ["-o", tmp], verbose)
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    build(verbose=True, resource_usage="--resource-usage" in sys.argv, profile="--profile" in sys.argv,
          replay="--replay" in sys.argv)
