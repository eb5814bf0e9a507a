"""Builds libmoe.so (all HIP kernels + the C ABI) for gfx950 with hipcc, in-tree."""
from __future__ import annotations

import glob
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
# MOE_SANITIZE=1: host code (argument checks, workspace layout, dispatch) built with
# AddressSanitizer and UndefinedBehaviorSanitizer into a library of its own; device code unchanged
SANITIZE = os.environ.get("MOE_SANITIZE") == "1"
LIB = os.path.join(PKG, "libmoe_san.so" if SANITIZE else "libmoe.so")
HOST_SAN_FLAGS = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
                  "-Xarch_host", "-fno-sanitize-recover=undefined", "-Xarch_host", "-fno-omit-frame-pointer"]

HIPCC_FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
    # keep the compiler from forming packed fp32 instructions
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function",
]


def sources():
    return sorted(glob.glob(os.path.join(CSRC, "*.hip")))


PROBE_SRC = os.path.join(ROOT, "tests", "probes", "mfma_sum_probe.hip")
PROBE_LIB = os.path.join(ROOT, "tests", "probes", "libmfma_probe.so")


def build_probe(verbose: bool = False) -> str:
    """The test-only matrix-core numerics probe (tests/probes), built beside its source."""
    hipcc = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
    tmp = PROBE_LIB + ".tmp"
    cmd = [hipcc, *HIPCC_FLAGS, "-o", tmp, PROBE_SRC]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        sys.stderr.write(res.stdout + res.stderr)
        raise RuntimeError("hipcc failed building the matrix-core probe")
    os.replace(tmp, PROBE_LIB)
    return PROBE_LIB


def build(verbose: bool = False) -> str:
    hipcc = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
    tmp = LIB + ".tmp"
    cmd = [hipcc, *HIPCC_FLAGS, *(HOST_SAN_FLAGS if SANITIZE else []), "-I", os.path.join(ROOT, "include"),
           "-o", tmp, *sources()]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        sys.stderr.write(res.stdout + res.stderr)
        raise RuntimeError("hipcc failed building libmoe.so")
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
