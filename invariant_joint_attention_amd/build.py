"""Build the gfx950 library libqi.so in-tree with hipcc.

The arithmetic contract is fixed at build time: no fast math, no FP
contraction, FP32 denormals kept, correctly rounded FP32 division and square
root, and no packed-FP32 VALU instructions.  There is no runtime switch.
"""
from __future__ import annotations

import glob
import os
import subprocess

PKG = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(PKG, "csrc")
LIB = os.path.join(PKG, "libqi.so")
# the strict probe alone, built with -ffast-math: its verdict on a GPU must
# be the strict failure (the probe detects a relaxed build)
PROBE_SRC = os.path.join(CSRC, "probe", "qi_probe_lib.hip")
PROBE_FASTMATH_LIB = os.path.join(PKG, "libqi_probe_fastmath.so")

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-shared",
    "-ffp-contract=off",
    "-fno-fast-math",
    "-fhip-fp32-correctly-rounded-divide-sqrt",
    "-fno-gpu-flush-denormals-to-zero",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall",
    "-Wno-unused-result",
]


def sources() -> list:
    return sorted(glob.glob(os.path.join(CSRC, "*.hip")))


def _compile(srcs, out, flags, verbose):
    tmp = out + ".tmp"
    cmd = [HIPCC, *flags, *srcs, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, out)


def build(verbose: bool = False, extra_flags=()) -> str:
    """Compile every HIP source of the library into libqi.so, and the probe
    alone with -ffast-math into libqi_probe_fastmath.so (always)."""
    _compile(sources(), LIB, [*FLAGS, *extra_flags], verbose)
    # -ffast-math after the strict flags overrides them (fast math, FP
    # contraction, finite-math assumptions)
    _compile([PROBE_SRC], PROBE_FASTMATH_LIB, [*FLAGS, "-ffast-math"], verbose)
    return LIB


if __name__ == "__main__":
    build(verbose=True)
