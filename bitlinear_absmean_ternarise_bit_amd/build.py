"""Build libbitlinear.so in-tree with hipcc for gfx950.

    python -m bitlinear_absmean_ternarise_bit_amd.build
"""
from __future__ import annotations

import glob
import os
import subprocess
import sys

PKG_DIR = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG_DIR)
LIB_NAME = "libbitlinear.so"
LIB_PATH = os.path.join(PKG_DIR, LIB_NAME)
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

HIP_FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-shared",
    # the quantisers must round exactly like the float32 definition: no
    # contraction into FMA, no fast-math reciprocal division
    "-ffp-contract=off",
    "-fno-fast-math",
    # keep the compiler from emitting packed-FP32 VALU instructions
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]


def sources():
    return sorted(glob.glob(os.path.join(PKG_DIR, "csrc", "*.hip")))


def build_library(verbose: bool = False) -> str:
    """Compile every HIP source into one shared library next to this file."""
    tmp = LIB_PATH + ".tmp"
    cmd = [HIPCC, *HIP_FLAGS, "-I", os.path.join(ROOT, "include"), "-o", tmp, *sources()]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        sys.stderr.write(res.stdout + res.stderr)
        raise RuntimeError(f"hipcc failed with status {res.returncode}")
    os.replace(tmp, LIB_PATH)
    return LIB_PATH


if __name__ == "__main__":
    print(build_library(verbose=True))
