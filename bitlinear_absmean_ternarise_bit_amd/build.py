"""Build the HIP libraries in-tree with hipcc for gfx950.

    python -m bitlinear_absmean_ternarise_bit_amd.build

libbitlinear.so        the BitLinear library (csrc/*.hip, the ABI of include/bitlinear.h)
libbitlinear_probe.so  the benchmark's attainable-peak probes (probe/probe.hip,
                       include/bitlinear_probe.h); not part of the BitLinear ABI

Each source is compiled to its own object in _build/ (in parallel), then the
objects are linked.
"""
from __future__ import annotations

import concurrent.futures as cf
import glob
import os
import subprocess
import sys

PKG_DIR = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG_DIR)
LIB_NAME = "libbitlinear.so"
LIB_PATH = os.path.join(PKG_DIR, LIB_NAME)
PROBE_LIB_PATH = os.path.join(PKG_DIR, "libbitlinear_probe.so")
BUILD_DIR = os.path.join(ROOT, "_build")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

HIP_FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-fPIC",
    # the quantisers must round exactly like the float32 definition: no
    # contraction into FMA, no fast-math reciprocal division
    "-ffp-contract=off",
    "-fno-fast-math",
    # keep the compiler from emitting packed-FP32 VALU instructions
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]


def sources():
    return sorted(glob.glob(os.path.join(PKG_DIR, "csrc", "*.hip")))


def probe_sources():
    return [os.path.join(PKG_DIR, "probe", "probe.hip")]


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        sys.stderr.write(res.stdout + res.stderr)
        raise RuntimeError(f"hipcc failed with status {res.returncode}: {' '.join(cmd[-3:])}")


def _link(objs, out, verbose):
    tmp = out + ".tmp"
    _run([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp, *objs], verbose)
    os.replace(tmp, out)
    return out


def build_library(verbose: bool = False, jobs: int = 0) -> str:
    """Compile every HIP source and link both libraries next to this file."""
    os.makedirs(BUILD_DIR, exist_ok=True)
    inc = ["-I", os.path.join(ROOT, "include")]
    units = [(src, os.path.join(BUILD_DIR, os.path.basename(src)[:-4] + ".o"))
             for src in sources() + probe_sources()]
    jobs = jobs or min(len(units), max(1, min(16, os.cpu_count() or 1)))
    with cf.ThreadPoolExecutor(max_workers=jobs) as ex:
        futs = [ex.submit(_run, [HIPCC, *HIP_FLAGS, *inc, "-c", src, "-o", obj], verbose)
                for src, obj in units]
        for f in futs:
            f.result()
    objs = {src: obj for src, obj in units}
    _link([objs[s] for s in sources()], LIB_PATH, verbose)
    _link([objs[s] for s in probe_sources()], PROBE_LIB_PATH, verbose)
    return LIB_PATH


if __name__ == "__main__":
    print(build_library(verbose=True))
