"""Build the gfx950 shared library ``libra.so`` in-tree with hipcc.

Usage: ``python -m ring_blockwise_softmax_amd.build`` (also called by
``__graft_entry__.build()``).  Always recompiles.
"""

from __future__ import annotations

import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(HERE, "libra.so")

SOURCES = ["ra_kernels.hip", "ra_api.cpp", "ra_plan.cpp"]

COMMON = [
    "-O3", "-std=c++17", "-fPIC", "-Wall", "-Wno-unused-function",
    f"-I{INCLUDE}", f"-I{CSRC}",
]
# Device code: gfx950 only; packed fp32 VALU forms are disabled.
# -fno-honor-nans: no kernel tests for NaN; without it every fmax pays a
# NaN-quieting canonicalisation.
# The iterative ILP scheduler orders the attention stage better than the
# default occupancy-driven one at the kernel's three-waves-per-SIMD budget.
DEVICE = ["--offload-arch=gfx950", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
          "-fno-honor-nans", "-mllvm", "-amdgpu-sched-strategy=iterative-ilp"]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found: the HIP library cannot be built")


def build(verbose: bool = False) -> str:
    cc = hipcc()
    objdir = os.path.join(HERE, "_build")
    os.makedirs(objdir, exist_ok=True)
    objs = []
    for src in SOURCES:
        path = os.path.join(CSRC, src)
        obj = os.path.join(objdir, src + ".o")
        if src.endswith(".hip"):
            cmd = [cc, *COMMON, *DEVICE, "-c", path, "-o", obj]
        else:
            # Host-only translation units (no device code).
            cmd = [cc, *COMMON, "-D__HIP_PLATFORM_AMD__", "-I/opt/rocm/include", "-x", "c++", "-c", path, "-o", obj]
        if verbose:
            print(" ".join(cmd), flush=True)
        subprocess.run(cmd, check=True)
        objs.append(obj)
    tmp = LIB + ".tmp"
    cmd = [cc, "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB)
    build_probe(cc, verbose)
    return LIB


PROBE_LIB = os.path.join(HERE, "libra_probe.so")


def build_probe(cc: str, verbose: bool = False) -> str:
    """The benchmark's MFMA-throughput probe, a library of its own.  Built
    with the default scheduler: the ILP one places two products on the same
    accumulator back to back in its loop, which stalls the matrix pipe."""
    tmp = PROBE_LIB + ".tmp"
    flags = [f for f in DEVICE if f not in ("-mllvm", "-amdgpu-sched-strategy=iterative-ilp")]
    cmd = [cc, *COMMON, *flags, "-shared", os.path.join(CSRC, "mfma_ceiling.hip"), "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, PROBE_LIB)
    return PROBE_LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
