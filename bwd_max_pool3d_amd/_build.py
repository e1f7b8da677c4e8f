"""Build libmp3d.so (the HIP kernels and the C ABI) in-tree for gfx950.

Each source is compiled to an object of its own (in parallel), then the
objects are linked into the shared library.
"""
from __future__ import annotations

import os
import subprocess
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIBRARY = os.path.join(HERE, "libmp3d.so")
OBJDIR = os.path.join(HERE, "_build")
SOURCES = ["api.hip", "plan.hip", "forward.hip", "forward_fixed.hip", "forward_col.hip",
           "backward.hip", "backward_owner.hip", "small.hip", "forward_ex.hip"]

HIPCC_FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
    "-Wall", "-Wno-unused-result",
    # keep IEEE subnormals and exact rounding: no fast-math, no FTZ
    "-fno-fast-math", "-ffp-contract=off",
    # no packed-FP32 instructions in the generated code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]


def sources() -> list[str]:
    return [os.path.join(CSRC, s) for s in SOURCES]


def _jobs() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    return max(1, min(8, n, int(os.environ.get("MAX_JOBS", "8"))))


def build(out: str = LIBRARY, verbose: bool = False) -> str:
    hipcc = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
    os.makedirs(OBJDIR, exist_ok=True)
    pid = os.getpid()

    def compile_one(src: str) -> str:
        obj = os.path.join(OBJDIR, os.path.basename(src) + ".%d.o" % pid)
        cmd = [hipcc, *HIPCC_FLAGS, "-c", "-o", obj, src]
        if verbose:
            print(" ".join(cmd), flush=True)
        subprocess.run(cmd, check=True)
        return obj

    with ThreadPoolExecutor(_jobs()) as pool:
        objs = list(pool.map(compile_one, sources()))
    tmp = out + ".tmp%d" % pid
    cmd = [hipcc, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp, *objs]
    if verbose:
        print(" ".join(cmd), flush=True)
    try:
        subprocess.run(cmd, check=True)
    finally:
        for o in objs:
            if os.path.exists(o):
                os.remove(o)
    os.replace(tmp, out)
    return out


def build_executable(src: str, out: str, verbose: bool = False) -> str:
    """Compile a stand-alone HIP program (the HBM ceiling benchmark) with the
    library's flags."""
    hipcc = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
    os.makedirs(os.path.dirname(out), exist_ok=True)
    tmp = out + ".tmp%d" % os.getpid()
    cmd = [hipcc, *[f for f in HIPCC_FLAGS if f != "-fPIC"], "-o", tmp, src]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build(verbose=True))
