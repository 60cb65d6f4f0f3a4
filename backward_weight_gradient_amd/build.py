"""Builds libforge.so (the gfx950 kernels and the C ABI) in-tree with hipcc."""

import concurrent.futures
import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libforge.so")
# forge_device.h holds the kernels (all templates); each forge_k_*.hip
# instantiates one optimizer family's, so the families compile in parallel.
SOURCES = sorted(f for f in os.listdir(CSRC) if f.endswith(".hip")) + ["forge_dispatch.cpp", "forge_api.cpp"]

# -ffp-contract=off: the step's fp32 op sequence is exactly the written one
# (explicit fmaf only).  Packed-fp32 instructions are disabled.
HIP_FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
    "-ffp-contract=off",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function",
]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build libforge)")


def build(verbose: bool = False, jobs: int = 0) -> str:
    """Compile every source for gfx950 (in parallel) and link libforge.so next to this file."""
    build_dir = os.path.join(HERE, "_build")
    os.makedirs(build_dir, exist_ok=True)
    cc = hipcc()

    def compile_one(src):
        obj = os.path.join(build_dir, os.path.splitext(src)[0] + ".o")
        cmd = [cc, *HIP_FLAGS, "-c", os.path.join(CSRC, src), "-o", obj]
        if verbose:
            print(" ".join(cmd), flush=True)
        subprocess.run(cmd, check=True)
        return obj

    jobs = jobs or max(1, min(len(SOURCES), os.cpu_count() or 1, 16))
    with concurrent.futures.ThreadPoolExecutor(jobs) as pool:
        objs = list(pool.map(compile_one, SOURCES))
    tmp = LIB + ".tmp"
    cmd = [cc, "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
