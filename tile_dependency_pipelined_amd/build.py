"""Build the HIP library libcpchain.so in-tree for gfx950 (MI355X).

    python -m tile_dependency_pipelined_amd.build

Packed-fp32 instruction selection is disabled for all device code.
"""
import os
import subprocess
import sys
import time

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libcpchain.so")
SOURCES = [os.path.join(CSRC, "cp_kernels.hip"), os.path.join(CSRC, "cp_chain.cpp")]
ARCH = os.environ.get("CP_OFFLOAD_ARCH", "gfx950")


def hipcc() -> str:
    for cand in ("/opt/rocm/bin/hipcc", "hipcc"):
        if os.path.sep not in cand or os.path.exists(cand):
            return cand
    return "hipcc"


def build(verbose: bool = True, extra=None) -> str:
    cmd = [hipcc(), "-O3", "-std=c++17", f"--offload-arch={ARCH}", "-fPIC", "-shared",
           "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
           "-Wall", "-Wno-unused-result",
           "-I", INCLUDE, "-I", CSRC, "-o", LIB + ".tmp"] + SOURCES + list(extra or [])
    t0 = time.time()
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(LIB + ".tmp", LIB)
    if verbose:
        print(f"built {LIB} in {time.time() - t0:.1f}s", flush=True)
    return LIB


if __name__ == "__main__":
    build()
    sys.exit(0)
