"""Build the HIP library libcpchain.so in-tree for gfx950 (MI355X).

    python -m tile_dependency_pipelined_amd.build

Device code is compiled by hipcc with packed-fp32 instruction selection
disabled.  The library is linked against the same HIP runtime that PyTorch
loads (torch/lib/libamdhip64.so), so that the streams and device memory
handed over by PyTorch belong to the runtime that launches the kernels; two
HIP runtimes in one process do not share devices or streams.  Without an
importable torch it links ROCm's runtime instead.
"""
import importlib.util
import os
import subprocess
import sys
import time

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libcpchain.so")
BUILD_DIR = os.path.join(ROOT, "_build")
SOURCES = [os.path.join(CSRC, "cp_kernels.hip"), os.path.join(CSRC, "cp_chain.cpp")]
ARCH = os.environ.get("CP_OFFLOAD_ARCH", "gfx950")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")


def hipcc() -> str:
    p = os.path.join(ROCM, "bin", "hipcc")
    return p if os.path.exists(p) else "hipcc"


def torch_lib_dir():
    spec = importlib.util.find_spec("torch")
    if spec is None or not spec.submodule_search_locations:
        return None
    d = os.path.join(list(spec.submodule_search_locations)[0], "lib")
    return d if os.path.exists(os.path.join(d, "libamdhip64.so")) else None


def build(verbose: bool = True, extra=None) -> str:
    t0 = time.time()
    os.makedirs(BUILD_DIR, exist_ok=True)
    objs = []
    for src in SOURCES:
        obj = os.path.join(BUILD_DIR, os.path.basename(src) + ".o")
        cmd = [hipcc(), "-x", "hip", "-O3", "-std=c++17", f"--offload-arch={ARCH}",
               "-mcode-object-version=5", "-fPIC", "-c",
               "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
               "-Wall", "-Wno-unused-result", "-I", INCLUDE, "-I", CSRC,
               "-o", obj, src] + list(extra or [])
        if verbose:
            print(" ".join(cmd), flush=True)
        subprocess.run(cmd, check=True)
        objs.append(obj)
    tdir = torch_lib_dir()
    if tdir:
        runtime = ["-L" + tdir, "-l:libamdhip64.so", "-Wl,-rpath," + tdir]
    else:
        rl = os.path.join(ROCM, "lib")
        runtime = ["-L" + rl, "-lamdhip64", "-Wl,-rpath," + rl]
    cmd = ["g++", "-shared", "-fPIC", "-o", LIB + ".tmp"] + objs + runtime + ["-Wl,--no-undefined"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(LIB + ".tmp", LIB)
    if verbose:
        print(f"built {LIB} in {time.time() - t0:.1f}s (HIP runtime: {tdir or ROCM})", flush=True)
    return LIB


if __name__ == "__main__":
    build()
    sys.exit(0)
