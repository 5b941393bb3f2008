"""Compile the CPU oracle into oracle/liboracle.so with the host C compiler.

Test infrastructure: the oracle is a checker, never part of the product path.
"""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "oracle_chain.c")
LIB = os.path.join(HERE, "liboracle.so")


def build(verbose: bool = False, src: str = SRC, lib: str = LIB) -> str:
    cmd = ["gcc", "-O2", "-std=c11", "-D_GNU_SOURCE", "-fopenmp", "-fPIC", "-shared",
           "-Wall", "-Wextra", "-o", lib + ".tmp", src, "-lm"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(lib + ".tmp", lib)
    return lib


if __name__ == "__main__":
    print(build(verbose=True))
    sys.exit(0)
