"""Build the CPU oracle (plain C, gcc).  Test infrastructure only.

The oracle is compiled without -ffast-math and with FMA contraction off, so
that its binary32 divisions are IEEE round-to-nearest-even and its FP64
accumulations are the plain sums the source spells out.
"""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "puro_ref.c")
LIB = os.path.join(HERE, "libpuro_ref.so")


def build(verbose: bool = False) -> str:
    cmd = ["gcc", "-O2", "-std=c11", "-fopenmp", "-ffp-contract=off", "-fno-fast-math",
           "-fPIC", "-shared", "-Wall", "-Wextra", "-o", LIB + ".tmp", SRC, "-lm"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(LIB + ".tmp", LIB)
    return LIB


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
