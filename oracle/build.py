"""Builds the CPU oracle shared library (test infrastructure only).

    python oracle/build.py

Flags: -O2, no fast-math, -ffp-contract=off (no fused multiply-add, so every
binary32 operation is rounded on its own), SSE float evaluation, OpenMP.
"""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "dl_oracle.c")
LIB = os.path.join(HERE, "libdloracle.so")

CFLAGS = ["-O2", "-std=c11", "-fPIC", "-shared", "-ffp-contract=off", "-fno-fast-math",
          "-fno-unsafe-math-optimizations", "-mfpmath=sse", "-msse2", "-fopenmp",
          "-Wall", "-Wextra", "-Werror"]


def build(verbose: bool = False) -> str:
    cmd = ["gcc", *CFLAGS, "-o", LIB + ".tmp", SRC]
    if verbose:
        print(" ".join(cmd))
    subprocess.run(cmd, check=True)
    os.replace(LIB + ".tmp", LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
