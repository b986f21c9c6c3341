"""Build the CPU oracle (test infrastructure) into oracle/_build/liboracle.so.

Compiled with gcc, OpenMP, no fast-math and no floating-point contraction:
the quantiser's fp32 steps must be single correctly rounded operations.
"""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "gmm_oracle.c")
OUT_DIR = os.path.join(HERE, "_build")
LIB = os.path.join(OUT_DIR, "liboracle.so")


def build(verbose: bool = False) -> str:
    os.makedirs(OUT_DIR, exist_ok=True)
    tmp = LIB + ".tmp%d" % os.getpid()
    cmd = [
        "gcc", "-std=c99", "-O2", "-fopenmp", "-fPIC", "-shared",
        "-ffp-contract=off", "-fno-fast-math", "-frounding-math",
        "-Wall", "-Wno-unknown-pragmas",
        SRC, "-o", tmp, "-lm",
    ]
    if verbose:
        print(" ".join(cmd))
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
