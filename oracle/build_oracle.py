"""Build the CPU oracle (test infrastructure only) into oracle/libfp4idx_oracle.so.

Plain gcc, -O2 without fast-math (IEEE double arithmetic, round-to-nearest), OpenMP
over independent output rows.
"""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "fp4idx_oracle.c")
LIB = os.path.join(HERE, "libfp4idx_oracle.so")


def build(verbose: bool = False) -> str:
    cmd = ["gcc", "-O2", "-std=c11", "-fno-fast-math", "-ffp-contract=off", "-fopenmp",
           "-fPIC", "-shared", "-Wall", "-Wextra", "-o", LIB + ".tmp", SRC, "-lm"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(LIB + ".tmp", LIB)
    return LIB


if __name__ == "__main__":
    build(verbose="-v" in sys.argv)
