"""Builds the CPU oracle (plain C, OpenMP) into oracle/liboracle.so.

Test infrastructure: only the tests, the package smoke check and the
benchmark's CPU-baseline leg load the result.
"""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "moe_oracle.c")
LIB = os.path.join(HERE, "liboracle.so")


def build(verbose: bool = False) -> str:
    cmd = ["gcc", "-std=c99", "-O2", "-fno-fast-math", "-ffp-contract=off", "-fopenmp", "-fPIC",
           "-shared", "-Wall", "-Wextra", "-Wno-unused-parameter", SRC, "-o", LIB + ".tmp", "-lm"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(LIB + ".tmp", LIB)
    return LIB


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
