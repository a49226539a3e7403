"""Build the CPU oracle (test infrastructure) with gcc.

Compiles oracle_zero.c into liboracle_zero.so beside this file:
plain -O2, -ffp-contract=off so no multiply-add is fused, no fast-math,
no -march (SSE2 binary32 arithmetic with round-to-nearest-even).
"""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
LIB = os.path.join(HERE, "liboracle_zero.so")


def build(verbose: bool = False) -> str:
    src = os.path.join(HERE, "oracle_zero.c")
    cmd = ["gcc", "-O2", "-std=c11", "-ffp-contract=off", "-fno-fast-math",
           "-Wall", "-Wextra", "-fPIC", "-shared", "-o", LIB + ".tmp", src, "-lm"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(LIB + ".tmp", LIB)
    return LIB


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
