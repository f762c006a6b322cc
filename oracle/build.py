"""Compile the C oracle into ``oracle/liboracle.so`` (test infrastructure).

Plain gcc, fp64, OpenMP; no fast-math and no FMA contraction, so the result is
the written definition evaluated in source order.
"""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "kda_oracle.c")
LIB = os.path.join(HERE, "liboracle.so")


def build(verbose: bool = False) -> str:
    cmd = [
        "gcc", "-O2", "-std=c99", "-fPIC", "-shared", "-fopenmp",
        "-ffp-contract=off", "-fno-fast-math", "-Wall", "-Wextra",
        SRC, "-o", LIB + ".tmp", "-lm",
    ]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(LIB + ".tmp", LIB)
    return LIB


def ensure_built() -> str:
    if not os.path.exists(LIB) or os.path.getmtime(LIB) < os.path.getmtime(SRC):
        build()
    return LIB


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
