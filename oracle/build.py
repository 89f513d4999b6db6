"""Compile the fp64 oracle into oracle/liboracle.so (plain C, gcc, no fast-math).

Test infrastructure only: building the checker is not using it.
"""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "oracle.c")
OUT = os.path.join(HERE, "liboracle.so")


def build(verbose: bool = False) -> str:
    cmd = ["gcc", "-O2", "-std=c11", "-D_GNU_SOURCE", "-fno-fast-math", "-ffp-contract=off",
           "-fPIC", "-shared", "-Wall", "-Wextra", "-o", OUT + ".tmp", SRC, "-lm"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(OUT + ".tmp", OUT)
    return OUT


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
