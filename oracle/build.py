"""Builds the fp64 CPU oracle (test infrastructure) with gcc.

The oracle is plain C; it is compiled without fast-math so that every fp64
operation rounds as written.  Output: oracle/libhelm_oracle.so.
"""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "helm_oracle.c")
LIB = os.path.join(HERE, "libhelm_oracle.so")


def build(verbose: bool = False) -> str:
    tmp = LIB + ".tmp"
    cmd = ["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-fopenmp",
           "-fno-fast-math", "-ffp-contract=off", "-Wall", "-Wextra",
           SRC, "-o", tmp, "-lm"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
