"""Build the CPU oracle's shared library (test infrastructure only).

    python oracle/build.py

Compiles oracle/dsa_oracle.c with gcc into oracle/liboracle.so.  Plain -O2
(no intrinsics, no fast-math, so the fp64 arithmetic stays IEEE) with OpenMP.
"""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "dsa_oracle.c")
OUT = os.path.join(HERE, "liboracle.so")


def build(verbose: bool = False) -> str:
    cmd = ["gcc", "-O2", "-fno-fast-math", "-fopenmp", "-shared", "-fPIC", "-std=c11", "-Wall", "-Wextra",
           "-o", OUT + ".tmp", SRC, "-lm"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(OUT + ".tmp", OUT)
    return OUT


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
