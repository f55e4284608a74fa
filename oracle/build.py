"""Build the CPU oracle library (test infrastructure only).

    python -m oracle.build

Compiles ``kpool_oracle.c`` with gcc, OpenMP, and -ffp-contract=off (no fused
multiply-add anywhere in the oracle).
"""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
LIB = os.path.join(HERE, "libkpool_oracle.so")


def build(verbose: bool = False) -> str:
    src = os.path.join(HERE, "kpool_oracle.c")
    tmp = f"{LIB}.tmp{os.getpid()}"     # per process: parallel test workers may build at once
    cmd = ["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-fopenmp", "-ffp-contract=off",
           "-fno-fast-math", "-Wall", "-Wextra", "-o", tmp, src, "-lm"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.check_call(cmd)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
