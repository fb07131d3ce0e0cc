"""Builds the CPU oracle (test infrastructure) into oracle/liboracle.so.

Plain gcc, no fast-math, no fp contraction, OpenMP over independent output
rows only, so the arithmetic of every single element is the one written in
nq_oracle.c.
"""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "nq_oracle.c")
LIB = os.path.join(HERE, "liboracle.so")
FLAGS = ["-O2", "-ffp-contract=off", "-fno-fast-math", "-fopenmp", "-shared", "-fPIC",
         "-Wall", "-Wextra", "-std=c11"]


def build(verbose=False):
    tmp = LIB + ".tmp"
    cmd = ["gcc", *FLAGS, "-o", tmp, SRC, "-lm"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
