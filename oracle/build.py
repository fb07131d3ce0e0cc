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


# AddressSanitizer / UndefinedBehaviorSanitizer variant (gcc), for running
# the oracle's pins against:  LD_PRELOAD=$(gcc -print-file-name=libasan.so)
# ASAN_OPTIONS=detect_leaks=0 NQ_ORACLE_LIB=oracle/liboracle_san.so pytest ...
SAN_LIB = os.path.join(HERE, "liboracle_san.so")
SAN_FLAGS = ["-O1", "-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
             "-fno-sanitize-recover=undefined"]


def build(verbose=False, sanitize=False):
    lib = SAN_LIB if sanitize else LIB
    tmp = lib + ".tmp"
    flags = [f for f in FLAGS if not (sanitize and f == "-O2")] + (SAN_FLAGS if sanitize else [])
    cmd = ["gcc", *flags, "-o", tmp, SRC, "-lm"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, lib)
    return lib


if __name__ == "__main__":
    import sys
    print(build(verbose=True, sanitize="--sanitize" in sys.argv))
