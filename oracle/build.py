"""Builds liboracle.so from oracle.c (GEMM) and attention.c with gcc (test
infrastructure only).

-O2 without -ffast-math keeps every fp64 sum in k order; -ffp-contract=off
keeps products and sums separately rounded.
"""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "oracle.c")
SOURCES = [SRC, os.path.join(HERE, "attention.c")]
LIB_PATH = os.path.join(HERE, "liboracle.so")

CFLAGS = ["-O2", "-std=c11", "-fPIC", "-shared", "-fopenmp",
          "-ffp-contract=off", "-fno-fast-math", "-Wall", "-Wextra"]


def build_oracle(verbose=False):
    tmp = LIB_PATH + ".tmp"
    cmd = ["gcc", *CFLAGS, *SOURCES, "-o", tmp, "-lm"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB_PATH)
    return LIB_PATH


if __name__ == "__main__":
    print(build_oracle(verbose=True))
