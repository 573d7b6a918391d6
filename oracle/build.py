"""Builds the CPU oracle library (oracle/libfp8q_oracle.so) with gcc.

Test infrastructure: the oracle is built alongside the product so that the checker
exists wherever the tests run; nothing in the product path loads it.
"""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "fp8q_oracle.c")
LIB = os.path.join(HERE, "libfp8q_oracle.so")

# IEEE semantics: no fast-math, no implicit fused multiply-add.
CFLAGS = ["-O2", "-std=c11", "-ffp-contract=off", "-fno-fast-math", "-fopenmp", "-fPIC", "-shared",
          "-Wall", "-Wextra"]


def build(verbose: bool = False) -> str:
    tmp = LIB + ".tmp"
    cmd = ["gcc", *CFLAGS, SRC, "-o", tmp, "-lm"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    build(verbose="-v" in sys.argv)
