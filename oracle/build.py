"""Compile the CPU oracle (plain C, gcc) into oracle/libltc_oracle.so.

TEST INFRASTRUCTURE: the oracle is the checker, not the product.
"""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
LIB = os.path.join(HERE, "libltc_oracle.so")


def build(verbose: bool = False) -> str:
    src = os.path.join(HERE, "ltc_oracle.c")
    tmp = LIB + ".tmp"
    cmd = ["gcc", "-O2", "-std=c99", "-Wall", "-Wextra", "-fPIC", "-shared",
           "-fopenmp", src, "-o", tmp, "-lm"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
