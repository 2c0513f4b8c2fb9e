"""Build the CPU oracle (plain C, gcc + OpenMP) into oracle/libqref.so.

Test infrastructure: the library is the checker, not part of the product.
"""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "qref.c")
LIB = os.path.join(HERE, "libqref.so")


def build(verbose: bool = False, extra_flags=()) -> str:
    cmd = ["gcc", "-O2", "-std=c11", "-fopenmp", "-fPIC", "-shared", "-Wall", "-Wextra",
           *extra_flags, "-o", LIB, SRC, "-lm"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.check_call(cmd)
    return LIB


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
