"""Build the CPU oracle (test infrastructure) as a shared library.

Plain C11, single-threaded, -O2 with floating-point contraction off and no
fast-math, so that every fp32 operation is rounded on its own.
"""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
LIB = os.path.join(HERE, "liboracle.so")


def build(verbose=False):
    cmd = ["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-ffp-contract=off", "-fno-fast-math",
           "-Wall", "-Wextra", "-o", LIB, os.path.join(HERE, "oracle.c"), "-lm"]
    if verbose:
        print(" ".join(cmd))
    subprocess.run(cmd, check=True)
    return LIB


if __name__ == "__main__":
    build(verbose=True)
