"""Build the seeded input generator: a host library (gcc, OpenMP) and a
device library (hipcc, gfx950).  Both compile synth_core.h with
floating-point contraction off so that their values are bit-identical."""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
HOST_LIB = os.path.join(HERE, "libsynth.so")
DEV_LIB = os.path.join(HERE, "libsynth_dev.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")


def build(verbose=False):
    cmds = [
        ["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-fopenmp", "-ffp-contract=off",
         "-fno-fast-math", "-Wall", "-o", HOST_LIB, os.path.join(HERE, "synth.c"), "-lm"],
        [HIPCC, "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
         "-ffp-contract=off", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-o", DEV_LIB, os.path.join(HERE, "synth_dev.hip")],
    ]
    for cmd in cmds:
        if verbose:
            print(" ".join(cmd))
        subprocess.run(cmd, check=True, stderr=None if verbose else subprocess.DEVNULL)
    return HOST_LIB, DEV_LIB


if __name__ == "__main__":
    build(verbose=True)
