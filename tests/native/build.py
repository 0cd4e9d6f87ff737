"""Build the plain-C check of the C ABI (tests/native/abi_c_check.c): gcc,
the HIP runtime's C API, libonebit.so, and the oracle and host input
generator it compares against.  Run after those libraries are built; the
runpath is relative to the binary, so the tree can move."""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
EXE = os.path.join(HERE, "abi_c_check")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")


def build(verbose=False):
    pkg, orc, syn = (os.path.join(ROOT, d) for d in
                     ("communication_compressed_optimizer_amd", "oracle", "synth"))
    rpath = ":".join(["$ORIGIN/../../communication_compressed_optimizer_amd", "$ORIGIN/../../oracle",
                      "$ORIGIN/../../synth", os.path.join(ROCM, "lib")])
    cmd = ["gcc", "-std=c11", "-O2", "-Wall", "-Wextra", "-D__HIP_PLATFORM_AMD__",
           "-I", os.path.join(ROCM, "include"), "-I", os.path.join(ROOT, "include"), "-I", orc,
           os.path.join(HERE, "abi_c_check.c"), "-o", EXE, "-L", pkg, "-lonebit", "-L", orc,
           "-loracle", "-L", syn, "-lsynth", "-L", os.path.join(ROCM, "lib"), "-lamdhip64",
           "-Wl,-rpath," + rpath]
    if verbose:
        print(" ".join(cmd))
    subprocess.run(cmd, check=True)
    return EXE


if __name__ == "__main__":
    build(verbose=True)
