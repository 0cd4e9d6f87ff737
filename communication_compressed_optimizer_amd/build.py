"""Build libonebit.so (the C-ABI library and its gfx950 kernels) in-tree,
and libonebit_ceiling.so (pure-traffic kernels that measure the machine's
practical HBM ceiling for the same access patterns; used by bench.py only).

Flags that matter for results: contraction off (no fused multiply-add may
merge two roundings), correctly rounded fp32 division and square root, fp32
denormals kept, and no packed-fp32 instructions.
"""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
LIB = os.path.join(HERE, "libonebit.so")
CEILING_LIB = os.path.join(HERE, "libonebit_ceiling.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = os.environ.get("ONEBIT_ARCH", "gfx950")

FLAGS = ["--offload-arch=" + ARCH, "-O3", "-std=c++17", "-fPIC", "-shared", "-ffp-contract=off",
         "-fhip-fp32-correctly-rounded-divide-sqrt", "-fno-gpu-flush-denormals-to-zero",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", "-Wall"]


def _hipcc(src, out, verbose, extra):
    cmd = [HIPCC, *FLAGS, *extra, "-I", os.path.join(ROOT, "include"), "-I",
           os.path.join(HERE, "csrc"), "-o", out, src]
    if verbose:
        print(" ".join(cmd))
    res = subprocess.run(cmd, capture_output=True, text=True)
    msgs = [ln for ln in (res.stderr or "").splitlines() if "packed-fp32-ops" not in ln]
    if res.returncode != 0:
        sys.stderr.write("\n".join(msgs) + "\n")
        raise RuntimeError(f"hipcc failed building {os.path.basename(out)}")
    if verbose and msgs:
        print("\n".join(msgs))


def build(verbose=False, extra=()):
    _hipcc(os.path.join(HERE, "csrc", "onebit.hip"), LIB, verbose, extra)
    _hipcc(os.path.join(HERE, "csrc", "ceiling.hip"), CEILING_LIB, verbose, extra)
    return LIB


if __name__ == "__main__":
    build(verbose=True)
