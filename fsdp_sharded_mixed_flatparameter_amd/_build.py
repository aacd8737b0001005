"""Build libzeroflat.so in-tree: hipcc for gfx950 (MI355X).

Flags that fix the arithmetic: -ffp-contract=off (no FMA fusion: every fp32
operation rounds on its own, as the step is defined) and correctly rounded
fp32 division and square root.  Packed-fp32 instructions are disabled.
"""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
LIB = os.path.join(HERE, "libzeroflat.so")
SOURCES = [os.path.join(HERE, "csrc", "zeroflat_kernels.hip"),
           os.path.join(HERE, "csrc", "zeroflat_api.cpp")]

HIPCC_FLAGS = ["--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
               "-ffp-contract=off", "-fhip-fp32-correctly-rounded-divide-sqrt",
               "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
               "-Wall", "-I", os.path.join(ROOT, "include"), "-I", os.path.join(HERE, "csrc")]


def build(verbose: bool = False, extra_flags=()) -> str:
    tmp = LIB + ".tmp%d" % os.getpid()
    cmd = ["hipcc"] + HIPCC_FLAGS + list(extra_flags) + ["-o", tmp] + SOURCES
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    build(verbose=True)
