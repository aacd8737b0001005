"""Build libzeroflat.so in-tree: hipcc for gfx950 (MI355X).

Flags that fix the arithmetic: -ffp-contract=off (no FMA fusion: every fp32
operation rounds on its own, as the step is defined) and correctly rounded
fp32 division and square root.  Packed-fp32 instructions are disabled.
The host-only source (the ZeRO-Offload step) is built by ROCm's clang++ with
the same contraction rule and -fno-math-errno, which lets its square roots
vectorize and changes no result.
"""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
LIB = os.path.join(HERE, "libzeroflat.so")
SOURCES = [os.path.join(HERE, "csrc", "zeroflat_kernels.hip"),
           os.path.join(HERE, "csrc", "zeroflat_api.cpp")]
# host-only C++ (the ZeRO-Offload host step): built by the host compiler, so
# that it can carry one machine-code clone per x86 ISA level
HOST_SOURCES = [os.path.join(HERE, "csrc", "zeroflat_offload.cpp")]
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")
HOST_FLAGS = ["-O3", "-std=c++17", "-fPIC", "-ffp-contract=off", "-fno-math-errno", "-Wall",
              "-D__HIP_PLATFORM_AMD__", "-I", os.path.join(ROCM, "include"),
              "-I", os.path.join(ROOT, "include"), "-I", os.path.join(HERE, "csrc")]

HIPCC_FLAGS = ["--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
               "-ffp-contract=off", "-fhip-fp32-correctly-rounded-divide-sqrt",
               "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
               "-Wall", "-I", os.path.join(ROOT, "include"), "-I", os.path.join(HERE, "csrc")]


def build(verbose: bool = False, extra_flags=()) -> str:
    tmp = LIB + ".tmp%d" % os.getpid()
    tag = "_%d.o" % os.getpid()
    objs = []

    def run(cmd):
        if verbose:
            print(" ".join(cmd), flush=True)
        subprocess.run(cmd, check=True)

    try:
        for src in SOURCES:
            obj = os.path.join(HERE, os.path.splitext(os.path.basename(src))[0] + tag)
            objs.append(obj)
            run(["hipcc"] + HIPCC_FLAGS + list(extra_flags) + ["-c", "-o", obj, src])
        for src in HOST_SOURCES:
            obj = os.path.join(HERE, os.path.splitext(os.path.basename(src))[0] + tag)
            objs.append(obj)
            run([os.path.join(ROCM, "llvm", "bin", "clang++")] + HOST_FLAGS + ["-c", "-o", obj, src])
        run(["hipcc", "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp] + objs)
    finally:
        for obj in objs:
            if os.path.exists(obj):
                os.remove(obj)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    build(verbose=True)
