"""Build the synthetic-input generators: libsynth_cpu.so (gcc) and
libsynth_gpu.so (hipcc, gfx950)."""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
CPU_LIB = os.path.join(HERE, "libsynth_cpu.so")
GPU_LIB = os.path.join(HERE, "libsynth_gpu.so")

HIP_FLAGS = ["--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
             "-ffp-contract=off", "-fhip-fp32-correctly-rounded-divide-sqrt",
             "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)


def build(verbose: bool = False):
    tmp = CPU_LIB + ".tmp%d" % os.getpid()
    _run(["gcc", "-std=c11", "-O3", "-fPIC", "-shared", "-ffp-contract=off", "-Wall",
          "-o", tmp, os.path.join(HERE, "synth_cpu.c")], verbose)
    os.replace(tmp, CPU_LIB)
    tmp = GPU_LIB + ".tmp%d" % os.getpid()
    _run(["hipcc"] + HIP_FLAGS + ["-o", tmp, os.path.join(HERE, "synth_gpu.hip")], verbose)
    os.replace(tmp, GPU_LIB)
    return CPU_LIB, GPU_LIB


if __name__ == "__main__":
    build(verbose=True)
