"""Build the CPU oracle (test infrastructure only) into oracle/liboracle.so.

g++ with contraction off and no fast-math, so each float operation in
oracle.cpp is one IEEE-754 operation rounded to nearest-even.
"""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
LIB = os.path.join(HERE, "liboracle.so")


def build(verbose: bool = False) -> str:
    src = os.path.join(HERE, "oracle.cpp")
    tmp = LIB + ".tmp%d" % os.getpid()
    cmd = ["g++", "-std=c++17", "-O2", "-fPIC", "-shared", "-ffp-contract=off",
           "-fno-fast-math", "-mfpmath=sse", "-Wall", "-Wextra",
           "-o", tmp, src]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
