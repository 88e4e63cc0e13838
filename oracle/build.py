"""Compile the fp64 CPU oracle (test infrastructure) into oracle/liboracle.so.

Plain gcc with OpenMP; no GPU code.  Called by the package build entry point
and, when the library is missing, by the oracle wrapper itself.
"""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "attn_oracle.c")
LIB = os.path.join(HERE, "liboracle.so")

# x86-64-v3 (AVX2 + FMA) is the common baseline of the build host and the
# GPU hosts; no -ffast-math so the fp64 arithmetic keeps IEEE semantics
# (inf handling, no reassociation).
CFLAGS = ["-O3", "-march=x86-64-v3", "-fno-fast-math", "-fopenmp", "-fPIC",
          "-shared", "-std=c11", "-Wall", "-Wextra", "-Wno-unused-parameter"]


def build(verbose: bool = False) -> str:
    tmp = LIB + ".tmp%d" % os.getpid()
    cmd = ["gcc", *CFLAGS, SRC, "-o", tmp, "-lm"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
