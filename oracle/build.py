"""Build the CPU oracle library (oracle/liboracle.so) with gcc.

Test infrastructure: compiled by the package build step so that the checker
exists, but only the tests, the smoke check and the benchmark's CPU-baseline
leg load it.
"""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "oracle.c")
LIB = os.path.join(HERE, "liboracle.so")

# -ffp-contract=off: no implicit FMA; the only fused operations are the
# explicit fmaf() calls.  No -ffast-math, no -march flags.
CFLAGS = ["-O2", "-std=c11", "-ffp-contract=off", "-fno-fast-math", "-fPIC", "-shared", "-pthread",
          "-Wall", "-Wextra", "-fvisibility=hidden"]


def build(verbose: bool = False) -> str:
    tmp = LIB + ".tmp"
    cmd = ["gcc", *CFLAGS, "-o", tmp, SRC, "-lm"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
