"""Build the CPU oracle shared library with gcc.

Test infrastructure: the library this builds is loaded only by the test
suite, the smoke check and the benchmark's CPU-baseline leg.
"""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "nvfp4_oracle.c")
LIB = os.path.join(HERE, "liboracle_nvfp4.so")

# -ffp-contract=off: no silent FMA contraction; no -ffast-math: IEEE binary32
# semantics (correctly rounded division, signed zeros, RNE rint).
CFLAGS = ["-std=c11", "-O2", "-fopenmp", "-ffp-contract=off", "-fno-fast-math",
          "-fPIC", "-shared", "-Wall", "-Wextra"]


def build(verbose: bool = False) -> str:
    tmp = LIB + ".tmp%d" % os.getpid()
    cmd = ["gcc", *CFLAGS, SRC, "-o", tmp, "-lm"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
