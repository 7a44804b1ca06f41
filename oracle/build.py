"""Build the CPU oracle (oracle/liblco.so) with gcc.

Test infrastructure: the oracle is compiled so that the tests, the smoke check
and the benchmark's CPU-baseline leg can load it.  Every IEEE operation is
kept as written: no FMA contraction, no fast-math, subnormals kept.
"""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
LIB = os.path.join(HERE, "liblco.so")
CFLAGS = ["-std=c11", "-O2", "-ffp-contract=off", "-fno-fast-math",
          "-fno-unsafe-math-optimizations", "-Wall", "-Wextra", "-fPIC", "-shared"]


def build(verbose=False):
    src = os.path.join(HERE, "lco.c")
    tmp = LIB + ".tmp"
    cmd = ["gcc", *CFLAGS, "-o", tmp, src, "-lm"]
    if verbose:
        print(" ".join(cmd))
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
