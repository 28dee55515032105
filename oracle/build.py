"""Build the CPU oracle shared library (plain C, gcc).

Test infrastructure: the oracle is loaded only by the test suite, the smoke
check and the CPU-baseline leg of the benchmark.
"""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "fp4_oracle.c")
LIB = os.path.join(HERE, "libfp4_oracle.so")

# -ffp-contract=off: no fused multiply-add, every product and sum is rounded
# exactly where the source says.  No -ffast-math, so IEEE semantics hold.
CFLAGS = ["-O2", "-std=c11", "-fPIC", "-shared", "-ffp-contract=off", "-fno-fast-math",
          "-Wall", "-Wextra"]


def build(verbose: bool = False) -> str:
    cmd = ["gcc", *CFLAGS, SRC, "-o", LIB, "-lm"]
    if verbose:
        print(" ".join(cmd))
    subprocess.run(cmd, check=True)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
