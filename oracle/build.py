"""Build the CPU oracle (plain C, gcc) into oracle/libsckv_oracle.so.

Test infrastructure only: the library this builds is loaded by the tests, the
smoke check and the bench's CPU-baseline leg, never by the product path.
"""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "sckv_oracle.c")
LIB = os.path.join(HERE, "libsckv_oracle.so")

# Strict IEEE: no contraction into FMA, no fast-math, SSE2 binary32/binary64.
CFLAGS = ["-O2", "-std=gnu11", "-fPIC", "-shared", "-ffp-contract=off", "-fno-fast-math",
          "-fno-finite-math-only", "-Wall", "-Wextra"]


def build(verbose: bool = False) -> str:
    cmd = ["gcc", *CFLAGS, "-o", LIB + ".tmp", SRC, "-lm"]
    if verbose:
        print(" ".join(cmd))
    subprocess.run(cmd, check=True)
    os.replace(LIB + ".tmp", LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
