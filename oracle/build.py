"""Compile the C oracle into oracle/libkda_oracle.so with gcc.

-O3 may vectorise the loops over value columns j (independent sums, so the
result is unchanged); without -ffast-math gcc never reassociates a sum.

TEST INFRASTRUCTURE ONLY.  -ffp-contract=off keeps every multiply and add a
separately rounded fp32 operation, so the oracle's rounding is fixed by its
source order; -fno-fast-math keeps IEEE semantics (denormals, inf, NaN).
"""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "kda_oracle.c")
LIB = os.path.join(HERE, "libkda_oracle.so")

CFLAGS = ["-O3", "-std=c11", "-fPIC", "-shared", "-ffp-contract=off",
          "-fno-fast-math", "-Wall", "-Wextra"]


def build(verbose: bool = False) -> str:
    """Always recompiles (a build check must compile); returns the .so path."""
    tmp = LIB + ".tmp%d" % os.getpid()
    cmd = ["gcc", *CFLAGS, SRC, "-o", tmp, "-lm"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
