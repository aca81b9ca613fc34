"""Compile the C oracle into oracle/libkda_oracle.so with gcc.

-O3 may vectorise the loops over value columns j (independent sums, so the
result is unchanged); without -ffast-math gcc never reassociates a sum.

TEST INFRASTRUCTURE ONLY.  -ffp-contract=off keeps every multiply and add a
separately rounded fp32 operation, so the oracle's rounding is fixed by its
source order; -fno-fast-math keeps IEEE semantics (denormals, inf, NaN).
"""
from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "kda_oracle.c")
LIB = os.path.join(HERE, "libkda_oracle.so")

CFLAGS = ["-O3", "-std=c11", "-fPIC", "-shared", "-ffp-contract=off",
          "-fno-fast-math", "-Wall", "-Wextra"]


# A build for the sanitizer run of the oracle's pins (tests only): address
# and undefined-behaviour checks, the first report fatal.
SANITIZE_FLAGS = ["-O1", "-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
                  "-fno-sanitize-recover=all"]


def build(verbose: bool = False, out: str | None = None, sanitize: bool = False) -> str:
    """Always recompiles (a build check must compile); returns the .so path.
    `out` writes the library elsewhere; `sanitize` adds SANITIZE_FLAGS (a
    library for a process that preloads the sanitizer runtimes)."""
    dst = LIB if out is None else out
    tmp = dst + ".tmp%d" % os.getpid()
    cflags = [f for f in CFLAGS if f != "-O3"] + SANITIZE_FLAGS if sanitize else CFLAGS
    cmd = ["gcc", *cflags, SRC, "-o", tmp, "-lm"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, dst)
    return dst


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
