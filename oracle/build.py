"""Build the CPU oracle shared library (oracle/liboracle.so) with gcc.

TEST INFRASTRUCTURE ONLY: the oracle is the checker of the HIP library, never part of
it.  The flags fix the numeric ground rules the oracle is written against: IEEE binary32
on SSE2, no FMA contraction, no fast-math, round-to-nearest-even.
"""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "kvq_oracle.c")
LIB = os.path.join(HERE, "liboracle.so")

CFLAGS = ["-std=c11", "-O2", "-ffp-contract=off", "-fno-fast-math", "-fPIC", "-shared",
          "-Wall", "-Wextra", "-Wno-unused-parameter"]


def build(verbose: bool = False) -> str:
    """Compile the oracle; returns the path of the shared library."""
    tmp = LIB + ".tmp%d" % os.getpid()
    cmd = ["gcc"] + CFLAGS + ["-o", tmp, SRC, "-lm"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
    sys.exit(0)
