"""Build the CPU oracle (oracle/qmm_oracle.c) into oracle/liboracle.so with gcc.

Test infrastructure: the oracle is compiled with plain gcc, no HIP, strict
IEEE arithmetic (no contraction into fused multiply-adds, no fast-math), so
that every addition and product is the one written in the source.
"""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "qmm_oracle.c")
LIB = os.path.join(HERE, "liboracle.so")

CFLAGS = ["-O2", "-std=c11", "-fPIC", "-shared", "-ffp-contract=off", "-fno-fast-math",
          "-Wall", "-Wextra", "-pthread"]


def build(verbose=False):
    """Compile the oracle library; returns its path."""
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
