"""Compile the CPU oracle (orc.c) into oracle/liborc.so with gcc.

Test infrastructure: the oracle is plain C with IEEE fp32 arithmetic, built
without FMA contraction and without fast-math so that each product and
quotient is rounded once, to nearest even.
"""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "orc.c")
LIB = os.path.join(HERE, "liborc.so")

CFLAGS = ["-std=c99", "-O2", "-fPIC", "-shared", "-ffp-contract=off", "-fno-fast-math",
          "-Wall", "-Wextra", "-Wno-unused-parameter"]


def build(verbose: bool = False) -> str:
    cmd = ["gcc", *CFLAGS, SRC, "-o", LIB + ".tmp", "-lm"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(LIB + ".tmp", LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
