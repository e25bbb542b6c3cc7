"""Build the CPU oracle (plain C, gcc) into oracle/_build/liboracle.so.

Test infrastructure: the oracle is a checker, never part of the product path.
Flags keep fp32 arithmetic exactly as written: no contraction of a*b+c into
FMA (only the explicit fmaf calls fuse), no fast-math, IEEE single precision
in SSE registers.
"""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "growpage_oracle.c")
OUT_DIR = os.path.join(HERE, "_build")
LIB = os.path.join(OUT_DIR, "liboracle.so")

CFLAGS = ["-O2", "-std=c11", "-fPIC", "-shared", "-ffp-contract=off",
          "-fno-fast-math", "-mfma", "-Wall", "-Wextra"]


def build(verbose: bool = False) -> str:
    """Compile the oracle; returns the path of the shared library."""
    os.makedirs(OUT_DIR, exist_ok=True)
    tmp = LIB + ".tmp"
    cmd = ["gcc", *CFLAGS, SRC, "-o", tmp, "-lm"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
