"""Build the C oracle into oracle/libwkv_oracle.so with gcc.

Test infrastructure only (see oracle/__init__.py).  The flags keep the fp64
arithmetic exactly as written: no fast-math, no fused multiply-add
contraction.
"""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "wkv_oracle.c")
LIB = os.path.join(HERE, "libwkv_oracle.so")

CFLAGS = ["-O2", "-std=c99", "-fopenmp", "-ffp-contract=off", "-fno-fast-math",
          "-fno-unsafe-math-optimizations", "-fPIC", "-shared", "-Wall", "-Wextra"]


def build(verbose: bool = False) -> str:
    """Compile the oracle library (always recompiles) and return its path."""
    tmp = LIB + ".tmp"
    cmd = ["gcc", *CFLAGS, "-o", tmp, SRC, "-lm"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
