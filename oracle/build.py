"""Build the CPU oracle's shared library (oracle/liboracle.so) with gcc.

Test infrastructure only: the product library neither builds nor loads it.
"""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "gemm_ref.c")
LIB = os.path.join(HERE, "liboracle.so")

CFLAGS = ["-O2", "-std=c11", "-fopenmp", "-ffp-contract=off", "-fno-fast-math",
          "-fPIC", "-shared", "-Wall", "-Wextra"]


def build(verbose: bool = False) -> str:
    """Compile gemm_ref.c into liboracle.so (always recompiles) and return its path."""
    tmp = LIB + ".tmp"
    cmd = ["gcc", *CFLAGS, SRC, "-o", tmp, "-lm"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB)
    return LIB


def ensure_built() -> str:
    """Build the library if it is missing or older than its source."""
    if not os.path.exists(LIB) or os.path.getmtime(LIB) < os.path.getmtime(SRC):
        return build()
    return LIB


if __name__ == "__main__":
    build(verbose="-v" in sys.argv)
