"""Compile the fp64 CPU attention oracle (``fa_oracle.c``) into ``liboracle.so``.

Test infrastructure only: the library built here is loaded by the test suite,
the smoke check and the CPU-baseline leg of the benchmark, never by the
product path.
"""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "fa_oracle.c")
LIB = os.path.join(HERE, "liboracle.so")

# -ffp-contract=off: no fused multiply-add, every product and sum rounds once in fp64.
CFLAGS = ["-O3", "-fopenmp", "-fPIC", "-shared", "-ffp-contract=off", "-fno-fast-math", "-std=c11"]


def build(verbose: bool = False) -> str:
    """Always recompiles; returns the path of the shared library."""
    tmp = LIB + ".tmp"
    cmd = ["gcc", *CFLAGS, SRC, "-o", tmp, "-lm"]
    if verbose:
        print(" ".join(cmd))
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
