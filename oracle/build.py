"""Build the CPU oracle as a host shared library with g++ (no HIP, no SIMD flags).

Test infrastructure: see ``oracle/__init__.py``.
"""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
LIB = os.path.join(HERE, "librq_oracle.so")


def build(verbose: bool = False) -> str:
    src = os.path.join(HERE, "rq_oracle.cpp")
    # -ffp-contract=off: every rounding in the source is the rounding performed.
    cmd = ["g++", "-std=c++17", "-O2", "-fPIC", "-shared", "-ffp-contract=off",
           "-Wall", "-Wextra", "-o", LIB + ".tmp", src]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(LIB + ".tmp", LIB)
    return LIB


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
