"""Compiles the oracle's C++ source into ``oracle/libspconv_oracle.so``.

TEST INFRASTRUCTURE ONLY: the oracle is loaded by the tests, the smoke check
and the bench's CPU-baseline leg, never by the product path.
"""
from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "spconv_oracle.cpp")
LIB = os.path.join(HERE, "libspconv_oracle.so")


def build(verbose: bool = False) -> str:
    """Compile the oracle with g++ (no fast-math) and return the library path."""
    tmp = LIB + ".tmp"
    cmd = ["g++", "-O2", "-std=c++17", "-fopenmp", "-shared", "-fPIC", "-Wall", "-Wextra", "-o", tmp, SRC]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
