"""Compile the C oracle (gla_oracle.c) into oracle/libgla_oracle.so with gcc.

TEST INFRASTRUCTURE ONLY (see oracle/__init__.py).
"""
from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "gla_oracle.c")
LIB = os.path.join(HERE, "libgla_oracle.so")


def build(verbose: bool = False) -> str:
    """Compile the oracle library (always recompiles) and return its path."""
    tmp = LIB + ".tmp%d" % os.getpid()
    cmd = ["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-fopenmp",
           "-Wall", "-Wextra", "-o", tmp, SRC, "-lm"]
    if verbose:
        print(" ".join(cmd), file=sys.stderr)
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB)
    return LIB


def ensure_built() -> str:
    """Return the library path, building it only if it is missing or stale."""
    if (not os.path.exists(LIB)
            or os.path.getmtime(LIB) < os.path.getmtime(SRC)):
        return build()
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
