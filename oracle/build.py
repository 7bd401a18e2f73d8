"""Compile the plain-C oracle (``gdn2_oracle.c``) into ``oracle/libgdn2_oracle.so``.

TEST INFRASTRUCTURE ONLY. Built with the host C compiler (gcc), in IEEE
float64 (no fast-math), OpenMP across (sequence, value head) work items.
"""

from __future__ import annotations

import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "gdn2_oracle.c")
LIB = os.path.join(HERE, "libgdn2_oracle.so")


def build_c_oracle(verbose: bool = False) -> str:
    """Compile the C oracle; returns the path of the shared library."""
    tmp = LIB + ".tmp"
    cmd = ["gcc", "-O2", "-std=c11", "-fopenmp", "-fPIC", "-shared", "-Wall",
           "-Wextra", SRC, "-o", tmp, "-lm"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build_c_oracle(verbose=True))
