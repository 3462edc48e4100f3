"""Compile the fp64 CPU oracle (test infrastructure) with gcc.

Building the checker is not using it: the package build compiles it so that
tests and the CPU baseline find it ready.
"""

from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "lmhead_oracle.c")
LIB = os.path.join(HERE, "liboracle.so")


def build(force: bool = True) -> str:
    if not force and os.path.exists(LIB) and os.path.getmtime(LIB) >= os.path.getmtime(SRC):
        return LIB
    tmp = LIB + ".tmp"
    cmd = ["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-pthread",
           "-fno-fast-math", "-ffp-contract=off", SRC, "-o", tmp]
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(force="--lazy" not in sys.argv))
