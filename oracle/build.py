"""Builds the C oracle (``kda_oracle.c``, ``kda_oracle_bwd.c``) into ``oracle/libkda_oracle.so``
with gcc and OpenMP.

Test infrastructure: the HIP library neither builds nor loads this file.
"""

from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
SRCS = [os.path.join(HERE, "kda_oracle.c"), os.path.join(HERE, "kda_oracle_bwd.c")]
LIB = os.path.join(HERE, "libkda_oracle.so")


def build_oracle(force: bool = True) -> str:
    if not force and os.path.exists(LIB) and all(
            os.path.getmtime(LIB) >= os.path.getmtime(src) for src in SRCS):
        return LIB
    tmp = LIB + ".tmp"
    cmd = ["gcc", "-O2", "-std=c99", "-fopenmp", "-fPIC", "-shared", "-Wall", "-Wextra",
           *SRCS, "-o", tmp, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build_oracle(force="--if-stale" not in sys.argv))
