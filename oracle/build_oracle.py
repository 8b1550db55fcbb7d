"""Compile the C oracle into ``oracle/liboracle.so`` (gcc, OpenMP, no fast-math).

Test infrastructure only: building the checker is not using it.
"""
from __future__ import annotations

import os
import shutil
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "gemm_oracle.c")
LIB = os.path.join(HERE, "liboracle.so")

CFLAGS = [
    "-std=c11", "-O2", "-fPIC", "-shared", "-fopenmp",
    # Products of fp32 values are exact in fp64, so contraction could not
    # change a result; keep the arithmetic literal anyway.
    "-ffp-contract=off", "-fno-fast-math",
    "-Wall", "-Wextra",
]


def build(verbose: bool = False) -> str:
    cc = shutil.which("gcc") or shutil.which("cc")
    if cc is None:
        raise RuntimeError("no C compiler (gcc) found to build the oracle")
    tmp = LIB + f".tmp{os.getpid()}"
    cmd = [cc, *CFLAGS, SRC, "-o", tmp, "-lm"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
