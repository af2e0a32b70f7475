"""Compile the C oracle into oracle/liboracle.so (test infrastructure only)."""
from __future__ import annotations

import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "kv4_oracle.c")
LIB = os.path.join(HERE, "liboracle.so")

CFLAGS = ["-std=gnu11", "-O2", "-fno-fast-math", "-ffp-contract=off", "-fopenmp", "-fPIC",
          "-shared", "-Wall", "-Wextra", "-Wno-unused-parameter"]


def build(verbose: bool = False) -> str:
    tmp = LIB + f".tmp{os.getpid()}"
    cmd = ["gcc", *CFLAGS, "-o", tmp, SRC, "-lm"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
