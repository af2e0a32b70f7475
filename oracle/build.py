"""Compile the C oracle into oracle/liboracle.so (test infrastructure only)."""
from __future__ import annotations

import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "kv4_oracle.c")
LIB = os.path.join(HERE, "liboracle.so")

CFLAGS = ["-std=gnu11", "-O2", "-fno-fast-math", "-ffp-contract=off", "-fopenmp", "-fPIC",
          "-shared", "-Wall", "-Wextra", "-Wno-unused-parameter"]


# AddressSanitizer + UndefinedBehaviorSanitizer build of the same source (for
# the sanitized run of the oracle's pins; a process loading it needs libasan
# preloaded).  Host code only: the oracle has no GPU part.
SANITIZE = ["-fsanitize=address,undefined", "-fno-sanitize-recover=undefined", "-fno-omit-frame-pointer",
            "-g"]


def build(verbose: bool = False, sanitize: bool = False, out: str | None = None) -> str:
    lib = out or LIB
    tmp = lib + f".tmp{os.getpid()}"
    cmd = ["gcc", *CFLAGS, *(SANITIZE if sanitize else []), "-o", tmp, SRC, "-lm"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, lib)
    return lib


if __name__ == "__main__":
    print(build(verbose=True))
