"""Build libkv4.so (the HIP library behind include/kv4.h) for gfx950, in tree."""
from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libkv4.so")
SOURCES = ["kv4_api.hip", "kv4_quantize.hip", "kv4_decode.hip", "kv4_prefill_attn.hip", "kv4_bf16.hip"]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
INCLUDE = os.path.join(os.path.dirname(HERE), "include")

FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
    "-ffp-contract=off",                      # no silent FMA contraction: rounding is part of the rules
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function", "-I" + INCLUDE,
]


def build(verbose: bool = False, jobs: int = 4, defines=(), out: str | None = None) -> str:
    """Compile every source to an object in parallel, then link; returns the
    library path.  defines / out: a variant build of the same sources (for
    instance KV4_MAIN_WAVES_PER_SIMD=3) into another library file, for A/B
    measurements; the default is libkv4.so."""
    lib = out or LIB
    objdir = os.path.join(HERE, "_build" if not defines else "_build_" + "_".join(d.replace("=", "") for d in defines))
    os.makedirs(objdir, exist_ok=True)
    procs, objs = [], []
    for src in SOURCES:
        obj = os.path.join(objdir, src.replace(".hip", ".o"))
        cmd = [HIPCC, *[f for f in FLAGS if f != "-shared"], *["-D" + d for d in defines], "-c",
               os.path.join(CSRC, src), "-o", obj]
        if verbose:
            print(" ".join(cmd), flush=True)
        procs.append((src, subprocess.Popen(cmd)))
        objs.append(obj)
    failed = [src for src, p in procs if p.wait() != 0]
    if failed:
        raise RuntimeError(f"hipcc failed on {failed}")
    tmp = lib + f".tmp{os.getpid()}"
    cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp, *objs]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, lib)
    return lib


if __name__ == "__main__":
    import argparse
    ap = argparse.ArgumentParser()
    ap.add_argument("-v", action="store_true")
    ap.add_argument("--define", action="append", default=[], help="NAME=VALUE for every source")
    ap.add_argument("--out", default=None, help="library path (default: libkv4.so in the package)")
    args = ap.parse_args()
    print(build(verbose=args.v, defines=tuple(args.define), out=args.out))
