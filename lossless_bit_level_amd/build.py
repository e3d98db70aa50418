"""Build libibp.so (the IBP library) and libibp_ceiling.so (the gather-copy
floor the benchmark measures it against) in-tree with hipcc for gfx950.

Usage: python -m lossless_bit_level_amd.build
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
SRC = os.path.join(PKG, "csrc", "ibp.hip")
LIB = os.path.join(PKG, "libibp.so")
CEILING_SRC = os.path.join(PKG, "csrc", "ceiling.hip")
CEILING_LIB = os.path.join(PKG, "libibp_ceiling.so")
INCLUDE = os.path.join(ROOT, "include")


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build libibp)")


def command(out: str = LIB, extra=(), src: str = SRC) -> list[str]:
    return [hipcc(), "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
            "-Wall", "-I", INCLUDE,
            # packed fp32 instructions are kept out of every kernel
            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
            *extra, src, "-o", out]


def build(verbose: bool = False) -> str:
    """Compile both libraries, side by side (always recompiles; the IBP
    library takes about a minute)."""
    jobs = []
    for src, lib in ((SRC, LIB), (CEILING_SRC, CEILING_LIB)):
        cmd = command(lib + ".tmp", src=src)
        if verbose:
            print(" ".join(cmd), flush=True)
        jobs.append((lib, subprocess.Popen(cmd, stdout=subprocess.PIPE,
                                           stderr=subprocess.STDOUT, text=True)))
    failed = []
    for lib, proc in jobs:
        out, _ = proc.communicate()
        if proc.returncode != 0:
            sys.stderr.write(out)
            failed.append(os.path.basename(lib))
        else:
            os.replace(lib + ".tmp", lib)
    if failed:
        raise RuntimeError(f"hipcc failed to build {', '.join(failed)}")
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
