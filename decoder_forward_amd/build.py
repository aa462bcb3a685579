"""Build the HIP library libdecfwd.so in-tree for gfx950.

All HIP sources compile with hipcc, -O3, for gfx950 only. Packed-fp32
instruction selection is turned off for device code
(`-Xclang -target-feature -Xclang -packed-fp32-ops`); the host pass warns
that it does not know the feature, which is harmless.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libdecfwd.so")
SOURCES = ["runtime.hip", "decode.hip", "prefill.hip"]


def hipcc() -> str:
    for cand in (shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found")


def build(verbose: bool = False, jobs: int = 4) -> str:
    objs = []
    procs = []
    base = [hipcc(), "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
            "-Wall", "-Wno-unused-command-line-argument",
            "-I", os.path.join(HERE, "..", "include")]
    for src in SOURCES:
        path = os.path.join(CSRC, src)
        if not os.path.exists(path):
            continue
        obj = os.path.join(CSRC, src.replace(".hip", ".o"))
        cmd = base + ["-c", path, "-o", obj]
        if verbose:
            print(" ".join(cmd), flush=True)
        procs.append((subprocess.Popen(cmd), src))
        objs.append(obj)
        if len(procs) >= jobs:
            p, s = procs.pop(0)
            if p.wait() != 0:
                raise RuntimeError(f"hipcc failed on {s}")
    for p, s in procs:
        if p.wait() != 0:
            raise RuntimeError(f"hipcc failed on {s}")
    tmp = LIB + ".tmp"
    cmd = [hipcc(), "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp] + objs
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB)
    for o in objs:
        try:
            os.remove(o)
        except OSError:
            pass
    return LIB


if __name__ == "__main__":
    build(verbose="-v" in sys.argv)
