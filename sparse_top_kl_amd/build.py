"""Builds libfkl.so (HIP kernels + C ABI) in-tree for gfx950 with hipcc.

Usage: ``python -m sparse_top_kl_amd.build`` (or ``__graft_entry__.build()``).
The library is written next to this file; the binding loads it from there.
"""

from __future__ import annotations

import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(HERE, "libfkl.so")

SOURCES = ["kernels.hip", "topk.hip", "renorm.hip", "fkl_api.cpp", "topk_api.cpp",
           "renorm_api.cpp", "timing.cpp"]
ARCH = "gfx950"


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found: the HIP toolchain is required to build libfkl")


def compile_flags() -> list[str]:
    return [
        "-O3",
        "-std=c++17",
        f"--offload-arch={ARCH}",
        "-fPIC",
        "-Wall",
        "-Wno-unused-function",
        # keep the compiler from forming packed fp32 instructions
        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
        "-I", INCLUDE,
        "-I", CSRC,
    ]


def build(verbose: bool = False) -> str:
    cc = hipcc()
    objs = []
    os.makedirs(os.path.join(HERE, "_objs"), exist_ok=True)
    for src in SOURCES:
        obj = os.path.join(HERE, "_objs", os.path.splitext(src)[0] + ".o")
        cmd = [cc, *compile_flags(), "-x", "hip", "-c", os.path.join(CSRC, src), "-o", obj]
        _run(cmd, verbose)
        objs.append(obj)
    tmp = LIB + ".tmp"
    _run([cc, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp], verbose)
    os.replace(tmp, LIB)
    return LIB


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    noise = "'-packed-fp32-ops' is not a recognized feature for this target"
    err = "\n".join(l for l in res.stderr.splitlines() if noise not in l)
    if res.returncode != 0:
        raise RuntimeError(f"build failed: {' '.join(cmd)}\n{err}")
    if verbose and err.strip():
        print(err, file=sys.stderr)


if __name__ == "__main__":
    print(build(verbose=True))
