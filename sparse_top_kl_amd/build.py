"""Builds libfkl.so (HIP kernels + C ABI) in-tree for gfx950 with hipcc.

Usage: ``python -m sparse_top_kl_amd.build`` (or ``__graft_entry__.build()``).
The library is written next to this file; the binding loads it from there.
``python -m sparse_top_kl_amd.build --sanitize`` builds a host-instrumented
copy (ASan + UBSan) under _objs_sanitized/, which a process selects with
FKL_LIBRARY and runs with the ASan runtime preloaded (sanitizer_runtime()).
"""

from __future__ import annotations

import concurrent.futures
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


# Host-side AddressSanitizer + UndefinedBehaviorSanitizer build of the same
# sources (the device code is compiled as usual): argument validation,
# workspace planning and the launch loops run instrumented. Each -fsanitize=
# is preceded by -Xarch_host so that it applies to the host compilation only.
SANITIZE_FLAGS = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
                  "-Xarch_host", "-fno-sanitize-recover=undefined",
                  "-Xarch_host", "-fno-omit-frame-pointer"]
SANITIZED_LIB = os.path.join(HERE, "_objs_sanitized", "libfkl_sanitized.so")


def sanitizer_runtime() -> str:
    """The clang ASan runtime (with the UBSan handlers) that a process using
    the sanitized library must preload."""
    llvm = os.path.join(os.path.dirname(os.path.dirname(hipcc())), "lib", "llvm", "lib", "clang")
    for ver in sorted(os.listdir(llvm), reverse=True):
        path = os.path.join(llvm, ver, "lib", "linux", "libclang_rt.asan-x86_64.so")
        if os.path.exists(path):
            return path
    raise RuntimeError("clang ASan runtime not found")


def build(verbose: bool = False, jobs: int | None = None, sanitize: bool = False) -> str:
    cc = hipcc()
    objdir = os.path.join(HERE, "_objs_sanitized" if sanitize else "_objs")
    os.makedirs(objdir, exist_ok=True)
    extra = ["-O1", "-g", *SANITIZE_FLAGS] if sanitize else []
    cmds, objs = [], []
    for src in SOURCES:
        obj = os.path.join(objdir, os.path.splitext(src)[0] + ".o")
        cmds.append([cc, *compile_flags(), *extra, "-x", "hip", "-c", os.path.join(CSRC, src),
                     "-o", obj])
        objs.append(obj)
    # one hipcc process per source, a few at a time
    jobs = jobs or min(len(cmds), max(1, min(4, (os.cpu_count() or 1) // 2)))
    with concurrent.futures.ThreadPoolExecutor(max_workers=jobs) as pool:
        for fut in [pool.submit(_run, c, verbose) for c in cmds]:
            fut.result()
    out = SANITIZED_LIB if sanitize else LIB
    tmp = out + ".tmp"
    link_extra = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
                  "-Xarch_host", "-shared-libsan"] if sanitize else []
    _run([cc, f"--offload-arch={ARCH}", "-shared", "-fPIC", *link_extra, *objs, "-o", tmp],
         verbose)
    os.replace(tmp, out)
    return out


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
    print(build(verbose=True, sanitize="--sanitize" in sys.argv[1:]))
