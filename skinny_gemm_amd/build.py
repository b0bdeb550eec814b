"""Build libskinny_gemm.so in-tree with hipcc for gfx950.

Each .hip file under csrc/ compiles to an object in parallel, then one link
produces skinny_gemm_amd/libskinny_gemm.so.  Run as
``python -m skinny_gemm_amd.build`` or through ``__graft_entry__.build()``.
"""
from __future__ import annotations

import concurrent.futures
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libskinny_gemm.so")
ARCH = "gfx950"


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (need ROCm with gfx950 support)")


def compile_flags():
    return [
        "--offload-arch=" + ARCH, "-O3", "-std=c++17", "-fPIC",
        "-I", CSRC, "-I", INCLUDE,
        # keep the compiler from forming packed-fp32 instructions
        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
        # matrix-core results in ordinary VGPRs: the integer block sums feed
        # float epilogues directly instead of through accumulation registers
        "-mllvm", "-amdgpu-mfma-vgpr-form",
        # kernel arguments arrive in SGPRs with the wave instead of through a
        # scalar load at its start: every launch reaches its first weight load
        # sooner (MI355X, the Llama-2-7B Q4_0 decode token: 1.109 -> 1.056 ms
        # at M = 1, 1.625 -> 1.566 ms at M = 8, same box)
        "-mllvm", "-amdgpu-kernarg-preload-count=16",
        "-Wall", "-Wno-unused-function",
    ]


def sources():
    return sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith(".hip"))


def _compile(src: str) -> str:
    obj = os.path.join(BUILD, os.path.basename(src)[:-4] + ".o")
    cmd = [hipcc()] + compile_flags() + ["-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("compile failed: %s\n%s\n%s" % (" ".join(cmd), r.stdout, r.stderr))
    return obj


def build(verbose: bool = True) -> str:
    """Compile every source (always) and link the shared library."""
    os.makedirs(BUILD, exist_ok=True)
    srcs = sources()
    workers = min(len(srcs), max(1, min(8, os.cpu_count() or 1)))
    with concurrent.futures.ThreadPoolExecutor(workers) as ex:
        objs = list(ex.map(_compile, srcs))
    tmp = LIB + ".tmp%d" % os.getpid()
    cmd = [hipcc(), "--offload-arch=" + ARCH, "-shared", "-fPIC", "-o", tmp] + objs
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed: %s\n%s\n%s" % (" ".join(cmd), r.stdout, r.stderr))
    os.replace(tmp, LIB)
    if verbose:
        print("built", LIB, file=sys.stderr)
    return LIB


if __name__ == "__main__":
    build()
