"""Build libbi.so (the C-ABI HIP library) for gfx950 with hipcc.

One fixed flag set for every kernel: -O3, no fast-math, -ffp-contract=off
(a*b+c stays a rounded multiply then a rounded add), packed-fp32 ops off,
MFMA results kept in ordinary VGPRs.
Run as ``python -m invariant_bi_matmul_amd._build``; ``__graft_entry__.build()``
calls :func:`build`.
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
OBJDIR = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libbi.so")
# the same library with BI_DEBUG_CHECKS: attention calls validate their index arrays first
DEBUG_LIB = os.path.join(HERE, "libbi_debug.so")
SOURCES = ["rmsnorm.hip", "matmul.hip", "attention.hip", "model.hip", "measure.hip", "checks.hip",
           "api.cpp"]
ARCH = "gfx950"

FLAGS = [
    "-O3", "-std=c++17", "-fPIC", "--offload-arch=" + ARCH,
    "-ffp-contract=off", "-fno-fast-math",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # MFMA results in ordinary VGPRs: the softmax and fold read them with VALU,
    # and accumulation registers would need a copy per value
    "-mllvm", "-amdgpu-mfma-vgpr-form=true",
    "-Wall", "-Wno-unused-function",
]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found: the HIP library cannot be built")


def _compile(src: str, debug: bool = False) -> str:
    obj = os.path.join(OBJDIR, os.path.splitext(src)[0] + ("_debug" if debug else "") + ".o")
    cmd = [hipcc()] + FLAGS + (["-DBI_DEBUG_CHECKS"] if debug else []) + ["-I", INCLUDE, "-I", CSRC]
    if src.endswith(".cpp"):
        cmd += ["-x", "hip"]
    cmd += ["-c", os.path.join(CSRC, src), "-o", obj]
    res = subprocess.run(cmd, capture_output=True, text=True)
    # hipcc's host pass does not know the packed-fp32 feature; that note is harmless
    noise = "'-packed-fp32-ops' is not a recognized feature"
    err = "\n".join(l for l in res.stderr.splitlines() if noise not in l)
    if res.returncode != 0:
        raise RuntimeError("hipcc failed on %s:\n%s" % (src, err))
    if err.strip():
        sys.stderr.write(err + "\n")
    return obj


def _link(objs, lib: str) -> None:
    tmp = lib + ".tmp%d" % os.getpid()
    cmd = [hipcc(), "-shared", "-fPIC", "--offload-arch=" + ARCH] + objs + ["-o", tmp]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError("link failed:\n" + res.stderr)
    os.replace(tmp, lib)


def build(verbose: bool = True) -> str:
    """Compile every source and link libbi.so and libbi_debug.so in-tree (the
    debug library differs only in api.cpp).  Always rebuilds."""
    os.makedirs(OBJDIR, exist_ok=True)
    jobs = [(src, False) for src in SOURCES] + [("api.cpp", True)]
    with concurrent.futures.ThreadPoolExecutor(max_workers=len(jobs)) as ex:
        objs = list(ex.map(lambda j: _compile(*j), jobs))
    release, debug_api = objs[:len(SOURCES)], objs[-1]
    _link(release, LIB)
    _link([o for o in release if not o.endswith(os.sep + "api.o")] + [debug_api], DEBUG_LIB)
    if verbose:
        print("built", LIB, "and", DEBUG_LIB)
    return LIB


if __name__ == "__main__":
    build()
