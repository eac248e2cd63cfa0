"""Build libmla_paged_kv.so (hand-written HIP for gfx950) in-tree.

    python -m mla_paged_kv_02_amd.build            # the library
    python -m mla_paged_kv_02_amd.build --stamps   # + libmla_paged_kv_stamps.so

Each source compiles to an object under _build/ in parallel, then one
hipcc link produces mla_paged_kv_02_amd/libmla_paged_kv.so.  With --stamps
a second copy is built with MLA_STAMPS=1: its decode kernels also record
each workgroup's start and end (mla_paged_kv_02_amd/stamps.py reads them);
the library itself never contains that code.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libmla_paged_kv.so")
STAMPS_LIB = os.path.join(PKG, "libmla_paged_kv_stamps.so")
SOURCES = ["abi.cpp", "metadata.hip", "decode.hip", "decode_wide.hip", "combine.hip", "absorb.hip",
           "probes.hip", "noalloc.hip"]
ARCH = "gfx950"
FLAGS = ["--offload-arch=" + ARCH, "-O3", "-std=c++17", "-fPIC", "-Wall",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-I" + os.path.join(ROOT, "include")]


def _hipcc() -> str:
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found; ROCm is required to build libmla_paged_kv.so")


def _compile(src: str, stamps: bool = False) -> str:
    obj = os.path.join(BUILD, os.path.basename(src) + (".stamps.o" if stamps else ".o"))
    extra = ["-DMLA_STAMPS=1"] if stamps else []
    cmd = [_hipcc(), *FLAGS, *extra, "-x", "hip", "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("hipcc failed for %s:\n%s\n%s" % (src, " ".join(cmd), r.stderr))
    return obj


def build(verbose: bool = False, stamps: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    lib = STAMPS_LIB if stamps else LIB
    with cf.ThreadPoolExecutor(max_workers=min(len(SOURCES), os.cpu_count() or 1)) as ex:
        objs = list(ex.map(lambda s: _compile(s, stamps), SOURCES))
    tmp = lib + ".tmp%d" % os.getpid()
    cmd = [_hipcc(), "--offload-arch=" + ARCH, "-shared", "-fPIC", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed:\n%s\n%s" % (" ".join(cmd), r.stderr))
    os.replace(tmp, lib)
    if verbose:
        print("built", lib)
    return lib


if __name__ == "__main__":
    build(verbose=True)
    if "--stamps" in sys.argv[1:]:
        build(verbose=True, stamps=True)
    sys.exit(0)
