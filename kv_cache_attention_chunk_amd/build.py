"""Build libchunkattn.so (the C-ABI HIP library) in-tree for gfx950 with hipcc.

Each source under csrc/ is compiled to an object in parallel, then linked.
The library lands next to this file; the Python binding loads it from there.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libchunkattn.so")
# roof probes timed by the benchmark (bf16 MFMA peak, HBM read), kept out of
# the chunk-attention library
ROOFS_SRC = "roofs.hip"
ROOFS_LIB = os.path.join(PKG, "libchunkattn_roofs.so")
SOURCES = ["attn_fwd.hip", "pbsa.hip", "select.hip", "merge.hip", "pack.hip", "mla.hip",
           "api.hip"]
ARCH = "gfx950"

# Packed-FP32 instructions are disabled for all device code (ordinary float
# code is compiled to scalar VALU ops instead).
FLAGS = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-I", INCLUDE, "-I", CSRC, "-Wall", "-Wno-unused-function"]


def hipcc() -> str:
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found")


def _compile(src: str, extra) -> str:
    obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
    cmd = [hipcc(), *FLAGS, *extra, "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    return obj


def _link(objs, out):
    tmp = out + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, out)


def build(extra_flags=(), verbose: bool = False) -> str:
    """Compile every HIP source and link libchunkattn.so (and the
    benchmark's roof probes, libchunkattn_roofs.so); returns the main
    library's path."""
    os.makedirs(BUILD, exist_ok=True)
    srcs = SOURCES + [ROOFS_SRC]
    with cf.ThreadPoolExecutor(max_workers=len(srcs)) as ex:
        objs = list(ex.map(lambda s: _compile(s, list(extra_flags)), srcs))
    _link(objs[:len(SOURCES)], LIB)
    _link(objs[len(SOURCES):], ROOFS_LIB)
    if verbose:
        print(f"built {LIB} and {ROOFS_LIB}")
    return LIB


if __name__ == "__main__":
    build(verbose=True)
