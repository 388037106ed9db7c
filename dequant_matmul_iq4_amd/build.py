"""Compile the HIP sources of the library into ``libiq4.so`` (gfx950), in-tree.

Run as ``python -m dequant_matmul_iq4_amd.build``; ``__graft_entry__.build()`` calls
``build()``.  Every source is compiled each time (objects are written to ``_build/``).
"""
from __future__ import annotations

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
OUT = os.path.join(PKG, "libiq4.so")
OBJ = os.path.join(ROOT, "_build")

SOURCES = ["api.hip", "format.hip", "qmv.hip", "route.hip", "gemm.hip", "moe.hip", "xs.hip"]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"
FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    # results must not depend on how the compiler contracts a*b+c: every FMA is explicit
    "-ffp-contract=off",
    "-fhip-fp32-correctly-rounded-divide-sqrt",
    # no packed-fp32 instructions anywhere
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function",
    "-I", os.path.join(ROOT, "include"),
]


def _compile(src: str) -> str:
    obj = os.path.join(OBJ, os.path.splitext(src)[0] + ".o")
    cmd = [HIPCC, *FLAGS, "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{r.stdout}\n{r.stderr}")
    err = "\n".join(l for l in r.stderr.splitlines() if "packed-fp32-ops" not in l)
    if err.strip():
        print(err, file=sys.stderr)
    return obj


# The benchmark's reference kernels (streaming read, pure matrix-core loop), a library of
# their own: the product library never loads them.
CEIL_SOURCES = ["ceilings.hip"]
CEIL_OUT = os.path.join(PKG, "libiq4_ceilings.so")


def _link(objs, out):
    tmp = out + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, out)


def build(verbose: bool = True) -> str:
    os.makedirs(OBJ, exist_ok=True)
    with ThreadPoolExecutor(min(8, len(SOURCES) + len(CEIL_SOURCES))) as ex:
        objs = list(ex.map(_compile, SOURCES + CEIL_SOURCES))
    _link(objs[:len(SOURCES)], OUT)
    _link(objs[len(SOURCES):], CEIL_OUT)
    if verbose:
        print(f"built {OUT} and {CEIL_OUT}")
    return OUT


if __name__ == "__main__":
    build()
