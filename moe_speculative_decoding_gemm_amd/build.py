"""Build libacceptmoe.so for gfx950 with hipcc, in-tree.

    python moe_speculative_decoding_gemm_amd/build.py [--jobs N]

(run it as a script: importing the package first would load the library
that is about to be rebuilt).

Objects go to ``_build/`` at the repository root; the shared library lands
next to this file.  hipcc cross-compiles gfx950 code without a GPU.
"""

from __future__ import annotations

import argparse
import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libacceptmoe.so")
ARCH = "gfx950"

SOURCES = ["select.hip", "permute.hip", "grouped.hip", "gemm.hip", "capi.cpp", "noalloc.hip"]

# -packed-fp32-ops off: hipcc would otherwise emit packed fp32 adds/multiplies
# on its own; the device code here is written for the unpacked forms.
CFLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-Wall",
    "-Wno-unused-function", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", INCLUDE, "-I", CSRC,
]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build the HIP library)")


def _compile(src: str) -> str:
    obj = os.path.join(BUILD, os.path.basename(src) + ".o")
    cmd = [hipcc(), *CFLAGS, "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    msgs = "\n".join(line for line in (r.stdout + r.stderr).splitlines()
                     if "packed-fp32-ops" not in line)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{msgs}")
    if msgs.strip():
        sys.stderr.write(msgs + "\n")
    return obj


def build(jobs: int = 4, verbose: bool = False) -> str:
    """Compile every source and link the shared library; returns its path."""
    os.makedirs(BUILD, exist_ok=True)
    with cf.ThreadPoolExecutor(max_workers=max(1, jobs)) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = LIB + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}{r.stderr}")
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB}")
    return LIB


if __name__ == "__main__":
    ap = argparse.ArgumentParser()
    ap.add_argument("--jobs", type=int, default=4)
    args = ap.parse_args()
    build(args.jobs, verbose=True)
