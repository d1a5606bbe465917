"""Build libsplitkv.so in-tree with hipcc for gfx950.

Usage: ``python -m split_kv_exact_amd.build`` (or ``__graft_entry__.build()``).
Objects go to ``_build/`` at the repository root; the library is written next to
this file and replaced atomically, so a process that already loaded it is unaffected.
"""

from __future__ import annotations

import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libsplitkv.so")

SOURCES = ["abi.cpp", "plan.cpp", "partial_bf16.hip", "partial_mma.hip", "partial_f32.hip", "merge.hip",
           "backward_bf16.hip", "scratch.hip"]

ARCH = "gfx950"
COMMON = [
    f"--offload-arch={ARCH}",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-Wall",
    "-Wno-unused-function",
    f"-I{INCLUDE}",
    f"-I{CSRC}",
    # Packed fp32 VALU instructions are kept out of the device code.
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]


# Per-source extra flags. The bf16 partial kernel produces no NaN from finite inputs
# (every -inf - -inf is guarded), so its row max needs no NaN quieting.
EXTRA = {"partial_bf16.hip": ["-fno-honor-nans", "-mllvm", "-amdgpu-atomic-optimizer-strategy=None"],
         "partial_mma.hip": ["-fno-honor-nans"]}


def _hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build libsplitkv)")


def _run(cmd):
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    out = "\n".join(line for line in r.stdout.splitlines() if "packed-fp32-ops" not in line)
    if r.returncode != 0:
        raise RuntimeError(f"command failed ({r.returncode}): {' '.join(cmd)}\n{out}")
    return out


def build(verbose: bool = False) -> str:
    """Compile every source and link libsplitkv.so; returns its path."""
    hipcc = _hipcc()
    os.makedirs(BUILD, exist_ok=True)
    jobs = []
    for src in SOURCES:
        obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
        lang = ["-x", "hip"] if src.endswith(".hip") else []
        extra = EXTRA.get(src, [])
        jobs.append((obj, [hipcc, *COMMON, *extra, *lang, "-c", os.path.join(CSRC, src), "-o", obj]))
    workers = min(len(jobs), int(os.environ.get("MAX_JOBS", "8")), 16)
    with ThreadPoolExecutor(max_workers=max(1, workers)) as ex:
        outs = list(ex.map(lambda j: _run(j[1]), jobs))
    if verbose:
        for (obj, cmd), out in zip(jobs, outs):
            print(" ".join(cmd))
            if out.strip():
                print(out)
    tmp = LIB + f".tmp{os.getpid()}"
    _run([hipcc, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *[j[0] for j in jobs]])
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
