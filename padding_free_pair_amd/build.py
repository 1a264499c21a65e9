"""Compile the gfx950 library libntpair.so in-tree with hipcc.

Usage: python -m padding_free_pair_amd.build   (or build() from Python)
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libntpair.so")
ARCH = "gfx950"


def _hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    return "hipcc"


COMMON = [
    f"--offload-arch={ARCH}", "-O3", "-fPIC", "-std=c++17", "-Wall",
    f"-I{INCLUDE}", f"-I{CSRC}",
    # keep the compiler from forming packed fp32 ops (v_pk_*_f32)
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # "#pragma unroll" loops are meant to unroll fully, however long the body
    "-mllvm", "-pragma-unroll-threshold=1000000",
]


# Per-file flags: matrix-core accumulators in ordinary VGPRs.
# - The weight-stationary transition keeps both weights in the accumulation
#   registers (AGPRs) as product operands.
# - The recomputing weight gradient masks its recomputed products with VALU
#   work; in the AGPR form the compiler also moved its long-lived
#   accumulators between AGPRs and VGPRs every 64-cell block (192 moves per
#   64 products).
# - The fused SwiGLU gradient reads every chunk's three results in VALU
#   work (its x and G operands are placed in AGPRs instead).
FILE_FLAGS = {
    "nt_transition_ws.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"],
    "nt_wgrad.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"],
    "nt_swiglu_bwd32.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"],
}


def sources():
    return sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC)
                  if f.endswith(".hip") or f.endswith(".cpp"))


def _compile(src: str) -> str:
    obj = os.path.join(BUILD, os.path.basename(src) + ".o")
    lang = ["-x", "hip"] if src.endswith(".hip") else []
    extra = FILE_FLAGS.get(os.path.basename(src), [])
    cmd = [_hipcc(), *COMMON, *extra, *lang, "-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    noise = "is not a recognized feature for this target"
    err = "\n".join(l for l in (r.stderr or "").splitlines() if noise not in l)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{err}")
    if err.strip():
        sys.stderr.write(err + "\n")
    return obj


def build(verbose: bool = True) -> str:
    """Compile every source and link libntpair.so; returns its path."""
    os.makedirs(BUILD, exist_ok=True)
    srcs = sources()
    workers = min(len(srcs), max(1, min(8, os.cpu_count() or 1)))
    with cf.ThreadPoolExecutor(workers) as ex:
        objs = list(ex.map(_compile, srcs))
    tmp = LIB + ".tmp"
    cmd = [_hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB}")
    return LIB


if __name__ == "__main__":
    build()
