"""Build the Sol-Attn HIP library (libsolattn.so) in-tree for gfx950.

Usage: python -m free_block_sparse_mean_amd.build   (or build() from Python)
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
LIB = os.path.join(PKG, "libsolattn.so")
SOURCES = ["api.cpp", "prepass.hip", "fused.hip", "route.hip", "noalloc.hip"]
# the tile loop's issue-rate microbenchmark (bench.py --tile-mix), not part of libsolattn.so
MIX_LIB = os.path.join(PKG, "libsoltilemix.so")
MIX_SOURCE = "tile_mix.hip"

HIPCC_FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
    "-Wall", "-Wno-unused-command-line-argument",
    # no packed-fp32 instructions in device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # MFMA accumulators in VGPRs: the online-softmax rescale and the epilogue
    # then touch them without accvgpr moves
    "-mllvm", "-amdgpu-mfma-vgpr-form=1",
]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm toolchain required to build libsolattn.so)")


# The bf16 per-row-correction kernels: fused.hip once more, alone in a
# translation unit built with the max-ILP scheduler (their register demand then
# fits without spills; the other kernels are faster under the default one).
ROW_TU_FLAGS = ["-DSOL_FUSED_ROW_TU", "-mllvm", "-amdgpu-sched-strategy=max-ilp"]


def _run(cmd, verbose: bool) -> None:
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    out = "\n".join(l for l in (r.stdout + r.stderr).splitlines()
                    if "packed-fp32-ops" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed ({r.returncode}):\n{out}")
    if out.strip() and verbose:
        print(out, file=sys.stderr)


def build(verbose: bool = False) -> str:
    """Compile every source into libsolattn.so next to this file; returns its path."""
    tmp = LIB + ".tmp"
    row_obj = os.path.join(PKG, "fused_row.tmp.o")
    inc = ["-I", os.path.join(ROOT, "include")]
    obj_flags = [f for f in HIPCC_FLAGS if f != "-shared"]
    try:
        _run([hipcc(), *obj_flags, *ROW_TU_FLAGS, *inc, "-c", os.path.join(CSRC, "fused.hip"), "-o", row_obj],
             verbose)
        _run([hipcc(), *HIPCC_FLAGS, *inc, *[os.path.join(CSRC, s) for s in SOURCES], "-x", "none", row_obj, "-o", tmp], verbose)
    finally:
        if os.path.exists(row_obj):
            os.remove(row_obj)
    os.replace(tmp, LIB)
    build_tile_mix(verbose)
    return LIB


def build_tile_mix(verbose: bool = False) -> str:
    """Compile the tile-loop microbenchmark into libsoltilemix.so; returns its path."""
    tmp = MIX_LIB + ".tmp"
    _run([hipcc(), *HIPCC_FLAGS, os.path.join(CSRC, MIX_SOURCE), "-o", tmp], verbose)   # the library's flags
    os.replace(tmp, MIX_LIB)
    return MIX_LIB


if __name__ == "__main__":
    print(build(verbose=True))
