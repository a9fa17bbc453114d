"""Compile libgka.so (the HIP kernels and the C ABI) for gfx950 with hipcc, in-tree.

Usage: python -m test_ridge_regression_amd.build  (or call build_library()).
Objects go to _build/ at the repository root; the library is written next to this file.
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
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libgka.so")
SOURCES = ["gka_api.cpp", "gka_step.hip", "gka_fwd.hip", "gka_walk_tok.hip", "gka_summary.hip",
           "gka_bwd.hip", "gka_bwd_tok.hip", "gka_noalloc.hip"]

HIPCC = os.environ.get("HIPCC", shutil.which("hipcc") or "/opt/rocm/bin/hipcc")
FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
    # packed fp32 arithmetic stays off: the compiler emits only scalar fp32 VALU forms
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I" + os.path.join(ROOT, "include"),
]


# Per-source flags. The token-owning kernels (the walk, the summaries, the backward) keep matrix-core results in vector registers (its
# products feed vector arithmetic directly); its resident operands are placed in the accumulator
# registers by the kernel itself.
EXTRA = {"gka_walk_tok.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"],
         "gka_summary.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"],
         "gka_bwd_tok.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"]}


def _compile(src: str, verbose: bool) -> str:
    obj = os.path.join(BUILD, os.path.basename(src) + ".o")
    cmd = [HIPCC, "-x", "hip", *FLAGS, *EXTRA.get(src, []), "-c", os.path.join(CSRC, src), "-o", obj]
    if verbose:
        cmd.insert(1, "-Rpass-analysis=kernel-resource-usage")
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stderr}")
    if verbose:
        sys.stderr.write(r.stderr)
    return obj


def build_library(verbose: bool = False) -> str:
    """Compile every source and link libgka.so; returns the library path."""
    os.makedirs(BUILD, exist_ok=True)
    with concurrent.futures.ThreadPoolExecutor(max_workers=len(SOURCES)) as ex:
        objs = list(ex.map(lambda s: _compile(s, verbose), SOURCES))
    tmp = LIB + ".tmp"
    cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build_library(verbose="-v" in sys.argv))
