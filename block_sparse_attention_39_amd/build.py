"""Build libbsa.so in-tree with hipcc for gfx950.

    python block_sparse_attention_39_amd/build.py

Every translation unit is compiled with hipcc (-O3, --offload-arch=gfx950) and
with packed FP32 instructions disabled; the objects go to ``_build/`` and the
shared library next to this file.
"""
from __future__ import annotations

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libbsa.so")
SOURCES = ["bsa_api.cpp", "permute.hip", "shape.hip", "plan.hip", "forward.hip", "backward.hip"]
ARCH = os.environ.get("BSA_OFFLOAD_ARCH", "gfx950")

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
CFLAGS = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}", "-I", INCLUDE, "-I", CSRC,
          "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
          # keep per-thread arrays in registers: LDS is budgeted by hand
          "-mllvm", "-disable-promote-alloca-to-lds",
          "-Wall", "-Wno-unused-result"]
# per-file additions: the attention kernel keeps its MFMA accumulators in
# ordinary VGPRs (its softmax rescales them with vector instructions, and the
# accumulation registers then hold the operand fragments)
EXTRA = {"forward.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"], "backward.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"]}


def _compile(src: str) -> str:
    obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
    cmd = [HIPCC, *CFLAGS, *EXTRA.get(src, []), "-x", "hip", "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{r.stderr}")
    return obj


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    with ThreadPoolExecutor(len(SOURCES)) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = LIB + ".tmp"
    cmd = [HIPCC, "-shared", "-fPIC", f"--offload-arch={ARCH}", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    os.replace(tmp, LIB)
    if verbose:
        print("built", LIB)
    return LIB


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
