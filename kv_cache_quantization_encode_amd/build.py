"""Build libturbokv.so in-tree with hipcc for gfx950.

Usage: python -m kv_cache_quantization_encode_amd.build  (or call build()).
Each source compiles to an object under csrc/_build/, then one shared
library is linked next to this file.  Always recompiles (a full build takes
well under a minute).
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
BUILD = os.path.join(CSRC, "_build")
LIB = os.path.join(HERE, "libturbokv.so")
SOURCES = ["attn.hip", "attn_fused.hip", "attn_fused4.hip", "attn_generic.hip", "attn_prefill.hip", "encode.hip", "tables.cpp", "api.cpp", "dequant.hip", "minmax.hip",
           "scratch.hip"]

# -packed-fp32-ops keeps the compiler from emitting packed fp32 (v_pk_*_f32)
# instructions; hipcc's host pass reports the feature as unknown, harmlessly.
# -amdgpu-mfma-vgpr-form lets MFMA results land in ordinary VGPRs (no
# accumulator-register copies before the VALU uses them).
COMMON = ["-O3", "-std=c++17", "-fPIC", "--offload-arch=gfx950",
          "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
          "-mllvm", "-amdgpu-mfma-vgpr-form",
          "-Wall", "-Werror=shadow", "-Werror=uninitialized", "-Wno-unused-function",
          "-I" + os.path.join(HERE, "..", "include")]


def _hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found: the HIP toolchain is required to build libturbokv")


def _compile(src: str) -> str:
    obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
    cmd = [_hipcc(), *COMMON, "-c", os.path.join(CSRC, src), "-o", obj]
    if src.endswith(".cpp"):
        cmd[1:1] = ["-x", "hip"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"compile failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    return obj


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    with cf.ThreadPoolExecutor(max_workers=min(len(SOURCES), 8)) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = LIB + ".tmp"
    cmd = [_hipcc(), "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, LIB)
    if verbose:
        print("built", LIB)
    return LIB


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
