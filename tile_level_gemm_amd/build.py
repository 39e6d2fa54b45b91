"""Build libtilegemm.so in-tree with hipcc for gfx950.

    python -m tile_level_gemm_amd.build

Objects go to tile_level_gemm_amd/_build/ (git-ignored); the library lands next to
this file so that it travels with the source tree.
"""

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
BUILD = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libtilegemm.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

SOURCES = ["abi.cpp", "plan.cpp", "copy_kernels.hip", "gemm_kernels.hip", "gemm_direct.hip",
           "gemm_direct_kk.hip", "gemm_direct_km.hip", "gemm_direct_mk.hip", "gemm_direct_mm.hip",
           "gemm_fp8.hip", "gemm_fp8_km.hip", "gemm_fp8_mk.hip", "gemm_fp8_mm.hip",
           "gemm_mx_kk.hip", "gemm_mx_km.hip", "gemm_mx_mk.hip", "gemm_mx_mm.hip", "gemm_mx_packed.hip", "gemm_mx_fp4.hip", "gemm_mx_fp6.hip",
           "frag.cpp", "frag_kernels.hip", "async_copy.hip"]

# -packed-fp32-ops: no v_pk_*_f32 in generated code (the device pass honours it; the
# host pass warns that it does not know the feature).
FLAGS = ["--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-mcode-object-version=5",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-Wall", "-Wno-unused-function", "-I", os.path.join(HERE, "..", "include")]


def _compile(src):
    path = os.path.join(CSRC, src)
    obj = os.path.join(BUILD, src + ".o")
    lang = ["-x", "hip"] if src.endswith(".hip") else []
    cmd = [HIPCC] + FLAGS + lang + ["-c", path, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    err = "\n".join(l for l in r.stderr.splitlines() if "packed-fp32-ops" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{err}")
    if err.strip():
        sys.stderr.write(err + "\n")
    return obj


def build(jobs=8):
    """Compile every source and link libtilegemm.so; returns the library path."""
    os.makedirs(BUILD, exist_ok=True)
    with ThreadPoolExecutor(max_workers=jobs) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = LIB + ".tmp"
    cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp] + objs
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build())
