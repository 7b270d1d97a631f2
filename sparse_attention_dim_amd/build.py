"""Build librtp.so (the gfx950 HIP kernels and the C ABI) in-tree with hipcc."""
from __future__ import annotations

import concurrent.futures as cf
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
OBJ = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "librtp.so")
SOURCES = ["abi.cpp", "append.hip", "select.hip", "select_chunk.hip", "attn_decode.hip", "attn_prefill.hip", "attn_sparse_prefill.hip"]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
# Per-file code generation options.  The chunk selection, the decode window
# kernel and the prefill attention tiles keep their MFMA results in VGPRs:
# they read (or rescale) every accumulator lane with VALU, and AGPR results
# would cost a v_accvgpr move for each (and, for the tiles, a second wave per
# SIMD).
FILE_FLAGS = {"select_chunk.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form=1"],
              "attn_decode.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form=1"],
              "attn_prefill.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form=1"],
              "attn_sparse_prefill.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form=1"]}
FLAGS = ["--offload-arch=gfx950", "-O3", "-fPIC", "-std=c++17", "-Wall",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]


def _compile(src: str) -> str:
    out = os.path.join(OBJ, os.path.splitext(src)[0] + ".o")
    cmd = [HIPCC, *FLAGS, *FILE_FLAGS.get(src, []), "-x", "hip", "-c", os.path.join(CSRC, src), "-o", out]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("hipcc failed for %s:\n%s" % (src, r.stderr))
    return out


def build(verbose: bool = False) -> str:
    os.makedirs(OBJ, exist_ok=True)
    with cf.ThreadPoolExecutor(max_workers=min(8, len(SOURCES))) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = LIB + ".tmp%d" % os.getpid()
    subprocess.check_call([HIPCC, "--offload-arch=gfx950", "-shared", "-o", tmp, *objs])
    os.replace(tmp, LIB)
    if verbose:
        print("built", LIB)
    return LIB


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
