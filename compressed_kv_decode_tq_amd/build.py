"""Build libtq.so (HIP kernels + C ABI) in-tree for gfx950 with hipcc.

Usage: python -m compressed_kv_decode_tq_amd.build
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libtq.so")
BUILD_DIR = os.path.join(PKG, "_build")

SOURCES = ["tq_api.cpp", "tq_codebook.cpp", "tq_plan.cpp", "tq_encode.hip", "tq_decode.hip", "tq_decode_mfma.hip", "tq_noalloc.hip"]
ARCH = os.environ.get("TQ_OFFLOAD_ARCH", "gfx950")
# MFMA results land in ordinary VGPRs in the decode scan (no accumulator-register
# copies: every result is consumed by VALU code right away).  The decode scan
# also runs with the IEEE mode bit clear and no NaN operands assumed: its
# maxima then need no quieting of their inputs, so a DPP row move folds into
# the max (the file's kernels read their indices through the hardware
# builtins, so no device-library call is left behind by the mode change).
SOURCE_FLAGS = {"tq_decode_mfma.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form", "-mno-amdgpu-ieee", "-fno-honor-nans"]}


def _hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build libtq)")


def _flags() -> list[str]:
    return [
        f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", f"-I{INCLUDE}", f"-I{CSRC}",
        # packed fp32 instructions are disabled on purpose: plain fp32 code only
        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
        "-Wall", "-Wno-unused-function", "-Wno-unused-variable",
    ]


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD_DIR, exist_ok=True)
    cc = _hipcc()
    objs = []

    def compile_one(src: str) -> str:
        obj = os.path.join(BUILD_DIR, os.path.splitext(src)[0] + ".o")
        lang = ["-x", "hip"] if src.endswith(".hip") else []
        cmd = [cc, *_flags(), *SOURCE_FLAGS.get(src, []), *lang, "-c", os.path.join(CSRC, src), "-o", obj]
        res = subprocess.run(cmd, capture_output=True, text=True)
        msgs = "\n".join(l for l in (res.stdout + res.stderr).splitlines()
                         if "packed-fp32-ops" not in l)
        if res.returncode != 0:
            raise RuntimeError(f"hipcc failed for {src}:\n{msgs}")
        if verbose and msgs.strip():
            print(msgs, file=sys.stderr)
        return obj

    with cf.ThreadPoolExecutor(len(SOURCES)) as ex:
        objs = list(ex.map(compile_one, SOURCES))
    tmp = LIB + ".tmp"
    cmd = [cc, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError("link failed:\n" + res.stdout + res.stderr)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
