"""Builds libnvfp4.so (the C-ABI library) from csrc/ with hipcc for gfx950.

Usage: python -m bit_block_scaled_bf16_amd.build   (or build() from Python)

Objects go to _build/ at the repository root; the library is written next to
this file so that it travels with the source tree.
"""

from __future__ import annotations

import concurrent.futures
import os
import shutil
import subprocess
import sys

PKG_DIR = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG_DIR)
CSRC = os.path.join(PKG_DIR, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD_DIR = os.path.join(ROOT, "_build")
LIB_NAME = "libnvfp4.so"
LIB_PATH = os.path.join(PKG_DIR, LIB_NAME)

SOURCES = ["abi.cpp", "quantize.hip", "dequant.hip", "gemm.hip", "mxfp4.hip", "fp8.hip", "f8f6f4_gemm.hip", "noalloc.hip",
           "stream.hip"]

# -ffp-contract=off: the quantizer's float32 steps are single roundings each
#   (no fused multiply-add), as the format definition requires.
# -packed-fp32-ops disabled: no packed float32 instructions are generated.
COMMON_FLAGS = [
    "-O3",
    "-std=c++17",
    "-fPIC",
    "--offload-arch=gfx950",
    "-ffp-contract=off",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall",
    "-I", INCLUDE,
    "-I", CSRC,
]


def _hipcc() -> str:
    for cand in (shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found; the NVFP4 library needs ROCm's hipcc")


def _compile(src: str) -> str:
    obj = os.path.join(BUILD_DIR, os.path.splitext(src)[0] + ".o")
    cmd = [_hipcc(), *COMMON_FLAGS, "-c", os.path.join(CSRC, src), "-o", obj]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{res.stdout}\n{res.stderr}")
    return obj


def build(verbose: bool = False) -> str:
    """Compiles every source and links libnvfp4.so; returns its path."""
    os.makedirs(BUILD_DIR, exist_ok=True)
    with concurrent.futures.ThreadPoolExecutor(max_workers=min(8, len(SOURCES))) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = LIB_PATH + ".tmp"
    cmd = [_hipcc(), "-shared", "-fPIC", "--offload-arch=gfx950", *objs, "-o", tmp]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"link failed:\n{res.stdout}\n{res.stderr}")
    os.replace(tmp, LIB_PATH)
    if verbose:
        print(f"built {LIB_PATH}")
    return LIB_PATH


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
