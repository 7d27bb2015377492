"""Build ``libbqmm.so`` in-tree with hipcc for gfx950.

Every HIP source is compiled on its own (in parallel) and linked into one
shared library next to this file.  Flags:
  -ffp-contract=off   floating-point contraction only where a kernel writes
                      an explicit fma, so results do not depend on inlining;
  -packed-fp32-ops    removed from the target features: no packed f32 VALU;
  -amdgpu-mfma-vgpr-form=1 (MMQ only)
                      MFMA sources and results in ordinary VGPRs, so the
                      VALU fold reads the int32 block sums without copies.
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
BUILD_DIR = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libbqmm.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"

SOURCES = ["q8_1_quantize.hip", "q8_0_gemv.hip", "q8_0_gemv_mma.hip", "q8_0_gemm.hip", "e4m3.hip", "e4m3_exact.hip", "e4m3_gemv.hip", "f16_mirror.hip", "e4m3_blk.hip", "strerror.cpp"]

HIPFLAGS = [
    f"--offload-arch={ARCH}",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-ffp-contract=off",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", INCLUDE,
    "-I", CSRC,
]
# Per-source extra flags.  The MMQ folds each MFMA result on the VALU, so its
# MFMAs write ordinary VGPRs; the e4m3 GEMM keeps its large accumulator tiles
# in AGPRs (the default form).
EXTRA = {
    "q8_0_gemm.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form=1"],
    "q8_0_gemv_mma.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form=1"],
    "e4m3_exact.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form=1"],
    "e4m3_blk.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form=1"],
}


def _compile(src: str) -> str:
    obj = os.path.join(BUILD_DIR, os.path.splitext(src)[0] + ".o")
    cmd = [HIPCC, *HIPFLAGS, *EXTRA.get(src, []), "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stdout}\n{r.stderr}")
    return obj


def build(verbose: bool = False) -> str:
    """Compile every source and link ``libbqmm.so``; returns its path."""
    os.makedirs(BUILD_DIR, exist_ok=True)
    with cf.ThreadPoolExecutor(max_workers=min(len(SOURCES), os.cpu_count() or 4)) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = LIB + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB}")
    return LIB


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
