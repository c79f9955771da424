"""Build ``libgla.so`` (the C-ABI HIP library) in-tree with hipcc for gfx950.

Usage: ``python -m gated_linear_attention_fwd_amd.build`` (or ``build_library()``).
Each source is compiled in parallel to ``_build/*.o`` and linked next to this
file, where the Python binding loads it.
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
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libgla.so")
ARCH = "gfx950"

SOURCES = ["gla_api.cpp", "anchor.hip", "carry.hip", "valu.hip", "mfma.hip", "bwd.hip", "bwd_mfma.hip", "gdn.hip", "gdn_mfma.hip", "noalloc.hip", "probe.hip"]

# Packed fp32 arithmetic is switched off for the device code (the compiler then
# emits plain v_fma_f32 / v_add_f32 / v_mul_f32).
DEVICE_FLAGS = ["-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]
COMMON = ["-O3", "-std=c++17", "-fPIC", "-fvisibility=hidden", "-Wall",
          "--offload-arch=" + ARCH, "-I" + os.path.join(ROOT, "include")]
# Per-source additions. The softmax kernels run with the IEEE mode bit off and
# no NaN handling (their inputs are finite by precondition): the running max is
# then a single v_max_f32 per score instead of two (NaN canonicalisation), and
# the MFMA accumulators, which the softmax reads and rescales every block, stay
# in ordinary VGPRs rather than moving through AGPRs.
# The kv kernels scale their MFMA accumulators in place at d = 128 (the
# running state of a frame group): with the accumulators in VGPRs that is plain
# vector work; in AGPRs it would copy them through VGPRs (229 registers, 2
# waves per SIMD, against 165 and 3). Measured neutral for the other kernels of
# the file.
EXTRA_FLAGS = {"anchor.hip": ["-mno-amdgpu-ieee", "-fno-honor-nans",
                              "-mllvm", "-amdgpu-mfma-vgpr-form"],
               "mfma.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"]}


def hipcc() -> str:
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found (ROCm is required to build libgla.so)")


def _compile(src: str) -> str:
    obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
    cmd = [hipcc(), *COMMON, *DEVICE_FLAGS, *EXTRA_FLAGS.get(src, []), "-c",
           os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("compiling %s failed:\n%s\n%s" % (src, " ".join(cmd), r.stderr))
    return obj


def build_library(verbose: bool = False) -> str:
    """Compile every HIP/C++ source for gfx950 and link libgla.so; returns its path."""
    os.makedirs(BUILD, exist_ok=True)
    with cf.ThreadPoolExecutor(max_workers=min(8, len(SOURCES))) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = LIB + ".tmp%d" % os.getpid()
    cmd = [hipcc(), "-shared", "-fPIC", "--offload-arch=" + ARCH, *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("linking libgla.so failed:\n%s\n%s" % (" ".join(cmd), r.stderr))
    os.replace(tmp, LIB)
    if verbose:
        print("built", LIB)
    return LIB


if __name__ == "__main__":
    build_library(verbose=True)
    sys.exit(0)
