"""Build libatlas.so (HIP for gfx950) in-tree with hipcc.

Every ``.hip`` file under ``csrc/`` is compiled for gfx950 only, plus the
host-side ABI layer ``csrc/abi.cpp``; the objects are linked into
``windowed_global_local_amd/libatlas.so``.  Packed-fp32 instruction selection
is disabled for device code (the flag is a device target feature; the host
pass warns that it does not know it, which is harmless).  The forward
attention keeps MFMA results in VGPRs; the backward kernels hold larger
accumulator sets and leave them to the compiler (AGPRs).
"""
from __future__ import annotations

import glob
import os
import shutil
import subprocess
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libatlas.so")
BUILD_DIR = os.path.join(ROOT, "_build")
ARCH = "gfx950"

COMMON = ["-O3", "-std=c++17", "-fPIC", "-Wall", f"-I{INCLUDE}", f"-I{CSRC}"]
DEVICE = [f"--offload-arch={ARCH}", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]
# forward attention: MFMA results in VGPRs, since the softmax reads every S^T
# accumulator with VALU ops and AGPR-form accumulators would need a
# v_accvgpr_read per element per tile
PER_FILE = {"hier_attn.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"]}


def hipcc() -> str:
    for cand in (shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm toolchain required to build libatlas.so)")


def _compile(src: str) -> str:
    os.makedirs(BUILD_DIR, exist_ok=True)
    obj = os.path.join(BUILD_DIR, os.path.basename(src) + ".o")
    extra = PER_FILE.get(os.path.basename(src), [])
    cmd = [hipcc()] + COMMON + (DEVICE if src.endswith(".hip") else []) + extra + ["-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"compile failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    return obj


def build(verbose: bool = False) -> str:
    srcs = sorted(glob.glob(os.path.join(CSRC, "*.hip"))) + [os.path.join(CSRC, "abi.cpp")]
    with ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        objs = list(ex.map(_compile, srcs))
    tmp = LIB + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp] + objs
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB}")
    return LIB


if __name__ == "__main__":
    build(verbose=True)
