"""Build libsparda.so (all HIP sources, gfx950) in-tree.

    python -m kv_block_selection_amd.build

Compiles every csrc/*.hip and csrc/*.cpp to an object under _build/ with hipcc
(in parallel), then links kv_block_selection_amd/libsparda.so.
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
BUILD = os.path.join(ROOT, "_build", "sparda")
LIB = os.path.join(PKG, "libsparda.so")

ARCH = "gfx950"
# Packed fp32 VALU ops are kept out of every kernel (the compiler must not form them).
DEVICE_FLAGS = ["-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]
COMMON = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}", "-fvisibility=hidden",
          "-I", INCLUDE, "-I", CSRC, "-Wall", "-Wno-unused-function"]
# Per-source extras. Prefill attention keeps its matrix-core accumulators in
# VGPRs (it normalises them on the vector ALUs); left to itself the register
# allocator fills the AGPRs as well and spills.
FILE_FLAGS = {
    "attn_prefill.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form=1"],
    # window maxima of matrix-core results: no NaN quieting before each max
    "select_prefill.hip": ["-fno-honor-nans"],
    # products stay in VGPRs for the softmax arithmetic that follows them, and
    # no NaN quieting before each max
    "mhsel_prefill.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form=1", "-fno-honor-nans"],
}


def hipcc() -> str:
    path = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(path):
        raise RuntimeError("hipcc not found; ROCm is required to build libsparda.so")
    return path


def sources():
    return sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith((".hip", ".cpp")))


def _compile(src: str) -> str:
    obj = os.path.join(BUILD, os.path.basename(src) + ".o")
    cmd = [hipcc(), *COMMON, *DEVICE_FLAGS, *FILE_FLAGS.get(os.path.basename(src), []), "-c", src, "-o", obj]
    if src.endswith(".cpp"):
        cmd[1:1] = ["-x", "hip"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{r.stderr}")
    return obj


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    srcs = sources()
    with cf.ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        objs = list(ex.map(_compile, srcs))
    tmp = LIB + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB} from {len(srcs)} sources")
    return LIB


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
