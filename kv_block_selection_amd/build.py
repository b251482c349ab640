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


# Host-side AddressSanitizer + UndefinedBehaviorSanitizer build of the ABI layer
# (argument validation, workspace sizing, messages), for a CPU test: api.cpp is
# compiled with host instrumentation only (each -fsanitize= behind -Xarch_host;
# device code is untouched) and linked with the regular build's other objects.
# Load it with the sanitizer runtime preloaded (sanitizer_runtime()).
SAN_BUILD = os.path.join(ROOT, "_build", "host_sanitized")
SAN_LIB = os.path.join(SAN_BUILD, "libsparda_host_sanitized.so")
HOST_SAN_FLAGS = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
                  "-Xarch_host", "-fno-sanitize-recover=undefined", "-Xarch_host", "-fno-omit-frame-pointer",
                  "-shared-libasan"]


def sanitizer_runtime() -> str:
    r = subprocess.run([hipcc(), "-print-file-name=libclang_rt.asan-x86_64.so"], capture_output=True, text=True)
    path = r.stdout.strip()
    if r.returncode != 0 or not os.path.isabs(path) or not os.path.exists(path):
        raise RuntimeError("the ASan runtime of the ROCm clang was not found")
    return path


def build_host_sanitized() -> str:
    """libsparda with api.cpp built under host ASan + UBSan; needs build() first."""
    os.makedirs(SAN_BUILD, exist_ok=True)
    api = os.path.join(CSRC, "api.cpp")
    obj = os.path.join(SAN_BUILD, "api.cpp.o")
    cmd = [hipcc(), "-x", "hip", *COMMON, *DEVICE_FLAGS, *HOST_SAN_FLAGS, "-c", api, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {api}:\n{r.stderr}")
    others = [os.path.join(BUILD, os.path.basename(src) + ".o") for src in sources() if not src.endswith("api.cpp")]
    missing = [o for o in others if not os.path.exists(o)]
    if missing:
        raise RuntimeError(f"run build() first: missing {missing[0]}")
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", *HOST_SAN_FLAGS, "-o", SAN_LIB, obj, *others]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    return SAN_LIB


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
