"""Fill device (or, through a device bounce buffer, pinned host) tensors with the
seeded synthetic inputs, bit-identical to ``synth.generate``."""

from __future__ import annotations

import ctypes
import os
import shutil
import subprocess

import numpy as np

from . import Recipe, normal_table, stream_base

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libsynthfill.so")
SRC = os.path.join(HERE, "fill.hip")

_LIB = None
_TABLES = {}


def build() -> str:
    hipcc = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    tmp = LIB_PATH + ".tmp"
    cmd = [hipcc, "-O3", "-std=c++17", "-fPIC", "-shared", "--offload-arch=gfx950", "-ffp-contract=off",
           "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", SRC, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"building {SRC} failed:\n{r.stderr}")
    os.replace(tmp, LIB_PATH)
    return LIB_PATH


def _lib():
    global _LIB
    if _LIB is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is not built (synth.gpu.build())")
        lib = ctypes.CDLL(LIB_PATH)
        c = ctypes
        lib.synth_fill.restype = c.c_int
        lib.synth_fill.argtypes = [c.c_void_p, c.c_void_p, c.c_uint64, c.c_uint64, c.c_int, c.c_float, c.c_int,
                                   c.c_float, c.c_long, c.c_long, c.c_long, c.c_long, c.c_long, c.c_int, c.c_void_p]
        _LIB = lib
    return _LIB


def _table(device):
    import torch
    key = str(device)
    if key not in _TABLES:
        _TABLES[key] = torch.from_numpy(np.array(normal_table(), copy=True)).to(device)
    return _TABLES[key]


def fill_(t, recipe: Recipe, shape: tuple | None = None, start: int = 0) -> None:
    """Fill device tensor ``t`` with flat indices [start, start + t.numel()) of
    the tensor of logical ``shape`` (default: t.shape) drawn by ``recipe``."""
    import torch
    shape = tuple(t.shape) if shape is None else tuple(shape)
    want = torch.float32 if recipe.dtype == "fp32" else torch.bfloat16
    if t.dtype != want or not t.is_cuda or not t.is_contiguous():
        raise ValueError(f"fill_ needs a contiguous {want} GPU tensor")
    T, d = shape[-2], shape[-1]
    off_base = stream_base(recipe.seed, recipe.offset_tag) if recipe.offset_tag is not None else 0
    st = _lib().synth_fill(t.data_ptr(), _table(t.device).data_ptr(), stream_base(recipe.seed, recipe.tag), off_base,
                           int(recipe.scale is not None), float(recipe.scale or 0.0),
                           int(recipe.offset_tag is not None), float(recipe.offset_std), T, d, recipe.block, start,
                           t.numel(), int(recipe.dtype == "bf16"), torch.cuda.current_stream(t.device).cuda_stream)
    if st != 0:
        raise RuntimeError(f"synth_fill failed with status {st}")


def tensor(recipe: Recipe, shape: tuple, device="cuda"):
    import torch
    dt = torch.float32 if recipe.dtype == "fp32" else torch.bfloat16
    t = torch.empty(shape, dtype=dt, device=device)
    fill_(t, recipe)
    return t


def pinned_tensor(recipe: Recipe, shape: tuple, device="cuda", chunk_bytes: int = 1 << 30):
    """A pinned host tensor filled on the GPU chunk by chunk and copied down."""
    import torch
    dt = torch.float32 if recipe.dtype == "fp32" else torch.bfloat16
    host = torch.empty(shape, dtype=dt, pin_memory=True)
    flat = host.view(-1)
    per = max(1, chunk_bytes // host.element_size())
    buf = torch.empty(min(per, flat.numel()), dtype=dt, device=device)
    for s in range(0, flat.numel(), per):
        e = min(flat.numel(), s + per)
        b = buf[: e - s]
        fill_(b, recipe, shape, start=s)
        flat[s:e].copy_(b)
    torch.cuda.synchronize(device)
    return host
