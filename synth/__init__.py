"""Seeded, counter-based synthetic inputs for the block-selection hot path.

This module is shared by the GPU tests, the benchmark and the oracle's tests,
and it holds none of the method's arithmetic: it only produces the Q, K, V and
Forecast tensors (and their per-block offsets) that stand in for a model's
per-layer projections.

Definition (every value is a pure function of (seed, tag, flat index)):

* ``r = mix64(base + (i + 1) * GAMMA)`` with ``base = mix64((seed << 32) ^ tag)``
  -- the i-th output of a SplitMix64 generator (Steele, Lea and Flood,
  "Fast splittable pseudorandom number generators", OOPSLA 2014) whose state
  starts at ``base``. All arithmetic is modulo 2**64.
* A standard-normal draw takes the top 16 bits of ``r`` as an interval index
  ``j`` into a table of 65537 knots ``t[j] = Phi^-1((j + 0.5) / 65537)`` (fp64,
  rounded to fp32) and the next 16 bits as a fraction ``u = bits * 2**-16``;
  the value is ``t[j] + u * (t[j+1] - t[j])``, evaluated in fp32 with each
  operation rounded separately (no fused multiply-add). This is inverse-CDF
  sampling with a piecewise-linear quantile function: N(0,1) to well within
  bf16 resolution, truncated at +-4.32.
* Tensors are filled in row-major order of their logical shape; ``i`` is the
  flat index. Any affine recipe on top (a scale, a per-block offset) is done in
  fp32 with separately rounded operations, then rounded to the storage dtype
  (fp32 as is, bf16 by round-to-nearest-even).

Because only integer operations, one table lookup and correctly rounded fp32
operations are involved, the numpy code here and the HIP fill kernel in
``synth/fill.hip`` produce identical bits.
"""

from __future__ import annotations

import statistics
from dataclasses import dataclass

import numpy as np

MASK64 = (1 << 64) - 1
GAMMA = 0x9E3779B97F4A7C15
MIX_M1 = 0xBF58476D1CE4E5B9
MIX_M2 = 0x94D049BB133111EB
TABLE_INTERVALS = 65536

# Tensor tags: one independent stream per tensor of a layer.
TAG_Q = 1
TAG_K = 2
TAG_V = 3
TAG_F = 4
TAG_K_OFFSET = 5
TAG_V_OFFSET = 6
TAG_F_SELF = 7
TAG_F_AHEAD = 8  # Forecast of the layer j > 1 ahead: tag 8 + (j - 2), j <= 9
LAYER_TAG_STRIDE = 16  # layer l uses tag + 16 * l
# Hidden states and projection weights live in their own tag range (+ 16 * layer)
TAG_HIDDEN = 4096
TAG_W_QKVF = 4097


def _mix64_int(z: int) -> int:
    z &= MASK64
    z = ((z ^ (z >> 30)) * MIX_M1) & MASK64
    z = ((z ^ (z >> 27)) * MIX_M2) & MASK64
    return z ^ (z >> 31)


def stream_base(seed: int, tag: int) -> int:
    """State of the SplitMix64 stream for (seed, tag)."""
    return _mix64_int(((seed & 0xFFFFFFFF) << 32) ^ (tag & 0xFFFFFFFF))


def _mix64(z: np.ndarray) -> np.ndarray:
    z = (z ^ (z >> np.uint64(30))) * np.uint64(MIX_M1)
    z = (z ^ (z >> np.uint64(27))) * np.uint64(MIX_M2)
    return z ^ (z >> np.uint64(31))


def raw64(seed: int, tag: int, idx: np.ndarray) -> np.ndarray:
    """64-bit outputs for flat indices ``idx`` (uint64 array)."""
    base = np.uint64(stream_base(seed, tag))
    idx = np.asarray(idx, dtype=np.uint64)
    with np.errstate(over="ignore"):
        state = base + (idx + np.uint64(1)) * np.uint64(GAMMA)
        return _mix64(state)


_TABLE = None


def normal_table() -> np.ndarray:
    """The 65537 fp32 quantile knots used by ``std_normal``."""
    global _TABLE
    if _TABLE is None:
        nd = statistics.NormalDist()
        n = TABLE_INTERVALS + 1
        knots = [nd.inv_cdf((j + 0.5) / n) for j in range(n)]
        _TABLE = np.asarray(knots, dtype=np.float64).astype(np.float32)
        _TABLE.setflags(write=False)
    return _TABLE


def std_normal(seed: int, tag: int, idx: np.ndarray) -> np.ndarray:
    """fp32 N(0,1) draws for flat indices ``idx``."""
    r = raw64(seed, tag, idx)
    j = (r >> np.uint64(48)).astype(np.int64)
    frac = ((r >> np.uint64(32)) & np.uint64(0xFFFF)).astype(np.float32)
    u = frac * np.float32(2.0 ** -16)
    t = normal_table()
    t0 = t[j]
    t1 = t[j + 1]
    return t0 + u * (t1 - t0)


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round fp32 to bf16 (round to nearest, ties to even); returns uint16 bits."""
    b = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    rounded = (b + np.uint64(0x7FFF) + ((b >> np.uint64(16)) & np.uint64(1))) >> np.uint64(16)
    return rounded.astype(np.uint16)


def bf16_bits_to_f32(h: np.ndarray) -> np.ndarray:
    """Exact widening of bf16 bits to fp32."""
    return (np.asarray(h, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


@dataclass(frozen=True)
class Recipe:
    """How one tensor is drawn.

    ``scale``: multiply each N(0,1) draw by this fp32 constant (None: no scale).
    ``offset_tag``/``offset_std``/``block``: add ``offset_std * z_off`` where
    z_off is one N(0,1) d-vector per (leading indices, token // block), drawn
    from stream ``offset_tag`` at flat index ((lead * nblocks + blk) * d + c).
    ``dtype``: "fp32" or "bf16".
    """

    seed: int
    tag: int
    dtype: str = "bf16"
    scale: float | None = None
    offset_tag: int | None = None
    offset_std: float = 0.5
    block: int = 64


def values_f32(recipe: Recipe, shape: tuple, flat_idx: np.ndarray) -> np.ndarray:
    """fp32 values (before storage rounding) at the given flat indices."""
    flat_idx = np.asarray(flat_idx, dtype=np.int64)
    z = std_normal(recipe.seed, recipe.tag, flat_idx.astype(np.uint64))
    if recipe.scale is not None:
        z = z * np.float32(recipe.scale)
    if recipe.offset_tag is not None:
        *lead, T, d = shape
        nblk = T // recipe.block
        c = flat_idx % d
        t = (flat_idx // d) % T
        lead_i = flat_idx // (d * T)
        off_idx = (lead_i * nblk + t // recipe.block) * d + c
        zo = std_normal(recipe.seed, recipe.offset_tag, off_idx.astype(np.uint64))
        z = z + np.float32(recipe.offset_std) * zo
    return z.astype(np.float32)


def generate(recipe: Recipe, shape: tuple) -> np.ndarray:
    """Whole tensor in its storage format: float32 array, or uint16 bf16 bits."""
    n = int(np.prod(shape))
    out_dtype = np.float32 if recipe.dtype == "fp32" else np.uint16
    out = np.empty(n, dtype=out_dtype)
    chunk = 1 << 22
    for s in range(0, n, chunk):
        e = min(n, s + chunk)
        v = values_f32(recipe, shape, np.arange(s, e, dtype=np.int64))
        out[s:e] = v if recipe.dtype == "fp32" else f32_to_bf16_bits(v)
    return out.reshape(shape)


def generate_slice(recipe: Recipe, shape: tuple, lead: tuple, t0: int = 0, t1: int | None = None) -> np.ndarray:
    """Rows [t0, t1) of the trailing [T, d] matrix at leading index ``lead``."""
    *lead_shape, T, d = shape
    t1 = T if t1 is None else t1
    lin = int(np.ravel_multi_index(lead, lead_shape)) if lead_shape else 0
    base = (lin * T + t0) * d
    idx = np.arange(base, base + (t1 - t0) * d, dtype=np.int64)
    v = values_f32(recipe, shape, idx)
    v = v if recipe.dtype == "fp32" else f32_to_bf16_bits(v)
    return v.reshape(t1 - t0, d)


def as_float64(x: np.ndarray, dtype: str) -> np.ndarray:
    """Exact fp64 view of stored values (bf16 bits or fp32)."""
    if dtype == "bf16":
        return bf16_bits_to_f32(x).astype(np.float64)
    return np.asarray(x, dtype=np.float32).astype(np.float64)
