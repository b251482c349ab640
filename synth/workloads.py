"""The five synthetic workloads of the block-selection hot path.

Shapes stand in for one layer of an 8B GQA model at long context (32 query
heads over 8 KV heads, head dim 128, 64-token KV blocks, keys compressed with
kernel 32 / stride 16). Values are synthetic and seeded; see ``synth`` for the
generator definition. No method arithmetic here.
"""

from __future__ import annotations

from dataclasses import dataclass, field

from . import (LAYER_TAG_STRIDE, TAG_F, TAG_F_AHEAD, TAG_F_SELF, TAG_HIDDEN, TAG_K, TAG_K_OFFSET, TAG_Q, TAG_V,
               TAG_V_OFFSET, TAG_W_QKVF, Recipe)

INV_SQRT_128 = 0.08838834764831845  # 1/sqrt(128); rounded to fp32 where applied


@dataclass(frozen=True)
class Workload:
    name: str
    description: str
    dtype: str  # "fp32" | "bf16"
    B: int
    Hq: int
    Hkv: int
    T: int
    d: int
    Tq: int
    q_start: int
    k: int
    seed: int
    block: int = 64
    kernel: int = 32
    stride: int = 16
    tile: int = 64
    value_scale: float | None = None   # every tensor multiplied by this (tiny fp32 config)
    block_offsets: bool = False        # K/V get a per-block N(0, 0.5^2) offset vector
    layers: int = 1
    extra: dict = field(default_factory=dict)

    @property
    def G(self) -> int:
        return self.Hq // self.Hkv

    @property
    def nB(self) -> int:
        return self.T // self.block

    @property
    def W(self) -> int:
        return (self.T - self.kernel) // self.stride + 1

    @property
    def n_tiles(self) -> int:
        return -(-self.Tq // self.tile)

    @property
    def scale(self) -> float:
        return self.d ** -0.5

    def shape(self, name: str) -> tuple:
        if name == "Q":
            return (self.B, self.Hq, self.Tq, self.d)
        if name in ("F", "F_self"):
            return (self.B, self.Hkv, self.Tq, self.d)
        if name in ("K", "V"):
            return (self.B, self.Hkv, self.T, self.d)
        if name == "Kc":
            return (self.B, self.Hkv, self.W, self.d)
        raise KeyError(name)

    def recipe(self, name: str, layer: int = 0, ahead: int = 1) -> Recipe:
        """``ahead`` (for "F" only): how many layers ahead the Forecast looks."""
        tags = {"Q": TAG_Q, "K": TAG_K, "V": TAG_V, "F": TAG_F, "F_self": TAG_F_SELF}
        off = {"K": TAG_K_OFFSET, "V": TAG_V_OFFSET}
        shift = LAYER_TAG_STRIDE * layer
        offset_tag = off[name] + shift if (self.block_offsets and name in off) else None
        tag = tags[name]
        if name == "F" and ahead != 1:
            if not 2 <= ahead <= 9:
                raise ValueError("a Forecast looks 1 to 9 layers ahead")
            tag = TAG_F_AHEAD + ahead - 2
        return Recipe(seed=self.seed, tag=tag + shift, dtype=self.dtype, scale=self.value_scale,
                      offset_tag=offset_tag, offset_std=0.5, block=self.block)


C1_TINY = Workload(
    name="c1_tiny_decode_fp32",
    description="tiny decode, fp32: B=1, T=4096, 4 query heads / 1 KV head, d=128, top-16 of 64 blocks",
    dtype="fp32", B=1, Hq=4, Hkv=1, T=4096, d=128, Tq=1, q_start=4095, k=16, seed=0,
    value_scale=INV_SQRT_128)

C2_DECODE_32K = Workload(
    name="c2_decode_32k_bf16",
    description="single-sequence decode, bf16: B=1, T=32768, 32/8 heads, d=128, top-64 of 512 blocks",
    dtype="bf16", B=1, Hq=32, Hkv=8, T=32768, d=128, Tq=1, q_start=32767, k=64, seed=1,
    block_offsets=True)

C3_DECODE_128K = Workload(
    name="c3_decode_128k_b16_bf16",
    description="batched long-context decode, bf16: B=16, T=131072, 32/8 heads, d=128, top-64 of 2048 blocks",
    dtype="bf16", B=16, Hq=32, Hkv=8, T=131072, d=128, Tq=1, q_start=131071, k=64, seed=2,
    block_offsets=True)

C4_OFFLOAD = Workload(
    name="c4_offload_lookahead_b64_bf16",
    description=("offloaded decode with lookahead prefetch, bf16: B=64, T=131072, 32/8 heads, d=128, "
                 "top-64; layer 1 KV in pinned host memory, two layers"),
    dtype="bf16", B=64, Hq=32, Hkv=8, T=131072, d=128, Tq=1, q_start=131071, k=64, seed=3,
    block_offsets=True, layers=2)

C5_PREFILL = Workload(
    name="c5_chunked_prefill_bf16",
    description=("chunked prefill, bf16: B=1, 4096 queries at positions 126976..131071 of T=131072, "
                 "32/8 heads, d=128, causal, top-64 per 64-query tile"),
    dtype="bf16", B=1, Hq=32, Hkv=8, T=131072, d=128, Tq=4096, q_start=126976, k=64, seed=4)

ALL = [C1_TINY, C2_DECODE_32K, C3_DECODE_128K, C4_OFFLOAD, C5_PREFILL]
BY_NAME = {w.name: w for w in ALL}


def scaled(w: Workload, **changes) -> Workload:
    """A smaller variant of a workload (same recipe), for parity at oracle-friendly sizes."""
    from dataclasses import replace
    return replace(w, **changes)


# --------------------------------------------- the projections upstream ----
MODEL_DIM = 4096  # hidden size of the 8B models the pages measure on


def qkvf_rows(w: Workload, n_f: int = 1) -> int:
    """Rows of the concatenated Q/K/V/Forecast weight matrix."""
    return (w.Hq + 2 * w.Hkv + n_f * w.Hkv) * w.d


def hidden_recipe(w: Workload, layer: int = 0) -> Recipe:
    """Hidden states x [B, D] of one decode token per sequence, N(0, 1)."""
    return Recipe(seed=w.seed, tag=TAG_HIDDEN + LAYER_TAG_STRIDE * layer, dtype=w.dtype)


def qkvf_weight_recipe(w: Workload, D: int = MODEL_DIM, layer: int = 0) -> Recipe:
    """Random projection weights [qkvf_rows, D], N(0, 1/D), so that the
    projected vectors are about N(0, 1) like the other synthetic inputs."""
    return Recipe(seed=w.seed, tag=TAG_W_QKVF + LAYER_TAG_STRIDE * layer, dtype=w.dtype, scale=D ** -0.5)
