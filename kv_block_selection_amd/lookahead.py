"""One decode step of two layers with lookahead prefetch of offloaded KV blocks.

SparDA's runtime (bittide.aicompass.dev summary post, paragraphs on the
decoupled Forecast and on prefetching over a separate stream; techwalker.com
article, section 三): layer L's Forecast vector scores layer L+1's compressed
keys, so the blocks layer L+1 will attend over are known before layer L's
attention runs. Their transfer from pinned host memory then overlaps layer L's
attention. Layer 0 keeps its KV in HBM and selects with a Forecast of its own
layer (techwalker.com article, section 三).

This module only orders the library's calls on two HIP streams with events;
every step runs in libsparda's kernels. Per step, on the caller's stream
("main") and a side stream:

  main: select(F0->1,  K~1) -> top-k -> idx1, record e_idx1
        select(F0_self, K~0) -> top-k -> idx0       (these two overlap
        attention(Q0, KV0 in HBM, idx0)              the gather)
        wait e_stage
        attention(Q1, staging, idx1)
  side: wait e_idx1
        prefetch(host KV1, idx1 -> staging), record e_stage

Layer 1's selection goes first because only it gates the gather, which is the
long pole (it crosses the host link); all of layer 0's work then runs beside it.

With ``cache_slots`` set, the staging buffer is kept as a cache of host blocks
across steps (sparda_prefetch_blocks_cached): a block the previous steps
already staged is not fetched again, and layer 1 attends through the slot map
the gather writes.

Hazards across steps are covered by stream order: e_idx1 of step n+1 is
recorded after the layer-1 attention of step n was enqueued on main, so the
prefetch of step n+1 cannot overwrite staging still being read; and main waited
for e_stage of step n before step n+1's top-k rewrites idx1, which that
prefetch reads.
"""

from __future__ import annotations

from . import (BLOCK, HEAD_DIM, KV_SLOTS, KV_STAGING, OP_BLOCK_SPARSE_ATTN, block_sparse_attn, prefetch_blocks,
               prefetch_blocks_cached, select_forecast, topk_blocks, workspace_bytes)


class LookaheadStep:
    """Buffers, side stream and events of the two-layer offloaded decode step.

    Layer inputs are passed to :meth:`step` as dicts of tensors:
      layer0: ``Q`` [B,Hq,1,128], ``F_self`` and ``F_next`` [B,Hkv,1,128],
              ``K``, ``V`` [B,Hkv,T,128] in HBM, ``Kc`` [B,Hkv,W,128];
      layer1: ``Q`` [B,Hq,1,128], ``Kc`` [B,Hkv,W,128] in HBM and
              ``host_K``, ``host_V`` [B,Hkv,T,128] in pinned host memory.
    The outputs and indices are buffers owned by this object, overwritten by
    the next step.
    """

    def __init__(self, B: int, Hq: int, Hkv: int, T: int, k: int, dtype, device="cuda",
                 num_workgroups: int = 0, cache_slots: int = 0, markers: bool = False):
        import torch
        self.B, self.Hq, self.Hkv, self.T, self.k = B, Hq, Hkv, T, k
        # markers: host-side ranges around each phase's enqueue (roctx through
        # torch.cuda.nvtx; rocprofv3 --marker-trace shows them)
        self.markers = markers
        self.device = torch.device(device)
        self.num_workgroups = num_workgroups
        nB = T // BLOCK
        f32, i32 = torch.float32, torch.int32
        dev = self.device
        self.scores0 = torch.empty((B, Hkv, 1, nB), dtype=f32, device=dev)
        self.scores1 = torch.empty((B, Hkv, 1, nB), dtype=f32, device=dev)
        self.idx0 = torch.empty((B, Hkv, 1, k), dtype=i32, device=dev)
        self.idx1 = torch.empty((B, Hkv, 1, k), dtype=i32, device=dev)
        self.cache_slots = cache_slots
        slots = cache_slots if cache_slots else k
        self.stage_k = torch.empty((B, Hkv, slots, BLOCK, HEAD_DIM), dtype=dtype, device=dev)
        self.stage_v = torch.empty_like(self.stage_k)
        if cache_slots:
            if cache_slots < k:
                raise ValueError("cache_slots must be at least k")
            self.slot_tags = torch.full((B, Hkv, cache_slots), -1, dtype=i32, device=dev)  # all empty
            self.slot_of = torch.empty((B, Hkv, k), dtype=i32, device=dev)
        self.out0 = torch.empty((B, Hq, 1, HEAD_DIM), dtype=dtype, device=dev)
        self.out1 = torch.empty_like(self.out0)
        # both attentions run on the main stream, one after the other: one workspace
        self.ws = torch.empty(workspace_bytes(OP_BLOCK_SPARSE_ATTN, B, Hq, Hkv, 1, T, k), dtype=torch.uint8,
                              device=dev)
        self.side = torch.cuda.Stream(device=dev)  # default priority
        self.e_idx1 = torch.cuda.Event()
        self.e_stage = torch.cuda.Event()

    def select_next(self, layer0: dict, layer1: dict, main) -> None:
        """Lookahead selection on ``main``: layer 0's Forecast of layer 1 -> idx1."""
        T, q = self.T, self.T - 1
        select_forecast(layer0["F_next"], layer1["Kc"], T, q, out=self.scores1, stream=main)
        topk_blocks(self.scores1, self.k, out=self.idx1, stream=main)

    def select_self(self, layer0: dict, main) -> None:
        """Layer 0's own selection on ``main`` (same-layer Forecast) -> idx0."""
        T, q = self.T, self.T - 1
        select_forecast(layer0["F_self"], layer0["Kc"], T, q, out=self.scores0, stream=main)
        topk_blocks(self.scores0, self.k, out=self.idx0, stream=main)

    def select(self, layer0: dict, layer1: dict, main) -> None:
        """Both selections on ``main``."""
        self.select_next(layer0, layer1, main)
        self.select_self(layer0, main)

    def prefetch(self, layer1: dict) -> None:
        """Gather layer 1's selected blocks into staging on the side stream."""
        idx = self.idx1.view(self.B, self.Hkv, self.k)
        if self.cache_slots:
            prefetch_blocks_cached(layer1["host_K"], layer1["host_V"], idx, self.slot_tags, self.slot_of,
                                   self.stage_k, self.stage_v, num_workgroups=self.num_workgroups, stream=self.side)
        else:
            prefetch_blocks(layer1["host_K"], layer1["host_V"], idx, self.stage_k, self.stage_v,
                            num_workgroups=self.num_workgroups, stream=self.side)

    def attend_next(self, layer1: dict, main) -> None:
        """Layer 1's attention from staging on ``main``."""
        T, q = self.T, self.T - 1
        if self.cache_slots:
            block_sparse_attn(layer1["Q"], self.stage_k, self.stage_v, self.idx1, T, q, kv_mode=KV_SLOTS,
                              slot_of=self.slot_of, out=self.out1, ws=self.ws, stream=main)
        else:
            block_sparse_attn(layer1["Q"], self.stage_k, self.stage_v, self.idx1, T, q, kv_mode=KV_STAGING,
                              out=self.out1, ws=self.ws, stream=main)

    def _phase(self, name: str):
        """A marker range around one phase's enqueue (no-op unless ``markers``)."""
        import contextlib
        if not self.markers:
            return contextlib.nullcontext()
        import torch
        return torch.cuda.nvtx.range(name)

    def step(self, layer0: dict, layer1: dict, stream=None):
        """Enqueue one step; returns (out0, out1, idx0, idx1), valid once ``stream`` reaches this point."""
        import torch
        main = stream if stream is not None else torch.cuda.current_stream(self.device)
        T, q = self.T, self.T - 1
        with self._phase("select_layer1"):
            self.select_next(layer0, layer1, main)
            self.e_idx1.record(main)
        with self._phase("prefetch_layer1"):
            self.side.wait_event(self.e_idx1)
            self.prefetch(layer1)
            self.e_stage.record(self.side)
        with self._phase("select_layer0"):
            self.select_self(layer0, main)
        with self._phase("attend_layer0"):
            block_sparse_attn(layer0["Q"], layer0["K"], layer0["V"], self.idx0, T, q, out=self.out0, ws=self.ws,
                              stream=main)
        with self._phase("attend_layer1"):
            main.wait_event(self.e_stage)
            self.attend_next(layer1, main)
        return self.out0, self.out1, self.idx0, self.idx1
