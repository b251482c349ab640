"""A decode step over L layers whose KV (all but layer 0's) sits in pinned host
memory, with lookahead prefetch into staging buffers used in turn.

SparDA's runtime (bittide.aicompass.dev summary post, paragraphs on the
decoupled Forecast and on prefetching over a separate stream; techwalker.com
article, section 三) extended from one lookahead layer to a stack: at the start
of layer l the layer's Forecast vector scores layer l+1's compressed keys, and
layer l+1's selected blocks cross the host link into staging buffer (l+1) % 2
while layer l attends from buffer l % 2. Layer 0 keeps its KV in HBM and
selects with a Forecast of its own layer.

Only the order of the library's calls on two HIP streams lives here; every
step runs in libsparda's kernels. Per step, with "main" the caller's stream:

  main: select(F_0->1, K~1) -> idx1; record e_idx[1]
  side: wait e_idx[1]; gather layer 1 -> staging 1; record e_stage[1]
  main: select(F_0 self, K~0) -> idx0; attention of layer 0 from HBM
  for l = 1 .. L-1:
    main: select(F_l->l+1, K~l+1) -> idx[l+1]; record e_idx[l+1]     (l+1 < L)
    side: wait e_idx[l+1]; gather layer l+1 -> staging (l+1) % 2; record e_stage[l+1]
    main: wait e_stage[l]; attention of layer l from staging l % 2

The gather of layer l+1 overwrites the buffer layer l-1 attended from; it waits
for e_idx[l+1], recorded on main after that attention was enqueued. The next
step's first gather likewise follows this step's last attention, and main has
waited for every gather of this step before the next step's top-k rewrites the
indices those gathers read.

Lookahead of ``depth`` D > 1 layers (10100.com commentary, section 硅基观点,
names a Forecast that looks several layers ahead instead of one as a next step):
layer l's Forecast picks the blocks of layer l+D, so D gathers can be in
flight while a layer attends, in D+1 staging buffers used in turn. The layers
1 .. D have no layer D below them in the step; layer 0's input forecasts all
of them (F_ahead[j-1] for layer j), and their selections and gathers go first:

  main: for j = 1 .. D: select(F_0->j, K~j) -> idx[j]; side: gather j -> staging j % (D+1)
  main: select(F_0 self, K~0) -> idx0; attention of layer 0 from HBM
  for l = 1 .. L-1:
    main: select(F_l->l+D, K~l+D) -> idx[l+D]; side: gather -> staging (l+D) % (D+1)   (l+D < L)
    main: wait e_stage[l]; attention of layer l from staging l % (D+1)

Staging (l+D) % (D+1) is the buffer of layer l-1, so the hazard argument above
holds for every D.
"""

from __future__ import annotations

from . import (BLOCK, HEAD_DIM, KV_STAGING, OP_BLOCK_SPARSE_ATTN, block_sparse_attn, prefetch_blocks,
               select_forecast, topk_blocks, workspace_bytes)


class LayerPipeline:
    """Buffers, side stream and events of the L-layer offloaded decode step.

    :meth:`step` takes a list of L layer dicts: layer 0 with ``Q``, ``F_self``,
    ``F_next``, ``K``, ``V``, ``Kc`` in HBM; layers 1 .. L-1 with ``Q``, ``Kc``
    in HBM, ``host_K``, ``host_V`` in pinned host memory and, except the last,
    ``F_next``. Outputs and indices are buffers owned by this object.
    """

    def __init__(self, L: int, B: int, Hq: int, Hkv: int, T: int, k: int, dtype, device="cuda",
                 num_workgroups: int = 0, depth: int = 1):
        import torch
        if L < 1:
            raise ValueError("L must be at least 1")
        if depth < 1:
            raise ValueError("depth must be at least 1")
        self.L, self.B, self.Hq, self.Hkv, self.T, self.k = L, B, Hq, Hkv, T, k
        self.depth = depth
        self.device = torch.device(device)
        self.num_workgroups = num_workgroups
        dev = self.device
        nB = T // BLOCK
        self.scores = [torch.empty((B, Hkv, 1, nB), dtype=torch.float32, device=dev) for _ in range(L)]
        self.idx = [torch.empty((B, Hkv, 1, k), dtype=torch.int32, device=dev) for _ in range(L)]
        self.out = [torch.empty((B, Hq, 1, HEAD_DIM), dtype=dtype, device=dev) for _ in range(L)]
        n_stage = min(depth + 1, L - 1)  # never more than the offloaded layers
        self.stage = [(torch.empty((B, Hkv, k, BLOCK, HEAD_DIM), dtype=dtype, device=dev),
                       torch.empty((B, Hkv, k, BLOCK, HEAD_DIM), dtype=dtype, device=dev)) for _ in range(n_stage)]
        self.ws = torch.empty(workspace_bytes(OP_BLOCK_SPARSE_ATTN, B, Hq, Hkv, 1, T, k), dtype=torch.uint8,
                              device=dev)
        self.side = torch.cuda.Stream(device=dev)  # default priority
        self.e_idx = [torch.cuda.Event() for _ in range(L)]
        self.e_stage = [torch.cuda.Event() for _ in range(L)]

    def _select(self, f, kc, l: int, main) -> None:
        select_forecast(f, kc, self.T, self.T - 1, out=self.scores[l], stream=main)
        topk_blocks(self.scores[l], self.k, out=self.idx[l], stream=main)

    def _forecast(self, layers: list, src: int, dst: int):
        """Layer src's Forecast vector of layer dst's blocks."""
        fa = layers[src].get("F_ahead")
        if fa is None:  # one layer ahead
            if dst != src + 1:
                raise ValueError(f"layer {src} has no F_ahead for lookahead depth {self.depth}")
            return layers[src]["F_next"]
        return fa[dst - 1] if src == 0 else fa

    def _gather(self, layer: dict, l: int, main) -> None:
        self.e_idx[l].record(main)
        self.side.wait_event(self.e_idx[l])
        sk, sv = self.stage[l % len(self.stage)]
        prefetch_blocks(layer["host_K"], layer["host_V"], self.idx[l].view(self.B, self.Hkv, self.k), sk, sv,
                        num_workgroups=self.num_workgroups, stream=self.side)
        self.e_stage[l].record(self.side)

    def step(self, layers: list, stream=None):
        """Enqueue one step over the L layers; returns (outs, idxs), valid once
        ``stream`` reaches this point."""
        import torch
        if len(layers) != self.L:
            raise ValueError(f"expected {self.L} layers, got {len(layers)}")
        main = stream if stream is not None else torch.cuda.current_stream(self.device)
        T, q, D = self.T, self.T - 1, self.depth
        l0 = layers[0]
        for j in range(1, min(D, self.L - 1) + 1):
            self._select(self._forecast(layers, 0, j), layers[j]["Kc"], j, main)
            self._gather(layers[j], j, main)
        self._select(l0["F_self"], l0["Kc"], 0, main)
        block_sparse_attn(l0["Q"], l0["K"], l0["V"], self.idx[0], T, q, out=self.out[0], ws=self.ws, stream=main)
        for l in range(1, self.L):
            if l + D < self.L:
                self._select(self._forecast(layers, l, l + D), layers[l + D]["Kc"], l + D, main)
                self._gather(layers[l + D], l + D, main)
            main.wait_event(self.e_stage[l])
            sk, sv = self.stage[l % len(self.stage)]
            block_sparse_attn(layers[l]["Q"], sk, sv, self.idx[l], T, q, kv_mode=KV_STAGING, out=self.out[l],
                              ws=self.ws, stream=main)
        return self.out, self.idx
