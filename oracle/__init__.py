"""fp64 oracle for SparDA's decoupled block selection and block-sparse attention.

TEST INFRASTRUCTURE. Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this module. The product path
(``kv_block_selection_amd`` and ``libsparda.so``) never calls it, and this
module imports nothing from the product path: the two share no code.

Plain, slow, obviously correct numpy in float64. Inputs are the exact stored
values (bf16 or fp32 widened to fp64). Each function names the passage of the
source pages it follows. The pages:

* [P1] bittide.aicompass.dev: summary post on SparDA, followed by the arXiv
  abstract of "SparDA: Sparse Decoupled Attention for Efficient Long-Context
  LLM Inference" (arXiv:2606.04511). Cited by paragraph topic or "abstract".
* [P2] techwalker.com article on SparDA (NVIDIA/MIT); sections 一 (problem),
  二 (Forecast), 三 (implementation), 四 (training), 五 (experiments), 六 (limits).
* [P3] 10100.com commentary on arXiv:2606.04511; sections 痛点 (pain points),
  解法 (the method), 和现有工作的关系 (related work).

Where the pages leave a step open, the reading taken is stated at the function
(the pooling operator, how window scores become block scores, visibility,
ties, output order). Every function here is pinned by a ``-m "not gpu"`` test
against closed forms, hand-worked values, brute force or a library routine;
none is "parity unpinned".

Shapes (row-major):
  K, V      [B, Hkv, T, d]       keys / values of one layer
  Kc        [B, Hkv, W, d]       compressed keys, W = (T - kernel)//stride + 1
  F         [B, Hkv, Tq, d]      one Forecast vector per GQA group and query
  Q         [B, Hq, Tq, d]       query heads; head q uses KV head q // (Hq//Hkv)
  scores    [B, Hkv, nTiles, nB] block scores, -inf for non-candidates
  idx       [B, Hkv, nTiles, k]  int32 selected blocks, ascending, -1 padded
Query i of a chunk sits at position q_start + i; decode is Tq = 1,
q_start = T - 1.
"""

from __future__ import annotations

import numpy as np

NEG_INF = -np.inf


# ---------------------------------------------------------------- step 1 ----
def compress_keys(K: np.ndarray, kernel: int = 32, stride: int = 16) -> np.ndarray:
    """Mean-pooled key windows ([P2] 四: kernel 32, stride 16 at inference).

    Window w covers tokens [stride*w, stride*w + kernel). Only complete windows
    are formed, so W = (T - kernel)//stride + 1. The pages name no pooling
    operator for this step; the arithmetic mean is the reading taken.
    """
    K = np.asarray(K, dtype=np.float64)
    T = K.shape[-2]
    W = (T - kernel) // stride + 1
    out = np.empty(K.shape[:-2] + (W, K.shape[-1]), dtype=np.float64)
    for w in range(W):
        out[..., w, :] = K[..., w * stride: w * stride + kernel, :].mean(axis=-2)
    return out


def num_windows(T: int, kernel: int = 32, stride: int = 16) -> int:
    return (T - kernel) // stride + 1


# ------------------------------------------------ windows, blocks, causality --
def visible_window_count(p: int, W: int, kernel: int = 32, stride: int = 16) -> int:
    """Number of windows a query at position p may see.

    Reading: a window is visible when every token in it is at or before p,
    i.e. stride*w + kernel - 1 <= p (plain causality on compressed keys).
    Visible windows are always a prefix 0..n-1.
    """
    w = np.arange(W)
    return int(np.count_nonzero(w * stride + kernel - 1 <= p))


def block_window_ranges(T: int, block: int = 64, kernel: int = 32, stride: int = 16):
    """For every block beta: the first and last window whose span meets it.

    Block beta holds tokens [block*beta, block*beta + block). A window meets it
    when the two token intervals intersect. Reading: a block is scored from
    every window that overlaps it (none is dropped at block edges).
    Returns (lo, hi) int arrays of length nB.
    """
    W = num_windows(T, kernel, stride)
    nB = T // block
    starts = np.arange(W) * stride
    ends = starts + kernel  # exclusive
    beta = np.arange(nB)
    lo = np.searchsorted(ends, block * beta, side="right")          # windows ending at/before the block
    hi = np.searchsorted(starts, block * (beta + 1), side="left") - 1  # windows starting inside/before it
    return lo, hi


def pool_windows_to_blocks(win_scores: np.ndarray, n_visible: int, lo: np.ndarray, hi: np.ndarray) -> np.ndarray:
    """Block score = max of the window scores over the visible windows meeting the block.

    Reading: max, the same down-sampling operator the method uses to bring
    fine-grained scores to inference resolution ([P2] 四). A block with no
    visible window gets -inf (not a candidate).
    win_scores: [W] for one query. Returns [nB].
    """
    nB = lo.shape[0]
    out = np.full(nB, NEG_INF)
    for beta in range(nB):
        a = lo[beta]
        b = min(hi[beta], n_visible - 1)
        if a <= b:
            out[beta] = np.max(win_scores[a: b + 1])
    return out


# ---------------------------------------------------------------- step 2 ----
def forecast_window_scores(f: np.ndarray, kc: np.ndarray, scale: float) -> np.ndarray:
    """Forecast score of every window: scale * f . kc[w], no softmax.

    One Forecast head per GQA group scores the compressed keys directly; no
    per-query-head loop and no softmax ([P1] paragraph on one Forecast head
    per GQA group; [P2] 二; [P3] 解法). f: [d], kc: [W, d] -> [W].
    """
    return scale * (np.asarray(kc, np.float64) @ np.asarray(f, np.float64))


def multihead_window_scores(q_group: np.ndarray, kc: np.ndarray, scale: float, n_visible: int) -> np.ndarray:
    """The original selector: every query head of the group scores every window,
    softmax per head over the visible windows, then the sum over the group
    ([P1] paragraph on the standard selector; [P3] 痛点).

    q_group: [G, d]; kc: [W, d]. Returns [W]; invisible windows get -inf.
    """
    W = kc.shape[0]
    out = np.full(W, NEG_INF)
    if n_visible == 0:
        return out
    total = np.zeros(n_visible)
    for g in range(q_group.shape[0]):
        logits = scale * (np.asarray(kc[:n_visible], np.float64) @ np.asarray(q_group[g], np.float64))
        m = np.max(logits)
        e = np.exp(logits - m)
        total += e / np.sum(e)
    out[:n_visible] = total
    return out


def _tile_bounds(Tq: int, tile: int):
    n_tiles = -(-Tq // tile)
    return [(t * tile, min(Tq, (t + 1) * tile)) for t in range(n_tiles)]


def select_forecast_tile(f_rows: np.ndarray, kc: np.ndarray, positions, T: int, scale: float,
                         block: int = 64, kernel: int = 32, stride: int = 16) -> np.ndarray:
    """Block scores of one (sequence, KV head, query tile) under the Forecast.

    Reading for prefill: a tile of queries shares one selection, scored as the
    max over its queries of each query's block score. f_rows: [n, d].
    Returns [nB].
    """
    lo, hi = block_window_ranges(T, block, kernel, stride)
    W = kc.shape[0]
    acc = np.full(T // block, NEG_INF)
    for r, p in enumerate(positions):
        s = forecast_window_scores(f_rows[r], kc, scale)
        acc = np.maximum(acc, pool_windows_to_blocks(s, visible_window_count(p, W, kernel, stride), lo, hi))
    return acc


def select_multihead_tile(q_rows: np.ndarray, kc: np.ndarray, positions, T: int, scale: float,
                          block: int = 64, kernel: int = 32, stride: int = 16) -> np.ndarray:
    """Block scores of one (sequence, KV head, query tile) under the multi-head selector.

    q_rows: [G, n, d] (the group's query heads for the tile's queries).
    Returns [nB].
    """
    lo, hi = block_window_ranges(T, block, kernel, stride)
    W = kc.shape[0]
    acc = np.full(T // block, NEG_INF)
    for r, p in enumerate(positions):
        nv = visible_window_count(p, W, kernel, stride)
        s = multihead_window_scores(q_rows[:, r, :], kc, scale, nv)
        acc = np.maximum(acc, pool_windows_to_blocks(s, nv, lo, hi))
    return acc


def select_forecast(F: np.ndarray, Kc: np.ndarray, T: int, q_start: int, scale: float,
                    block: int = 64, kernel: int = 32, stride: int = 16, tile: int = 64) -> np.ndarray:
    """Forecast block scores [B, Hkv, nTiles, nB] for F [B, Hkv, Tq, d]."""
    B, Hkv, Tq, _ = F.shape
    tiles = _tile_bounds(Tq, tile)
    out = np.empty((B, Hkv, len(tiles), T // block))
    for b in range(B):
        for h in range(Hkv):
            for t, (i0, i1) in enumerate(tiles):
                pos = [q_start + i for i in range(i0, i1)]
                out[b, h, t] = select_forecast_tile(F[b, h, i0:i1], Kc[b, h], pos, T, scale, block, kernel, stride)
    return out


def select_multihead(Q: np.ndarray, Kc: np.ndarray, T: int, q_start: int, scale: float,
                     block: int = 64, kernel: int = 32, stride: int = 16, tile: int = 64) -> np.ndarray:
    """Multi-head-selector block scores [B, Hkv, nTiles, nB] for Q [B, Hq, Tq, d].

    Query head q belongs to the group of KV head q // G with G = Hq / Hkv
    (contiguous groups).
    """
    B, Hq, Tq, _ = Q.shape
    Hkv = Kc.shape[1]
    G = Hq // Hkv
    tiles = _tile_bounds(Tq, tile)
    out = np.empty((B, Hkv, len(tiles), T // block))
    for b in range(B):
        for h in range(Hkv):
            for t, (i0, i1) in enumerate(tiles):
                pos = [q_start + i for i in range(i0, i1)]
                out[b, h, t] = select_multihead_tile(Q[b, h * G:(h + 1) * G, i0:i1], Kc[b, h], pos, T, scale,
                                                     block, kernel, stride)
    return out


# ---------------------------------------------------------------- step 3 ----
def topk_row(scores: np.ndarray, k: int) -> np.ndarray:
    """Keep the k best blocks of one row ([P1]: score the blocks, keep the top-k).

    Candidates are the blocks with a finite score. They are ranked by score,
    higher first, ties going to the lower block index; the first min(k, #cand)
    are kept and returned in ascending block order, padded with -1.
    """
    scores = np.asarray(scores, dtype=np.float64)
    cand = np.nonzero(scores > NEG_INF)[0]
    order = cand[np.lexsort((cand, -scores[cand]))]  # primary: -score, secondary: index
    chosen = np.sort(order[:k])
    out = np.full(k, -1, dtype=np.int32)
    out[: chosen.size] = chosen
    return out


def topk_blocks(scores: np.ndarray, k: int) -> np.ndarray:
    """Row-wise ``topk_row`` over the last axis."""
    flat = scores.reshape(-1, scores.shape[-1])
    out = np.stack([topk_row(r, k) for r in flat]) if flat.shape[0] else np.zeros((0, k), np.int32)
    return out.reshape(scores.shape[:-1] + (k,))


# ---------------------------------------------------------------- step 4 ----
def attend(q: np.ndarray, keys: np.ndarray, values: np.ndarray, scale: float) -> np.ndarray:
    """softmax(scale * keys @ q) @ values in fp64, max-subtracted."""
    s = scale * (np.asarray(keys, np.float64) @ np.asarray(q, np.float64))
    e = np.exp(s - np.max(s))
    return (e / np.sum(e)) @ np.asarray(values, np.float64)


def selected_keys(idx_row: np.ndarray, p: int, block: int = 64) -> np.ndarray:
    """Token positions a query at position p attends: the union of the selected
    blocks, restricted to positions <= p ([P1]: attend only to the kept blocks;
    causal). -1 entries are padding."""
    toks = [np.arange(block * b, block * b + block) for b in sorted(set(int(x) for x in idx_row)) if b >= 0]
    if not toks:
        return np.zeros(0, dtype=np.int64)
    toks = np.concatenate(toks)
    return toks[toks <= p]


def block_sparse_attention(Q: np.ndarray, K: np.ndarray, V: np.ndarray, idx: np.ndarray, q_start: int,
                           scale: float, block: int = 64, tile: int = 64) -> np.ndarray:
    """GQA block-sparse attention: every query head of a group attends, with
    its own query, over the blocks selected for its KV head and query tile
    ([P1]: layer L+1's own queries run sparse attention over the blocks chosen
    for it; [P3] 解法).

    Q [B, Hq, Tq, d]; K, V [B, Hkv, T, d]; idx [B, Hkv, nTiles, k].
    Returns O [B, Hq, Tq, d]. A query with no key gets zeros.
    """
    B, Hq, Tq, d = Q.shape
    Hkv = K.shape[1]
    G = Hq // Hkv
    out = np.zeros((B, Hq, Tq, d))
    for b in range(B):
        for qh in range(Hq):
            h = qh // G
            for i in range(Tq):
                p = q_start + i
                J = selected_keys(idx[b, h, i // tile], p, block)
                if J.size:
                    out[b, qh, i] = attend(Q[b, qh, i], K[b, h, J], V[b, h, J], scale)
    return out


def dense_causal_attention(Q: np.ndarray, K: np.ndarray, V: np.ndarray, q_start: int, scale: float) -> np.ndarray:
    """Textbook dense causal GQA attention: query i at position q_start + i
    attends every key at or before it."""
    B, Hq, Tq, d = Q.shape
    Hkv = K.shape[1]
    G = Hq // Hkv
    out = np.zeros((B, Hq, Tq, d))
    for b in range(B):
        for qh in range(Hq):
            h = qh // G
            for i in range(Tq):
                p = q_start + i
                out[b, qh, i] = attend(Q[b, qh, i], K[b, h, : p + 1], V[b, h, : p + 1], scale)
    return out


# -------------------------------------------------------- step 5 (offload) ----
def gather_blocks(kv: np.ndarray, idx: np.ndarray, block: int = 64) -> np.ndarray:
    """Bit copy of the selected blocks into a staging array ([P1]/[P2] 二: the
    blocks the Forecast picks for the next layer are fetched from CPU memory
    to the GPU ahead of use).

    kv [B, Hkv, T, d] (any dtype) and idx [B, Hkv, k] -> [B, Hkv, k, block, d];
    slot j holds block idx[..., j]; -1 slots are left zero.
    """
    B, Hkv, T, d = kv.shape
    k = idx.shape[-1]
    out = np.zeros((B, Hkv, k, block, d), dtype=kv.dtype)
    for b in range(B):
        for h in range(Hkv):
            for j in range(k):
                beta = int(idx[b, h, j])
                if beta >= 0:
                    out[b, h, j] = kv[b, h, block * beta: block * beta + block]
    return out


def lookahead_decode_step(layer0: dict, layer1: dict, T: int, k: int, scale: float,
                          block: int = 64, kernel: int = 32, stride: int = 16):
    """One decode step of two layers with lookahead selection ([P1]: layer L's
    Forecast predicts the blocks layer L+1 needs; [P2] 三: layer 0 keeps its KV
    on the GPU and selects with a same-layer forecast).

    layerN dicts hold fp64 arrays: 'Q' [B,Hq,1,d], 'K','V' [B,Hkv,T,d],
    'Kc' [B,Hkv,W,d]; layer0 also 'F_self' and 'F_next' [B,Hkv,1,d].
    Returns (O0, O1, idx0, idx1).
    """
    q_start = T - 1
    s0 = select_forecast(layer0["F_self"], layer0["Kc"], T, q_start, scale, block, kernel, stride)
    idx0 = topk_blocks(s0, k)
    s1 = select_forecast(layer0["F_next"], layer1["Kc"], T, q_start, scale, block, kernel, stride)
    idx1 = topk_blocks(s1, k)
    O0 = block_sparse_attention(layer0["Q"], layer0["K"], layer0["V"], idx0, q_start, scale, block)
    O1 = block_sparse_attention(layer1["Q"], layer1["K"], layer1["V"], idx1, q_start, scale, block)
    return O0, O1, idx0, idx1


# ------------------------------------------ upstream: the four projections ----
def project_qkvf(x: np.ndarray, w: np.ndarray, Hq: int, Hkv: int, n_f: int, d: int = 128):
    """The projections a layer emits for one token per sequence: Q, K, V and
    the Forecast vector ([P1] paragraph on the four projections per layer;
    [P1] abstract: the Forecast is a fourth projection beside Query, Key and
    Value; [P2] 二). The weights of all four are one matrix whose rows are
    ordered [Hq query heads | Hkv key heads | Hkv value heads | n_f sets of
    Hkv Forecast heads], d rows per head (n_f = 2 for the first layer, whose
    extra set is its same-layer Forecast, [P2] 三).

    x [B, D], w [(Hq + 2 Hkv + n_f Hkv) d, D] -> q [B, Hq, 1, d],
    k and v [B, Hkv, 1, d], f [n_f, B, Hkv, 1, d] (None when n_f = 0).
    """
    B, D = x.shape
    assert w.shape == ((Hq + 2 * Hkv + n_f * Hkv) * d, D)
    y = np.asarray(x, dtype=np.float64) @ np.asarray(w, dtype=np.float64).T  # [B, N]
    heads = y.reshape(B, Hq + 2 * Hkv + n_f * Hkv, d)
    q = heads[:, :Hq].reshape(B, Hq, 1, d)
    k = heads[:, Hq:Hq + Hkv].reshape(B, Hkv, 1, d)
    v = heads[:, Hq + Hkv:Hq + 2 * Hkv].reshape(B, Hkv, 1, d)
    f = None
    if n_f:
        f = heads[:, Hq + 2 * Hkv:].reshape(B, n_f, Hkv, 1, d).transpose(1, 0, 2, 3, 4).copy()
    return q, k, v, f


# ------------------------------------------- token-level Forecast (variant) ----
# [P2] 六 names, as future work for models with token-level sparse attention,
# a forecaster that predicts importance scores per key token instead of per
# block; [P1] compares the method with DSA, whose small indexer picks the
# important tokens in place of the queries. The pages define neither the keys
# such a forecaster reads nor how many tokens it keeps. Reading taken: the
# layer's Forecast vector scores every visible key token directly (no
# compression, no pooling), the same top-k rule keeps the best k_tok tokens,
# and attention runs over exactly those tokens.
def _positions(B: int, q_start: int, positions) -> list[int]:
    return [int(q_start)] * B if positions is None else [int(x) for x in positions]


def forecast_token_scores(F: np.ndarray, K: np.ndarray, q_start: int, scale: float, positions=None) -> np.ndarray:
    """Decode-time token scores s[t] = scale * f . K[t] for every key token
    t <= p, -inf after p (the query's own position bounds what it may see).

    F [B, Hkv, 1, d]; K [B, Hkv, T, d] -> [B, Hkv, 1, T]. ``positions`` gives
    each sequence's query position (default q_start for all)."""
    B, Hkv, Tq, d = F.shape
    assert Tq == 1
    T = K.shape[2]
    pos = _positions(B, q_start, positions)
    out = np.full((B, Hkv, 1, T), NEG_INF)
    for b in range(B):
        p = min(pos[b], T - 1)
        if p < 0:
            continue
        for h in range(Hkv):
            out[b, h, 0, : p + 1] = scale * (np.asarray(K[b, h, : p + 1], np.float64) @ np.asarray(F[b, h, 0], np.float64))
    return out


def token_sparse_attention(Q: np.ndarray, K: np.ndarray, V: np.ndarray, tok_idx: np.ndarray, q_start: int,
                           scale: float, positions=None) -> np.ndarray:
    """GQA attention at decode over the selected key tokens only: every query
    head of a group attends, with its own query, over the tokens kept for its
    KV head, restricted to positions <= p; -1 entries are padding, and a query
    with no key gets zeros.

    Q [B, Hq, 1, d]; K, V [B, Hkv, T, d]; tok_idx [B, Hkv, 1, k_tok]."""
    B, Hq, Tq, d = Q.shape
    assert Tq == 1
    Hkv = K.shape[1]
    G = Hq // Hkv
    pos = _positions(B, q_start, positions)
    out = np.zeros((B, Hq, 1, d))
    for b in range(B):
        for qh in range(Hq):
            h = qh // G
            J = np.array(sorted(set(int(t) for t in tok_idx[b, h, 0] if 0 <= t <= pos[b])), dtype=np.int64)
            if J.size:
                out[b, qh, 0] = attend(Q[b, qh, 0], K[b, h, J], V[b, h, J], scale)
    return out
