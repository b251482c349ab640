"""Pins for the fp64 oracle: closed forms, hand-worked fixtures, brute force and
library routines, each independent of the oracle's own code. CPU only.

Each test names the step it pins; a plausible slip in the oracle (a dropped
window, an off-by-one in visibility or block overlap, softmax over the wrong
axis, a transposed GQA mapping, a tie broken the wrong way, a non-causal key)
fails at least one of them.
"""

import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


# ------------------------------------------------------------ compression ----
def test_compress_ramp_closed_form():
    g = golden("compress_ramp.json")
    T, d = g["T"], 5
    K = np.zeros((1, 1, T, d))
    K[0, 0, :, 0] = np.arange(T)
    kc = oracle.compress_keys(K, g["kernel"], g["stride"])
    assert kc.shape == (1, 1, g["windows"], d)
    np.testing.assert_array_equal(kc[0, 0, :, 0], g["first_component"])
    np.testing.assert_array_equal(kc[0, 0, :, 1:], 0.0)


def test_compress_constant_and_window_count():
    for T in (32, 48, 64, 4096):
        K = np.full((2, 3, T, 4), 0.375)
        kc = oracle.compress_keys(K)
        assert kc.shape[2] == (T - 32) // 16 + 1
        np.testing.assert_array_equal(kc, 0.375)
    assert oracle.num_windows(4096) == 255
    assert oracle.num_windows(32768) == 2047
    assert oracle.num_windows(131072) == 8191


def test_compress_matches_prefix_sum_brute_force():
    rng = np.random.default_rng(1)
    K = rng.integers(-8, 9, size=(2, 2, 256, 8)).astype(np.float64)
    kc = oracle.compress_keys(K)
    # independent route: integer prefix sums, exact
    c = np.concatenate([np.zeros((2, 2, 1, 8)), np.cumsum(K, axis=2)], axis=2)
    W = (256 - 32) // 16 + 1
    ref = np.stack([(c[:, :, 16 * w + 32] - c[:, :, 16 * w]) / 32 for w in range(W)], axis=2)
    np.testing.assert_array_equal(kc, ref)


# ------------------------------------------------- visibility and overlap ----
def test_visible_window_count_brute_force():
    W = oracle.num_windows(1024)
    for p in range(0, 1024):
        n = 0
        while n < W and 16 * n + 31 <= p:  # window n holds tokens 16n..16n+31
            n += 1
        assert oracle.visible_window_count(p, W) == n
    assert oracle.visible_window_count(30, W) == 0
    assert oracle.visible_window_count(31, W) == 1
    assert oracle.visible_window_count(1023, W) == W


def test_block_window_ranges_brute_force_and_closed_form():
    for (T, block, kernel, stride) in [(1024, 64, 32, 16), (512, 32, 16, 8), (256, 64, 32, 32), (640, 64, 48, 16)]:
        lo, hi = oracle.block_window_ranges(T, block, kernel, stride)
        W = (T - kernel) // stride + 1
        for beta in range(T // block):
            meet = [w for w in range(W)
                    if set(range(stride * w, stride * w + kernel)) & set(range(block * beta, block * beta + block))]
            assert (lo[beta], hi[beta]) == (meet[0], meet[-1])
    lo, hi = oracle.block_window_ranges(131072)
    beta = np.arange(2048)
    np.testing.assert_array_equal(lo, np.maximum(0, 4 * beta - 1))
    np.testing.assert_array_equal(hi, np.minimum(8190, 4 * beta + 3))


def test_pool_single_spike_lands_in_overlapping_blocks_only():
    T = 1024
    W = oracle.num_windows(T)
    lo, hi = oracle.block_window_ranges(T)
    for wstar in range(W):
        s = np.zeros(W)
        s[wstar] = 7.0
        out = oracle.pool_windows_to_blocks(s, W, lo, hi)
        hit = set(np.nonzero(out == 7.0)[0].tolist())
        # window w spans tokens [16w, 16w+32): blocks floor(16w/64) .. floor((16w+31)/64)
        assert hit == set(range((16 * wstar) // 64, (16 * wstar + 31) // 64 + 1))
        assert np.all(out[list(set(range(T // 64)) - hit)] == 0.0)


def test_pool_respects_visibility():
    T = 1024
    W = oracle.num_windows(T)
    lo, hi = oracle.block_window_ranges(T)
    s = np.arange(W, dtype=np.float64)
    for p in (31, 100, 500, 1023):
        n = oracle.visible_window_count(p, W)
        out = oracle.pool_windows_to_blocks(s, n, lo, hi)
        for beta in range(T // 64):
            vis = [w for w in range(lo[beta], hi[beta] + 1) if 16 * w + 31 <= p]
            assert out[beta] == (max(vis) if vis else -np.inf)


# -------------------------------------------------------------- scoring -----
def test_forecast_scores_exact_integers():
    rng = np.random.default_rng(2)
    f = rng.integers(-5, 6, size=16)
    kc = rng.integers(-5, 6, size=(40, 16))
    s = oracle.forecast_window_scores(f.astype(float), kc.astype(float), 1.0)
    ref = [sum(int(a) * int(b) for a, b in zip(f, row)) for row in kc]
    np.testing.assert_array_equal(s, ref)
    s2 = oracle.forecast_window_scores(f.astype(float), kc.astype(float), 0.25)
    np.testing.assert_array_equal(s2, np.array(ref) * 0.25)


def test_multihead_hand_summed_softmax():
    g = golden("multihead_group_sum.json")
    logits = np.array(g["logits"])
    G, W = logits.shape
    # logits = q_g . kc_w with kc = identity rows, q_g = logits row
    kc = np.eye(W)
    S = oracle.multihead_window_scores(logits, kc, 1.0, W)
    want = [x / g["group_sum_den"] for x in g["group_sum_num"]]
    np.testing.assert_allclose(S, want, rtol=1e-15)


def test_multihead_equal_logits_and_mass():
    rng = np.random.default_rng(3)
    for G in (1, 2, 4, 8):
        kc = np.ones((50, 4))
        q = np.ones((G, 4))
        for nv in (1, 7, 50):
            S = oracle.multihead_window_scores(q, kc, 0.5, nv)
            np.testing.assert_allclose(S[:nv], G / nv, rtol=1e-14)
            assert np.all(np.isneginf(S[nv:]))
        q = rng.standard_normal((G, 4))
        kc = rng.standard_normal((50, 4))
        S = oracle.multihead_window_scores(q, kc, 0.7, 33)
        assert abs(S[:33].sum() - G) < 1e-12  # each head's softmax has unit mass


def test_multihead_matches_torch_softmax():
    rng = np.random.default_rng(4)
    q = rng.standard_normal((4, 16))
    kc = rng.standard_normal((60, 16))
    nv = 45
    logits = torch.from_numpy(q) @ torch.from_numpy(kc[:nv]).T * 0.3
    ref = torch.softmax(logits, dim=1).sum(0).numpy()
    S = oracle.multihead_window_scores(q, kc, 0.3, nv)
    np.testing.assert_allclose(S[:nv], ref, rtol=1e-13)


def test_selector_link_single_head_same_topk():
    # one head: softmax is monotone, so the multi-head selector with G = 1 and
    # Q = F ranks blocks exactly as the Forecast selector does
    rng = np.random.default_rng(5)
    T, d = 2048, 16
    F = rng.standard_normal((2, 3, 1, d))
    Kc = rng.standard_normal((2, 3, oracle.num_windows(T), d))
    sf = oracle.select_forecast(F, Kc, T, T - 1, 0.25)
    sm = oracle.select_multihead(F, Kc, T, T - 1, 0.25)
    np.testing.assert_array_equal(oracle.topk_blocks(sf, 7), oracle.topk_blocks(sm, 7))
    assert not np.array_equal(sf, sm)


def test_select_gqa_group_mapping():
    # head q must belong to KV head q // G: put a huge logit only in head 5's
    # query (group 1 of G = 4) aimed at window 40 -> only KV head 1's scores see it
    T, d, Hq, Hkv = 1024, 8, 8, 2
    W = oracle.num_windows(T)
    Kc = np.zeros((1, Hkv, W, d))
    Kc[0, :, 40, 0] = 1.0
    Q = np.zeros((1, Hq, 1, d))
    Q[0, 5, 0, 0] = 50.0
    s = oracle.select_multihead(Q, Kc, T, T - 1, 1.0)
    blocks_of_40 = {10}  # window 40 spans tokens 640..671 -> block 10
    assert set(np.argsort(-s[0, 1, 0])[:1].tolist()) == blocks_of_40
    assert np.allclose(s[0, 0, 0], s[0, 0, 0, 0])  # group 0 uniform


def test_prefill_tile_is_max_over_queries_with_causality():
    rng = np.random.default_rng(6)
    T, d = 512, 8
    W = oracle.num_windows(T)
    Kc = rng.standard_normal((1, 1, W, d))
    F = rng.standard_normal((1, 1, 128, d))
    q_start = T - 128
    s = oracle.select_forecast(F, Kc, T, q_start, 1.0)
    assert s.shape == (1, 1, 2, T // 64)
    for t in range(2):
        rows = []
        for i in range(64 * t, 64 * t + 64):
            p = q_start + i
            w = Kc[0, 0] @ F[0, 0, i]
            row = []
            for beta in range(T // 64):
                vis = [w[x] for x in range(W)
                       if 16 * x + 31 <= p and 16 * x < 64 * beta + 64 and 16 * x + 32 > 64 * beta]
                row.append(max(vis) if vis else -np.inf)
            rows.append(row)
        np.testing.assert_allclose(s[0, 0, t], np.max(rows, axis=0), rtol=1e-14)
    # the last tile ends at position T-1 and may see every block; the first ends at T-65
    assert np.isfinite(s[0, 0, 1]).all()
    assert np.isneginf(s[0, 0, 0, -1])


# ----------------------------------------------------------------- top-k ----
def test_topk_golden_ties():
    g = golden("topk_ties.json")
    for case in g["cases"]:
        sc = np.array([-np.inf if x == "-inf" else float(x) for x in case["scores"]])
        np.testing.assert_array_equal(oracle.topk_row(sc, case["k"]), case["idx"])


def test_topk_equals_full_sort_with_index_tiebreak():
    rng = np.random.default_rng(7)
    for _ in range(200):
        n = int(rng.integers(1, 300))
        k = int(rng.integers(1, 80))
        sc = rng.integers(-4, 5, size=n).astype(float)  # many exact ties
        sc[rng.random(n) < 0.1] = -np.inf
        cand = [b for b in range(n) if sc[b] != -np.inf]
        ranked = sorted(cand, key=lambda b: (-sc[b], b))
        want = sorted(ranked[:k]) + [-1] * max(0, k - len(cand))
        np.testing.assert_array_equal(oracle.topk_row(sc, k), want)


def test_topk_all_blocks_and_batch_shape():
    sc = np.random.default_rng(8).standard_normal((2, 3, 1, 64))
    idx = oracle.topk_blocks(sc, 64)
    assert idx.shape == (2, 3, 1, 64) and idx.dtype == np.int32
    np.testing.assert_array_equal(idx, np.broadcast_to(np.arange(64), idx.shape))


# ------------------------------------------------------------- attention ----
def _sdpa_reference(Q, K, V, q_start, scale):
    """torch CPU fp64 scaled_dot_product_attention with an explicit causal mask."""
    B, Hq, Tq, d = Q.shape
    Hkv, T = K.shape[1], K.shape[2]
    G = Hq // Hkv
    Kx = torch.from_numpy(np.repeat(K, G, axis=1))
    Vx = torch.from_numpy(np.repeat(V, G, axis=1))
    pos = q_start + torch.arange(Tq)[:, None]
    mask = torch.arange(T)[None, :] <= pos
    return torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(Q), Kx, Vx, attn_mask=mask, scale=scale).numpy()


@pytest.mark.parametrize("Tq,q_start", [(1, 1023), (64, 960), (128, 896), (128, 0)])
def test_dense_causal_matches_torch_sdpa(Tq, q_start):
    rng = np.random.default_rng(9)
    T = q_start + Tq
    Q = rng.standard_normal((2, 4, Tq, 16))
    K = rng.standard_normal((2, 2, T, 16))
    V = rng.standard_normal((2, 2, T, 16))
    ref = _sdpa_reference(Q, K, V, q_start, 0.25)
    np.testing.assert_allclose(oracle.dense_causal_attention(Q, K, V, q_start, 0.25), ref, rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("Tq,q_start", [(1, 1023), (64, 960), (128, 896), (128, 0), (192, 64)])
def test_sparse_with_all_blocks_equals_dense(Tq, q_start):
    rng = np.random.default_rng(10)
    T = q_start + Tq
    nB = T // 64
    Q = rng.standard_normal((1, 8, Tq, 16))
    K = rng.standard_normal((1, 2, T, 16))
    V = rng.standard_normal((1, 2, T, 16))
    n_tiles = -(-Tq // 64)
    idx = np.broadcast_to(np.arange(nB, dtype=np.int32), (1, 2, n_tiles, nB)).copy()
    out = oracle.block_sparse_attention(Q, K, V, idx, q_start, 0.3)
    np.testing.assert_allclose(out, _sdpa_reference(Q, K, V, q_start, 0.3), rtol=1e-12, atol=1e-12)


def test_attention_golden_two_keys():
    g = golden("attention_two_keys.json")
    o = oracle.attend(np.array(g["q"]), np.array(g["k"]), np.array(g["v"]), 1.0)
    np.testing.assert_allclose(o, g["o"], rtol=1e-14)


def test_attention_invariants():
    rng = np.random.default_rng(11)
    T, d = 1024, 16
    Q = rng.standard_normal((1, 4, 1, d))
    K = rng.standard_normal((1, 1, T, d))
    V = np.broadcast_to(rng.standard_normal(d), (1, 1, T, d)).copy()
    idx = np.array([[[[3, 7, 11, 15]]]], dtype=np.int32)
    out = oracle.block_sparse_attention(Q, K, V, idx, T - 1, 0.25)
    np.testing.assert_allclose(out[0, :, 0], np.broadcast_to(V[0, 0, 0], (4, d)), rtol=1e-13)  # constant V
    V = rng.standard_normal((1, 1, T, d))
    a = oracle.block_sparse_attention(Q, K, V, idx, T - 1, 0.25)
    b = oracle.block_sparse_attention(Q, K, V, idx[..., ::-1].copy(), T - 1, 0.25)
    np.testing.assert_array_equal(a, b)  # order of idx does not matter
    # exactly the selected tokens matter: perturb keys outside them
    K2 = K.copy()
    K2[0, 0, :192] += 100.0
    np.testing.assert_array_equal(oracle.block_sparse_attention(Q, K2, V, idx, T - 1, 0.25), a)
    # padding -1 ignored
    idxp = np.array([[[[3, -1, 7, 11, -1, 15]]]], dtype=np.int32)
    np.testing.assert_array_equal(oracle.block_sparse_attention(Q, K, V, idxp, T - 1, 0.25), a)


def test_attention_single_visible_key():
    # prefill query at position 64*5 with only block 5 selected sees exactly one key
    rng = np.random.default_rng(12)
    T, d = 384, 8
    Q = rng.standard_normal((1, 1, 64, d))
    K = rng.standard_normal((1, 1, T, d))
    V = rng.standard_normal((1, 1, T, d))
    idx = np.array([[[[5]]]], dtype=np.int32)
    out = oracle.block_sparse_attention(Q, K, V, idx, 320, 1.0)
    np.testing.assert_array_equal(out[0, 0, 0], V[0, 0, 320])
    np.testing.assert_allclose(out[0, 0, 63], oracle.attend(Q[0, 0, 63], K[0, 0, 320:384], V[0, 0, 320:384], 1.0))


# ---------------------------------------------------------------- gather ----
def test_gather_is_bit_copy():
    rng = np.random.default_rng(13)
    kv = rng.integers(0, 65535, size=(2, 3, 1024, 8), dtype=np.uint16)
    idx = np.stack([np.stack([rng.choice(16, 5, replace=False) for _ in range(3)]) for _ in range(2)]).astype(np.int32)
    idx[1, 2, 4] = -1
    st = oracle.gather_blocks(kv, idx)
    blocks = kv.reshape(2, 3, 16, 64, 8)
    for b in range(2):
        for h in range(3):
            for j in range(5):
                if idx[b, h, j] >= 0:
                    assert st[b, h, j].tobytes() == blocks[b, h, idx[b, h, j]].tobytes()
                else:
                    assert not st[b, h, j].any()


def test_lookahead_step_structure():
    rng = np.random.default_rng(14)
    T, d, k = 1024, 8, 4
    W = oracle.num_windows(T)
    L = {n: rng.standard_normal(s) for n, s in
         [("Q", (1, 4, 1, d)), ("K", (1, 1, T, d)), ("V", (1, 1, T, d)), ("F_self", (1, 1, 1, d))]}
    L["Kc"] = oracle.compress_keys(L["K"])
    L["F_next"] = L["F_self"]
    O0, O1, i0, i1 = oracle.lookahead_decode_step(L, dict(L), T, k, 0.3)
    np.testing.assert_array_equal(O0, O1)
    np.testing.assert_array_equal(i0, i1)
    # layer 1 attends with its own Q over the blocks layer 0's Forecast chose
    L1 = {**L, "Q": rng.standard_normal((1, 4, 1, d))}
    _, O1b, _, i1b = oracle.lookahead_decode_step(L, L1, T, k, 0.3)
    np.testing.assert_array_equal(i1b, i0)
    np.testing.assert_allclose(O1b, oracle.block_sparse_attention(L1["Q"], L["K"], L["V"], i0, T - 1, 0.3))
    assert W == 63


def test_lookahead_step_layer_wiring():
    """Which Forecast scores which layer's compressed keys, and which layer's
    queries attend over which layer's K and V, with every input distinct.
    The compressed keys are spikes: window 4b + 1 lies inside block b alone
    (tokens 64b + 16 .. 64b + 47), so a Forecast along e0 or e1 picks exactly
    the blocks holding its spikes. Expected indices are written by hand:

      Kc0: e0 spikes at blocks 3 (10) and 7 (5); e1 spikes at blocks 5 (10) and 12 (5)
      Kc1: e0 spikes at blocks 9 (10) and 2 (5); e1 spikes at blocks 11 (10) and 14 (5)
      F_self = e0 (layer 0's own blocks), F_next = e1 (layer 1's blocks)

    so idx0 = [3, 7] and idx1 = [11, 14]. Swapping F_self and F_next gives
    [5, 12] and [2, 9]; scoring the other layer's Kc gives [2, 9] and [5, 12];
    every such swap fails here. The outputs are the textbook softmax of each
    layer's own queries over its own keys of those blocks; swapping Q, K or V
    between the layers changes them."""
    rng = np.random.default_rng(41)
    T, d, k, G = 1024, 8, 2, 2
    W = oracle.num_windows(T)
    e0, e1 = np.eye(d)[0], np.eye(d)[1]

    def spikes(pairs):
        kc = np.zeros((1, 1, W, d))
        for vec, blk, mag in pairs:
            kc[0, 0, 4 * blk + 1] = mag * vec
        return kc

    L0 = {"Q": rng.standard_normal((1, G, 1, d)), "K": rng.standard_normal((1, 1, T, d)),
          "V": rng.standard_normal((1, 1, T, d)),
          "Kc": spikes([(e0, 3, 10.0), (e0, 7, 5.0), (e1, 5, 10.0), (e1, 12, 5.0)]),
          "F_self": e0.reshape(1, 1, 1, d).copy(), "F_next": e1.reshape(1, 1, 1, d).copy()}
    L1 = {"Q": rng.standard_normal((1, G, 1, d)), "K": rng.standard_normal((1, 1, T, d)) + 1.0,
          "V": rng.standard_normal((1, 1, T, d)) - 1.0,
          "Kc": spikes([(e0, 9, 10.0), (e0, 2, 5.0), (e1, 11, 10.0), (e1, 14, 5.0)])}
    O0, O1, idx0, idx1 = oracle.lookahead_decode_step(L0, L1, T, k, 0.5)
    assert idx0.tolist() == [[[[3, 7]]]]
    assert idx1.tolist() == [[[[11, 14]]]]

    def softmax_attend(q, K, V, blocks):
        toks = np.concatenate([np.arange(64 * b, 64 * b + 64) for b in blocks])
        s = 0.5 * np.array([sum(q[c] * K[t, c] for c in range(d)) for t in toks])
        e = np.exp(s - s.max())
        return (e[:, None] * V[toks]).sum(axis=0) / e.sum()

    for g in range(G):
        np.testing.assert_allclose(O0[0, g, 0], softmax_attend(L0["Q"][0, g, 0], L0["K"][0, 0], L0["V"][0, 0], [3, 7]),
                                   rtol=1e-12, atol=1e-12)
        np.testing.assert_allclose(O1[0, g, 0],
                                   softmax_attend(L1["Q"][0, g, 0], L1["K"][0, 0], L1["V"][0, 0], [11, 14]),
                                   rtol=1e-12, atol=1e-12)


# ------------------------------------------------ the four projections ----
def test_project_qkvf_brute_force_and_layout():
    """Every output element as a pure-Python sum over D, read back at the
    position the weight-row order fixes (query heads, key heads, value heads,
    then the Forecast sets), with small integers so the sums are exact."""
    rng = np.random.default_rng(21)
    B, D, Hq, Hkv, n_f, d = 3, 8, 4, 2, 2, 4
    N = (Hq + 2 * Hkv + n_f * Hkv) * d
    x = rng.integers(-4, 5, size=(B, D)).astype(np.float64)
    w = rng.integers(-4, 5, size=(N, D)).astype(np.float64)
    q, k, v, f = oracle.project_qkvf(x, w, Hq, Hkv, n_f, d)
    assert q.shape == (B, Hq, 1, d) and k.shape == (B, Hkv, 1, d) and v.shape == (B, Hkv, 1, d)
    assert f.shape == (n_f, B, Hkv, 1, d)

    def y(b, n):
        return sum(float(x[b, c]) * float(w[n, c]) for c in range(D))

    for b in range(B):
        for c in range(d):
            for h in range(Hq):
                assert q[b, h, 0, c] == y(b, h * d + c)
            for h in range(Hkv):
                assert k[b, h, 0, c] == y(b, (Hq + h) * d + c)
                assert v[b, h, 0, c] == y(b, (Hq + Hkv + h) * d + c)
                for s in range(n_f):
                    assert f[s, b, h, 0, c] == y(b, (Hq + 2 * Hkv + s * Hkv + h) * d + c)


def test_project_qkvf_unit_rows_pick_inputs():
    """Weight rows that are unit vectors copy one input channel each: row n =
    e_perm[n] gives output n = x[:, perm[n]] exactly; and n_f = 0 has no
    Forecast output."""
    rng = np.random.default_rng(22)
    B, D, Hq, Hkv, d = 2, 64, 2, 1, 8
    for n_f in (0, 1):
        N = (Hq + 2 * Hkv + n_f * Hkv) * d
        perm = rng.integers(0, D, size=N)
        w = np.zeros((N, D))
        w[np.arange(N), perm] = 1.0
        x = rng.standard_normal((B, D))
        q, k, v, f = oracle.project_qkvf(x, w, Hq, Hkv, n_f, d)
        flat = np.concatenate([q.reshape(B, -1), k.reshape(B, -1), v.reshape(B, -1)]
                              + ([f.transpose(1, 0, 2, 3, 4).reshape(B, -1)] if n_f else []), axis=1)
        np.testing.assert_array_equal(flat, x[:, perm])
        assert (f is None) == (n_f == 0)


# ---- token-level Forecast variant -------------------------------------------
def test_token_scores_ramp_closed_form():
    # K[t] = t e_0 and f = e_0: the score of token t is scale * t up to the
    # query's position and -inf after it
    T, d, p = 40, 128, 30
    K = np.zeros((1, 1, T, d))
    K[0, 0, :, 0] = np.arange(T)
    F = np.zeros((1, 1, 1, d))
    F[0, 0, 0, 0] = 1.0
    s = oracle.forecast_token_scores(F, K, p, 0.5)
    assert np.array_equal(s[0, 0, 0, : p + 1], 0.5 * np.arange(p + 1))
    assert np.all(s[0, 0, 0, p + 1:] == -np.inf)


def test_token_scores_brute_force():
    rng = np.random.default_rng(11)
    B, Hkv, T, d = 2, 3, 24, 128
    K = rng.standard_normal((B, Hkv, T, d))
    F = rng.standard_normal((B, Hkv, 1, d))
    pos = [17, 5]
    s = oracle.forecast_token_scores(F, K, 0, 0.25, positions=pos)
    for b in range(B):
        for h in range(Hkv):
            for t in range(T):
                want = 0.25 * math.fsum(F[b, h, 0, c] * K[b, h, t, c] for c in range(d)) if t <= pos[b] else -np.inf
                assert s[b, h, 0, t] == pytest.approx(want, rel=1e-12, abs=1e-12)


def test_token_scores_nothing_visible():
    s = oracle.forecast_token_scores(np.ones((1, 2, 1, 128)), np.ones((1, 2, 8, 128)), 0, 1.0, positions=[-1])
    assert np.all(s == -np.inf)


def test_token_topk_keeps_every_visible_token():
    rng = np.random.default_rng(12)
    K = rng.standard_normal((1, 1, 50, 128))
    F = rng.standard_normal((1, 1, 1, 128))
    s = oracle.forecast_token_scores(F, K, 20, 1.0)
    idx = oracle.topk_blocks(s, 30)
    assert np.array_equal(idx[0, 0, 0, :21], np.arange(21))
    assert np.all(idx[0, 0, 0, 21:] == -1)


def test_token_attention_all_tokens_is_dense_causal():
    rng = np.random.default_rng(13)
    B, Hq, Hkv, T, d = 2, 4, 2, 70, 128
    Q = rng.standard_normal((B, Hq, 1, d))
    K = rng.standard_normal((B, Hkv, T, d))
    V = rng.standard_normal((B, Hkv, T, d))
    p = 52
    idx = np.broadcast_to(np.arange(T, dtype=np.int32), (B, Hkv, 1, T))  # tokens after p are ignored
    got = oracle.token_sparse_attention(Q, K, V, idx, p, 0.1)
    want = oracle.dense_causal_attention(Q, K[:, :, : p + 1], V[:, :, : p + 1], p, 0.1)
    assert np.allclose(got, want, rtol=1e-12, atol=1e-12)


def test_token_attention_equals_block_attention_on_the_same_tokens():
    rng = np.random.default_rng(14)
    B, Hq, Hkv, T, d = 1, 4, 2, 256, 128
    Q = rng.standard_normal((B, Hq, 1, d))
    K = rng.standard_normal((B, Hkv, T, d))
    V = rng.standard_normal((B, Hkv, T, d))
    blocks = np.array([[[[3, 0, -1]]], [[[1, 2, -1]]]], dtype=np.int32).reshape(B, Hkv, 1, 3)
    tok = np.full((B, Hkv, 1, 3 * 64), -1, dtype=np.int32)
    for h in range(Hkv):
        toks = np.concatenate([np.arange(64 * b, 64 * b + 64) for b in blocks[0, h, 0] if b >= 0])
        tok[0, h, 0, : toks.size] = toks[::-1]  # any order
    p = T - 30
    got = oracle.token_sparse_attention(Q, K, V, tok, p, 0.2)
    want = oracle.block_sparse_attention(Q, K, V, blocks, p, 0.2)
    assert np.allclose(got, want, rtol=1e-12, atol=1e-12)


def test_token_attention_single_token_and_empty():
    rng = np.random.default_rng(15)
    Q = rng.standard_normal((1, 2, 1, 128))
    K = rng.standard_normal((1, 1, 16, 128))
    V = rng.standard_normal((1, 1, 16, 128))
    one = np.array([-1, 9, -1], dtype=np.int32).reshape(1, 1, 1, 3)
    got = oracle.token_sparse_attention(Q, K, V, one, 15, 1.0)
    assert np.array_equal(got[0, 0, 0], V[0, 0, 9]) and np.array_equal(got[0, 1, 0], V[0, 0, 9])
    none = np.full((1, 1, 1, 3), -1, dtype=np.int32)
    assert np.all(oracle.token_sparse_attention(Q, K, V, none, 15, 1.0) == 0)
    # a token after the query's position is not visible
    late = np.array([12, -1, -1], dtype=np.int32).reshape(1, 1, 1, 3)
    assert np.all(oracle.token_sparse_attention(Q, K, V, late, 10, 1.0) == 0)
