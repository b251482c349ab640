"""GPU parity of the prefill path (a chunk of queries, 64-query tiles):
Forecast scoring on the matrix cores, top-k per tile, and block-sparse
attention on the matrix cores, against the fp64 oracle through the C ABI."""

import numpy as np
import pytest
import torch

import oracle
import synth.gpu as sg
from synth import workloads as wl
from tests import parity

pytestmark = pytest.mark.gpu
DEV = "cuda"


def say(*a):
    print(*a, flush=True)


def prefill(T, Tq, B=1, Hq=8, Hkv=2, k=5, seed=21, offsets=True):
    return wl.Workload(name="prefill", description="prefill", dtype="bf16", B=B, Hq=Hq, Hkv=Hkv, T=T, d=128, Tq=Tq,
                       q_start=T - Tq, k=k, seed=seed, block_offsets=offsets)


def gen(w, name):
    return sg.tensor(w.recipe(name), w.shape(name), DEV)


CASES = [prefill(64 * 37, 128), prefill(64 * 37, 64 * 37, k=7), prefill(2048, 64, B=2), prefill(4096, 1024, k=16),
         # five 256-window chunks of the scoring sweep, the last one partial,
         # and an odd tile count (the last workgroup's second tile is empty)
         prefill(64 * 258, 320, B=2, k=9)]


@pytest.mark.parametrize("w", CASES, ids=lambda w: f"T{w.T}-Tq{w.Tq}-B{w.B}")
def test_select_forecast_prefill_parity(gpu, w):
    say("prefill select", w.T, w.Tq)
    K, F = gen(w, "K"), gen(w, "F")
    Kc = gpu.compress_keys(K)
    s = gpu.select_forecast(F, Kc, w.T, w.q_start)
    torch.cuda.synchronize()
    assert s.shape == (w.B, w.Hkv, w.n_tiles, w.nB)
    ref = oracle.select_forecast(parity.to_f64(F), parity.to_f64(Kc), w.T, w.q_start, w.scale)
    worst = parity.check_scores(parity.to_f64(s), ref)
    idx = gpu.topk_blocks(s, w.k)
    banded = parity.check_topk_band(idx.cpu().numpy(), ref, w.k)
    say(f"  worst rel err {worst:.2e}, banded rows {banded}")


@pytest.mark.parametrize("w", CASES, ids=lambda w: f"T{w.T}-Tq{w.Tq}-B{w.B}")
def test_select_multihead_prefill_parity(gpu, w):
    say("prefill multihead select", w.T, w.Tq)
    Q, K = gen(w, "Q"), gen(w, "K")
    Kc = gpu.compress_keys(K)
    s = gpu.select_multihead(Q, Kc, w.T, w.q_start)
    torch.cuda.synchronize()
    assert s.shape == (w.B, w.Hkv, w.n_tiles, w.nB)
    ref = oracle.select_multihead(parity.to_f64(Q), parity.to_f64(Kc), w.T, w.q_start, w.scale)
    worst = parity.check_scores(parity.to_f64(s), ref)
    banded = parity.check_topk_band(gpu.topk_blocks(s, w.k).cpu().numpy(), ref, w.k)
    say(f"  worst rel err {worst:.2e}, banded rows {banded}")


@pytest.mark.parametrize("scale", [-0.07, 0.0, 0.3])
def test_prefill_selectors_any_scale(gpu, scale):
    """Both prefill selectors with a negative, a zero and a large scale (the
    Forecast kernel takes the max of the raw products only when the scale is
    positive; at zero every visible window ties), over 319 windows: one whole
    256-window chunk from the scalar-base loads and a partial one."""
    w = prefill(64 * 80, 256, k=9, seed=71)
    say("prefill selectors, scale", scale)
    Q, F, K = gen(w, "Q"), gen(w, "F"), gen(w, "K")
    Kc = gpu.compress_keys(K)
    s = gpu.select_forecast(F, Kc, w.T, w.q_start, scale=scale)
    m = gpu.select_multihead(Q, Kc, w.T, w.q_start, scale=scale)
    torch.cuda.synchronize()
    ref = oracle.select_forecast(parity.to_f64(F), parity.to_f64(Kc), w.T, w.q_start, scale)
    worst = parity.check_scores(parity.to_f64(s), ref)
    parity.check_topk_band(gpu.topk_blocks(s, w.k).cpu().numpy(), ref, w.k)
    ref_m = oracle.select_multihead(parity.to_f64(Q), parity.to_f64(Kc), w.T, w.q_start, scale)
    worst_m = parity.check_scores(parity.to_f64(m), ref_m)
    parity.check_topk_band(gpu.topk_blocks(m, w.k).cpu().numpy(), ref_m, w.k)
    say(f"  worst rel err {worst:.2e} / {worst_m:.2e}")


@pytest.mark.parametrize("G", [1, 2, 8])
def test_select_multihead_prefill_groups(gpu, G):
    """Every group size; 5 tiles, so the workgroups that hold several tiles
    (G < 4) end with a partial one."""
    w = prefill(64 * 21, 320, Hq=2 * G, k=4, seed=50 + G)
    say("prefill multihead select G", G)
    Q, K = gen(w, "Q"), gen(w, "K")
    Kc = gpu.compress_keys(K)
    s = gpu.select_multihead(Q, Kc, w.T, w.q_start)
    torch.cuda.synchronize()
    ref = oracle.select_multihead(parity.to_f64(Q), parity.to_f64(Kc), w.T, w.q_start, w.scale)
    worst = parity.check_scores(parity.to_f64(s), ref)
    parity.check_topk_band(gpu.topk_blocks(s, w.k).cpu().numpy(), ref, w.k)
    say(f"  worst rel err {worst:.2e}")


def test_select_multihead_prefill_is_deterministic(gpu):
    w = prefill(4096, 1024, k=16, seed=61)
    Q, K = gen(w, "Q"), gen(w, "K")
    Kc = gpu.compress_keys(K)
    a = gpu.select_multihead(Q, Kc, w.T, w.q_start)
    b = gpu.select_multihead(Q, Kc, w.T, w.q_start)
    torch.cuda.synchronize()
    assert torch.equal(a, b)


@pytest.mark.parametrize("G", [1, 2, 4, 8])
@pytest.mark.parametrize("k", [1, 6])
def test_attention_prefill_parity(gpu, G, k):
    w = prefill(64 * 37, 192, Hq=2 * G, k=k, seed=30 + G)
    say("prefill attention G", G, "k", k)
    Q, K, V = gen(w, "Q"), gen(w, "K"), gen(w, "V")
    rng = np.random.default_rng(G * 10 + k)
    idx = np.full((w.B, w.Hkv, w.n_tiles, k), -1, dtype=np.int32)
    for b in range(w.B):
        for h in range(w.Hkv):
            for t in range(w.n_tiles):
                last = (w.q_start + 64 * t + 63) // 64  # the tile's own (diagonal) block
                pool = np.arange(last)  # earlier blocks; the diagonal one is always added
                picks = rng.choice(pool, min(k - 1, pool.size), replace=False)
                picks = np.sort(np.append(picks, last))  # distinct, and the causal mask is exercised
                idx[b, h, t, : picks.size] = picks
    if k > 2:
        idx[0, 0, 0, 1] = -1  # an unused slot in the middle
    out = gpu.block_sparse_attn(Q, K, V, torch.from_numpy(idx).to(DEV), w.T, w.q_start)
    torch.cuda.synchronize()
    ref = oracle.block_sparse_attention(parity.to_f64(Q), parity.to_f64(K), parity.to_f64(V), idx, w.q_start, w.scale)
    err = parity.check_attention(parity.to_f64(out), ref, parity.ATTN_ATOL_BF16)
    say(f"  max abs err {err:.2e}")


def test_prefill_step_end_to_end(gpu):
    """select -> top-k per tile -> attention for a whole prefill from position 0."""
    w = prefill(2048, 2048, Hq=8, Hkv=2, k=6, seed=41)
    Q, K, V, F = gen(w, "Q"), gen(w, "K"), gen(w, "V"), gen(w, "F")
    Kc = gpu.compress_keys(K)
    s = gpu.select_forecast(F, Kc, w.T, w.q_start)
    idx = gpu.topk_blocks(s, w.k)
    out = gpu.block_sparse_attn(Q, K, V, idx, w.T, w.q_start)
    torch.cuda.synchronize()
    idx_np = idx.cpu().numpy()
    ref_s = oracle.select_forecast(parity.to_f64(F), parity.to_f64(Kc), w.T, w.q_start, w.scale)
    parity.check_topk_band(idx_np, ref_s, w.k)
    # early tiles have fewer candidates than k: padding must be -1
    assert (idx_np[..., 0, 1:] == -1).all()
    ref = oracle.block_sparse_attention(parity.to_f64(Q), parity.to_f64(K), parity.to_f64(V), idx_np, w.q_start,
                                        w.scale)
    parity.check_attention(parity.to_f64(out), ref, parity.ATTN_ATOL_BF16)


def test_c5_full_size_parity(gpu):
    """The 4096-query chunk at the end of a 128K context: 32 (KV head, tile)
    pairs, every head's first and last tile and 16 more drawn at random, all
    64 queries of each: Forecast scores and selection, and the attention of all
    4 query heads of the group; the multi-head selector on 8 of the pairs."""
    w = wl.C5_PREFILL
    say("generating", w.name)
    Q, K, V, F = gen(w, "Q"), gen(w, "K"), gen(w, "V"), gen(w, "F")
    Kc = gpu.compress_keys(K)
    s = gpu.select_forecast(F, Kc, w.T, w.q_start)
    sm = gpu.select_multihead(Q, Kc, w.T, w.q_start)
    idx = gpu.topk_blocks(s, w.k)
    idx_m = gpu.topk_blocks(sm, w.k).cpu().numpy()
    out = gpu.block_sparse_attn(Q, K, V, idx, w.T, w.q_start)
    torch.cuda.synchronize()
    idx_np = idx.cpu().numpy()
    s_np, sm_np, out_np = parity.to_f64(s), parity.to_f64(sm), parity.to_f64(out)
    assert idx_np.min() >= 0 and np.all(np.diff(idx_np, axis=-1) > 0)
    rng = np.random.default_rng(5)
    pairs = [(h, 0) for h in range(w.Hkv)] + [(h, w.n_tiles - 1) for h in range(w.Hkv)]
    pairs += [(int(h), int(t)) for h, t in zip(rng.integers(0, w.Hkv, 16), rng.integers(1, w.n_tiles - 1, 16))]
    worst = err = 0.0
    banded = 0
    for n, (h, t) in enumerate(pairs):
        kc64 = parity.to_f64(Kc[0, h])
        pos = [w.q_start + 64 * t + i for i in range(64)]
        ref_s = oracle.select_forecast_tile(parity.to_f64(F[0, h, 64 * t:64 * t + 64]), kc64, pos, w.T,
                                            w.scale)[None]
        worst = max(worst, parity.check_scores(s_np[0, h, t][None], ref_s))
        banded += parity.check_topk_band(idx_np[0, h, t][None], ref_s, w.k)
        q_rows = parity.to_f64(Q[0, h * w.G:(h + 1) * w.G, 64 * t:64 * t + 64])
        if n % 4 == 0:
            ref_m = oracle.select_multihead_tile(q_rows, kc64, pos, w.T, w.scale)[None]
            worst = max(worst, parity.check_scores(sm_np[0, h, t][None], ref_m))
            banded += parity.check_topk_band(idx_m[0, h, t][None], ref_m, w.k)
        # every query of the tile attends over the tile's selection cut at its
        # own position: the keys are gathered once and cut per query
        J_all = oracle.selected_keys(idx_np[0, h, t], pos[-1])
        Jt = torch.from_numpy(J_all).to(DEV)
        KJ, VJ = parity.to_f64(K[0, h].index_select(0, Jt)), parity.to_f64(V[0, h].index_select(0, Jt))
        for i, p in enumerate(pos):
            J = oracle.selected_keys(idx_np[0, h, t], p)
            assert np.array_equal(J, J_all[: J.size])
            for g in range(w.G):
                ref_o = oracle.attend(q_rows[g, i], KJ[: J.size], VJ[: J.size], w.scale)
                err = max(err, parity.check_attention(out_np[0, h * w.G + g, 64 * t + i], ref_o,
                                                      parity.ATTN_ATOL_BF16))
    say(f"c5 {len(pairs)} tiles: worst score error {worst:.2e}, banded tiles {banded}, attention max abs {err:.2e}")
