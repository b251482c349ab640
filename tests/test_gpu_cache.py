"""GPU parity with KV caches that have room to grow: queries inside the cache
(q_start + Tq < T), cache slots after the newest query holding unrelated
finite values, and a decode loop that appends one token per step and
compresses each newly completed key window with sparda_compress_windows."""

import numpy as np
import pytest
import torch

import oracle
import synth.gpu as sg
from synth import workloads as wl
from tests import parity

pytestmark = pytest.mark.gpu
DEV = "cuda"
GARBAGE = 1000.0  # finite, exact in bf16 and fp32, far from the data


def say(*a):
    print(*a, flush=True)


def cache_workload(dtype="bf16", T=64 * 37, Tq=1, q_start=None, **kw):
    base = dict(name="cache", description="cache", dtype=dtype, B=2, Hq=8, Hkv=2, T=T, d=128, Tq=Tq,
                q_start=T - Tq if q_start is None else q_start, k=6, seed=71, block_offsets=dtype == "bf16",
                value_scale=wl.INV_SQRT_128 if dtype == "fp32" else None)
    base.update(kw)
    return wl.Workload(**base)


def gen(w, name):
    return sg.tensor(w.recipe(name), w.shape(name), DEV)


def bits(t):
    return t.view(torch.int16) if t.dtype == torch.bfloat16 else t


def raw(t):
    """Integer view of the bits (equal NaNs compare equal)."""
    return t.view(torch.int16) if t.dtype == torch.bfloat16 else t.view(torch.int32)


def spoil_after(t, pos):
    """Overwrite cache rows at token positions > pos with GARBAGE (a copy)."""
    t = t.clone()
    t[:, :, pos + 1:] = GARBAGE
    return t


@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
@pytest.mark.parametrize("p", [20, 31, 100, 64 * 20 - 1, 64 * 20 + 5, 64 * 37 - 1])
def test_decode_inside_a_cache(gpu, dtype, p):
    """Decode at position p of a cache of T = 2368 tokens; tokens after p, and
    the compressed windows not yet complete at p, hold GARBAGE on the device."""
    w = cache_workload(dtype, q_start=p)
    say("decode inside a cache", dtype, "p", p)
    Q, K, V, F = gen(w, "Q"), gen(w, "K"), gen(w, "V"), gen(w, "F")
    Kc_true = gpu.compress_keys(K)
    n_vis = oracle.visible_window_count(p, w.W)
    Kc = Kc_true.clone()
    Kc[:, :, n_vis:] = GARBAGE
    Kd, Vd = spoil_after(K, p), spoil_after(V, p)
    sf = gpu.select_forecast(F, Kc, w.T, p)
    sm = gpu.select_multihead(Q, Kc, w.T, p)
    idx = gpu.topk_blocks(sf, w.k)
    out = gpu.block_sparse_attn(Q, Kd, Vd, idx, w.T, p)
    torch.cuda.synchronize()
    kc64 = parity.to_f64(Kc_true)
    ref_f = oracle.select_forecast(parity.to_f64(F), kc64, w.T, p, w.scale)
    ref_m = oracle.select_multihead(parity.to_f64(Q), kc64, w.T, p, w.scale)
    parity.check_scores(parity.to_f64(sf), ref_f)
    parity.check_scores(parity.to_f64(sm), ref_m)
    idx_np = idx.cpu().numpy()
    parity.check_topk_band(idx_np, ref_f, w.k)
    ref_o = oracle.block_sparse_attention(parity.to_f64(Q), parity.to_f64(K), parity.to_f64(V), idx_np, p, w.scale)
    tol = parity.ATTN_ATOL_BF16 if dtype == "bf16" else 1e-4
    err = parity.check_attention(parity.to_f64(out), ref_o, tol)
    if n_vis == 0:
        assert (idx_np == -1).all() and not torch.any(out.float() != 0)
    say(f"  visible windows {n_vis}, attention err {err:.2e}")


@pytest.mark.parametrize("q_start", [64 * 10, 64 * 10 + 17])
def test_prefill_chunk_inside_a_cache(gpu, q_start):
    """A 512-query chunk that ends before the cache does; tokens after the
    chunk's last query hold GARBAGE."""
    w = cache_workload("bf16", Tq=512, q_start=q_start, k=7, seed=73)
    last = q_start + w.Tq - 1
    say("prefill inside a cache, q_start", q_start)
    Q, K, V, F = gen(w, "Q"), gen(w, "K"), gen(w, "V"), gen(w, "F")
    Kc_true = gpu.compress_keys(K)
    Kc = Kc_true.clone()
    Kc[:, :, oracle.visible_window_count(last, w.W):] = GARBAGE
    Kd, Vd = spoil_after(K, last), spoil_after(V, last)
    sf = gpu.select_forecast(F, Kc, w.T, q_start)
    sm = gpu.select_multihead(Q, Kc, w.T, q_start)
    idx = gpu.topk_blocks(sf, w.k)
    out = gpu.block_sparse_attn(Q, Kd, Vd, idx, w.T, q_start)
    torch.cuda.synchronize()
    kc64 = parity.to_f64(Kc_true)
    ref_f = oracle.select_forecast(parity.to_f64(F), kc64, w.T, q_start, w.scale)
    ref_m = oracle.select_multihead(parity.to_f64(Q), kc64, w.T, q_start, w.scale)
    parity.check_scores(parity.to_f64(sf), ref_f)
    parity.check_scores(parity.to_f64(sm), ref_m)
    idx_np = idx.cpu().numpy()
    parity.check_topk_band(idx_np, ref_f, w.k)
    ref_o = oracle.block_sparse_attention(parity.to_f64(Q), parity.to_f64(K), parity.to_f64(V), idx_np, q_start,
                                          w.scale)
    err = parity.check_attention(parity.to_f64(out), ref_o, parity.ATTN_ATOL_BF16)
    say(f"  attention err {err:.2e}")


@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
def test_compress_windows_in_pieces_equals_full(gpu, dtype):
    w = cache_workload(dtype)
    K = gen(w, "K")
    full = gpu.compress_keys(K)
    part = torch.full_like(full, float("nan"))
    for a, b in [(0, 5), (5, 37), (37, 38), (38, w.W)]:
        gpu.compress_windows(K, part, a, b)
    torch.cuda.synchronize()
    assert torch.equal(bits(part), bits(full))
    # only the requested range is written
    part2 = torch.full_like(full, float("nan"))
    gpu.compress_windows(K, part2, 10, 20)
    torch.cuda.synchronize()
    assert torch.equal(bits(part2[:, :, 10:20]), bits(full[:, :, 10:20]))
    assert torch.isnan(part2[:, :, :10].float()).all() and torch.isnan(part2[:, :, 20:].float()).all()


def test_decode_loop_growing_cache(gpu):
    """The cache starts filled to position p0; each step appends token p, and
    when token p completes a window (16 w + 31 = p) that window is compressed
    on its own. Every step's selection, top-k and attention match the oracle
    on the true data."""
    w = cache_workload("bf16", T=64 * 24, k=6, seed=77)
    p0 = 64 * 10 + 7
    steps = 50
    K_true, V_true = gen(w, "K"), gen(w, "V")
    Q_all = sg.tensor(wl.scaled(w, seed=78).recipe("Q"), (w.B, w.Hq, steps, w.d), DEV)
    F_all = sg.tensor(wl.scaled(w, seed=78).recipe("F"), (w.B, w.Hkv, steps, w.d), DEV)
    K, V = spoil_after(K_true, p0 - 1), spoil_after(V_true, p0 - 1)  # tokens 0 .. p0-1 written
    Kc = torch.full((w.B, w.Hkv, w.W, w.d), GARBAGE, dtype=K.dtype, device=DEV)
    n0 = oracle.visible_window_count(p0 - 1, w.W)
    gpu.compress_windows(K, Kc, 0, n0)
    kc64_true = oracle.compress_keys(parity.to_f64(K_true))
    k64, v64 = parity.to_f64(K_true), parity.to_f64(V_true)
    compressed = n0
    for i in range(steps):
        p = p0 + i
        K[:, :, p] = K_true[:, :, p]  # append token p
        V[:, :, p] = V_true[:, :, p]
        n_vis = oracle.visible_window_count(p, w.W)
        if n_vis > compressed:  # token p completed window n_vis - 1
            gpu.compress_windows(K, Kc, compressed, n_vis)
            compressed = n_vis
        Q, F = Q_all[:, :, i:i + 1].contiguous(), F_all[:, :, i:i + 1].contiguous()
        s = gpu.select_forecast(F, Kc, w.T, p)
        idx = gpu.topk_blocks(s, w.k)
        out = gpu.block_sparse_attn(Q, K, V, idx, w.T, p)
        if i % 7 == 0 or i == steps - 1:
            torch.cuda.synchronize()
            F64 = parity.to_f64(F)
            # per op, on the windows the loop compressed (bf16, checked bitwise
            # against a full compression below) ...
            ref_s = oracle.select_forecast(F64, parity.to_f64(Kc), w.T, p, w.scale)
            parity.check_scores(parity.to_f64(s), ref_s)
            # ... and end to end from the true keys, compressed in fp64
            parity.check_scores(parity.to_f64(s), oracle.select_forecast(F64, kc64_true, w.T, p, w.scale), rtol=1e-2)
            idx_np = idx.cpu().numpy()
            parity.check_topk_band(idx_np, ref_s, w.k)
            ref_o = oracle.block_sparse_attention(parity.to_f64(Q), k64, v64, idx_np, p, w.scale)
            err = parity.check_attention(parity.to_f64(out), ref_o, parity.ATTN_ATOL_BF16)
            say(f"step {i} position {p}: windows {compressed}, attention err {err:.2e}")
    torch.cuda.synchronize()
    # the incrementally built windows equal a full compression of the true keys
    full = gpu.compress_keys(K_true)
    torch.cuda.synchronize()
    assert torch.equal(bits(Kc[:, :, :compressed]), bits(full[:, :, :compressed]))


# ------------------------------------------------ append, ragged sequences ---
def _gather_new(K_true, L, n):
    """The n tokens of each sequence b starting at L[b]: [B, Hkv, n, d]."""
    return torch.stack([K_true[b, :, L[b]:L[b] + n] for b in range(len(L))]).contiguous()


@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
@pytest.mark.parametrize("n_new,lens", [(1, [31, 100, 767, 0]), (16, [0, 15, 752, 17]), (37, [0, 47, 731, 300])])
def test_append_kv_tokens_and_windows(gpu, dtype, n_new, lens):
    """Each sequence's n_new tokens land at its own length; every window they
    complete equals the full compression bit for bit; nothing else changes.
    Cache slots at or after a sequence's length hold NaN before the call, so a
    window that read one would be NaN."""
    w = cache_workload(dtype, T=64 * 12, B=4, Hkv=2, seed=91)
    T_cap, W_cap = w.T, w.W
    say("append", dtype, "n_new", n_new, "lengths", lens)
    K_true, V_true = gen(w, "K"), gen(w, "V")
    K, V = K_true.clone(), V_true.clone()
    for b, L in enumerate(lens):
        K[b, :, L:] = float("nan")
        V[b, :, L:] = float("nan")
    Kc = torch.full((w.B, w.Hkv, W_cap, w.d), -3.0, dtype=K.dtype, device=DEV)
    K0, V0, Kc0 = K.clone(), V.clone(), Kc.clone()
    seq_len = torch.tensor(lens, dtype=torch.int32, device=DEV)
    status = torch.zeros(1, dtype=torch.int32, device=DEV)
    gpu.append_kv(_gather_new(K_true, lens, n_new), _gather_new(V_true, lens, n_new), K, V, seq_len, k_cmp=Kc,
                  status=status)
    full = gpu.compress_keys(K_true)
    torch.cuda.synchronize()
    assert int(status.item()) == 0
    expK, expV, expKc = K0.clone(), V0.clone(), Kc0.clone()
    for b, L in enumerate(lens):
        expK[b, :, L:L + n_new] = K_true[b, :, L:L + n_new]
        expV[b, :, L:L + n_new] = V_true[b, :, L:L + n_new]
        done = [x for x in range(W_cap) if L <= 16 * x + 31 <= L + n_new - 1]
        for x in done:
            expKc[b, :, x] = full[b, :, x]
    # bitwise, NaN slots included
    assert torch.equal(raw(K), raw(expK))
    assert torch.equal(raw(V), raw(expV))
    assert torch.equal(raw(Kc), raw(expKc))


def test_append_kv_overflow_leaves_sequence_untouched(gpu):
    w = cache_workload("bf16", T=64 * 4, B=3, Hkv=2, seed=92)
    K, V = gen(w, "K"), gen(w, "V")
    Kc = gpu.compress_keys(K)
    K0, V0, Kc0 = K.clone(), V.clone(), Kc.clone()
    n_new = 8
    kn = torch.ones((w.B, w.Hkv, n_new, w.d), dtype=K.dtype, device=DEV)
    lens = [w.T - n_new, w.T - n_new + 1, -1]  # fits exactly; one token too many; negative
    seq_len = torch.tensor(lens, dtype=torch.int32, device=DEV)
    status = torch.zeros(1, dtype=torch.int32, device=DEV)
    gpu.append_kv(kn, kn, K, V, seq_len, k_cmp=Kc, status=status)
    torch.cuda.synchronize()
    assert int(status.item()) == 1
    assert torch.equal(bits(K[0, :, -n_new:]), bits(kn[0])) and torch.equal(bits(K[0, :, :-n_new]), bits(K0[0, :, :-n_new]))
    for b in (1, 2):
        assert torch.equal(bits(K[b]), bits(K0[b])) and torch.equal(bits(V[b]), bits(V0[b]))
        assert torch.equal(bits(Kc[b]), bits(Kc0[b]))


@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
def test_ragged_decode_loop(gpu, dtype):
    """Sequences of different lengths in one batch: each step appends one token
    per sequence (append_kv, which also compresses completed windows), then
    selects, takes the top-k and attends at each sequence's own position
    (q_pos). Checked against the oracle run sequence by sequence."""
    w = cache_workload(dtype, T=64 * 24, B=4, Hkv=2, Hq=8, k=6, seed=93)
    lens0 = [40, 333, 700, 1300]
    steps = 24
    K_true, V_true = gen(w, "K"), gen(w, "V")
    Q_all = sg.tensor(wl.scaled(w, seed=94).recipe("Q"), (w.B, w.Hq, steps, w.d), DEV)
    F_all = sg.tensor(wl.scaled(w, seed=94).recipe("F"), (w.B, w.Hkv, steps, w.d), DEV)
    K = torch.full_like(K_true, GARBAGE)
    V = torch.full_like(V_true, GARBAGE)
    Kc = torch.full((w.B, w.Hkv, w.W, w.d), GARBAGE, dtype=K.dtype, device=DEV)
    # prefill: every sequence's first lens0[b] tokens, through append_kv as well
    for b, L in enumerate(lens0):
        one = torch.tensor([0], dtype=torch.int32, device=DEV)
        gpu.append_kv(K_true[b:b + 1, :, :L].contiguous(), V_true[b:b + 1, :, :L].contiguous(), K[b:b + 1], V[b:b + 1],
                      one, k_cmp=Kc[b:b + 1])
    seq_len = torch.tensor(lens0, dtype=torch.int32, device=DEV)
    k64, v64 = parity.to_f64(K_true), parity.to_f64(V_true)
    kc64_true = oracle.compress_keys(k64)
    tol = parity.ATTN_ATOL_BF16 if dtype == "bf16" else 1e-4
    for i in range(steps):
        lens = [lens0[b] + i for b in range(w.B)]
        gpu.append_kv(_gather_new(K_true, lens, 1), _gather_new(V_true, lens, 1), K, V, seq_len, k_cmp=Kc)
        q_pos = seq_len.clone()  # each query sits at its sequence's new token
        Q, F = Q_all[:, :, i:i + 1].contiguous(), F_all[:, :, i:i + 1].contiguous()
        s = gpu.select_forecast(F, Kc, w.T, 0, q_pos=q_pos)
        sm = gpu.select_multihead(Q, Kc, w.T, 0, q_pos=q_pos)
        idx = gpu.topk_blocks(s, w.k)
        out = gpu.block_sparse_attn(Q, K, V, idx, w.T, 0, q_pos=q_pos)
        seq_len += 1
        if i % 5 == 0 or i == steps - 1:
            torch.cuda.synchronize()
            kc64 = parity.to_f64(Kc)
            idx_np = idx.cpu().numpy()
            F64, Q64, s64, sm64, o64 = (parity.to_f64(x) for x in (F, Q, s, sm, out))
            for b, p in enumerate(lens):
                sl = slice(b, b + 1)
                ref_s = oracle.select_forecast(F64[sl], kc64[sl], w.T, p, w.scale)
                parity.check_scores(s64[sl], ref_s)
                parity.check_scores(s64[sl], oracle.select_forecast(F64[sl], kc64_true[sl], w.T, p, w.scale),
                                    rtol=1e-2 if dtype == "bf16" else 1e-3)
                parity.check_scores(sm64[sl], oracle.select_multihead(Q64[sl], kc64[sl], w.T, p, w.scale))
                parity.check_topk_band(idx_np[sl], ref_s, w.k)
                ref_o = oracle.block_sparse_attention(Q64[sl], k64[sl], v64[sl], idx_np[sl], p, w.scale)
                parity.check_attention(o64[sl], ref_o, tol)
            say(f"ragged step {i}: positions {lens}")
    torch.cuda.synchronize()
    full = gpu.compress_keys(K_true)
    for b in range(w.B):
        n = oracle.visible_window_count(lens0[b] + steps - 1, w.W)
        assert torch.equal(bits(Kc[b, :, :n]), bits(full[b, :, :n]))


def test_empty_sequence_position(gpu):
    """q_pos = -1 marks a sequence with no tokens: no candidate block, top-k
    all -1, attention output 0; its neighbours are unaffected."""
    w = cache_workload("bf16", T=64 * 8, B=2, Hkv=2, Hq=8, k=4, seed=95)
    Q, K, V, F = gen(w, "Q"), gen(w, "K"), gen(w, "V"), gen(w, "F")
    Kc = gpu.compress_keys(K)
    q_pos = torch.tensor([-1, 300], dtype=torch.int32, device=DEV)
    s = gpu.select_forecast(F, Kc, w.T, 0, q_pos=q_pos)
    idx = gpu.topk_blocks(s, w.k)
    out = gpu.block_sparse_attn(Q, K, V, idx, w.T, 0, q_pos=q_pos)
    torch.cuda.synchronize()
    assert torch.isneginf(s[0]).all() and (idx[0] == -1).all() and not torch.any(out[0].float() != 0)
    ref_s = oracle.select_forecast(parity.to_f64(F)[1:], parity.to_f64(Kc)[1:], w.T, 300, w.scale)
    parity.check_scores(parity.to_f64(s)[1:], ref_s)
    idx_np = idx.cpu().numpy()
    ref_o = oracle.block_sparse_attention(parity.to_f64(Q)[1:], parity.to_f64(K)[1:], parity.to_f64(V)[1:],
                                          idx_np[1:], 300, w.scale)
    parity.check_attention(parity.to_f64(out)[1:], ref_o, parity.ATTN_ATOL_BF16)
