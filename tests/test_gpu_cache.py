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
