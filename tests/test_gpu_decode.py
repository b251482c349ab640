"""GPU parity of the decode path (compress, Forecast and multi-head selection,
top-k, block-sparse attention, prefetch) against the fp64 oracle, through the
C ABI of libsparda.so. Inputs come from the seeded generator; the oracle sees
the exact stored bits."""

import numpy as np
import pytest
import torch

import oracle
import synth
import synth.gpu as sg
from synth import workloads as wl
from tests import parity

pytestmark = pytest.mark.gpu
DEV = "cuda"


def say(*a):
    print(*a, flush=True)


def gen(w: wl.Workload, name: str, layer: int = 0, shape=None):
    return sg.tensor(w.recipe(name, layer), shape or w.shape(name), DEV)


def small(dtype="bf16", **kw):
    base = dict(name="small", description="small decode", dtype=dtype, B=2, Hq=8, Hkv=2, T=64 * 37, d=128, Tq=1,
                q_start=64 * 37 - 1, k=5, seed=11, block_offsets=dtype == "bf16",
                value_scale=wl.INV_SQRT_128 if dtype == "fp32" else None)
    base.update(kw)
    if "T" in kw and "q_start" not in kw:
        base["q_start"] = kw["T"] - 1
    return wl.Workload(**base)


# ------------------------------------------------------------- generator ----
def test_gpu_fill_matches_numpy_generator(gpu):
    cases = [(wl.C1_TINY, "Q", wl.C1_TINY.shape("Q"), 0),
             (wl.C2_DECODE_32K, "K", (1, 2, 512, 128), 0),
             (wl.C5_PREFILL, "V", (1, 1, 256, 128), 0)]
    for w, name, shape, start in cases:
        say("fill", w.name, name, shape)
        t = sg.tensor(w.recipe(name), shape, DEV)
        ref = synth.generate(w.recipe(name), shape)
        got = t.view(torch.int16).cpu().numpy().view(np.uint16) if t.dtype == torch.bfloat16 else t.cpu().numpy()
        np.testing.assert_array_equal(got.view(np.uint8), ref.view(np.uint8))
    # a slice deep inside the 128K-context key tensor (per-block offsets included)
    w = wl.C3_DECODE_128K
    shape = w.shape("K")
    lead, t0 = (9, 5), 100_000
    start = (int(np.ravel_multi_index(lead, shape[:2])) * w.T + t0) * w.d
    t = torch.empty(300 * w.d, dtype=torch.bfloat16, device=DEV)
    sg.fill_(t, w.recipe("K"), shape, start=start)
    ref = synth.generate_slice(w.recipe("K"), shape, lead, t0, t0 + 300)
    np.testing.assert_array_equal(t.view(torch.int16).cpu().numpy().view(np.uint16), ref.ravel())


# -------------------------------------------------------------- compress ----
def _check_compress_rows(kbs, K, Kc, dtype, rows):
    Kf = K.view(-1, K.shape[-2], K.shape[-1])
    Kcf = Kc.view(-1, Kc.shape[-2], Kc.shape[-1])
    worst = 0.0
    for r in rows:
        k64 = parity.to_f64(Kf[r])
        ref = oracle.compress_keys(k64)
        mean_abs = oracle.compress_keys(np.abs(k64)) if dtype == "fp32" else None
        worst = max(worst, parity.check_compress(parity.to_f64(Kcf[r]), ref, dtype, mean_abs))
    return worst


@pytest.mark.parametrize("w", [small("bf16"), small("fp32"), small("bf16", T=64, k=1), wl.C1_TINY, wl.C2_DECODE_32K],
                         ids=lambda w: f"{w.name}-{w.dtype}-T{w.T}")
def test_compress_parity(gpu, w):
    say("compress", w.name, w.dtype, w.T)
    K = gen(w, "K")
    Kc = gpu.compress_keys(K)
    torch.cuda.synchronize()
    assert Kc.shape == w.shape("Kc")
    _check_compress_rows(gpu, K, Kc, w.dtype, range(w.B * w.Hkv))


# ------------------------------------------------------------- selection ----
def _select_inputs(w, kbs):
    K = gen(w, "K")
    Kc = kbs.compress_keys(K)
    return K, Kc


@pytest.mark.parametrize("w", [small("bf16"), small("fp32"), small("bf16", T=64, k=1), small("bf16", T=128, k=2),
                               wl.C1_TINY, wl.C2_DECODE_32K], ids=lambda w: f"{w.name}-{w.dtype}-T{w.T}")
def test_select_forecast_decode_parity(gpu, w):
    say("select_forecast", w.name, w.dtype, w.T)
    _, Kc = _select_inputs(w, gpu)
    F = gen(w, "F")
    s = gpu.select_forecast(F, Kc, w.T, w.q_start)
    torch.cuda.synchronize()
    ref = oracle.select_forecast(parity.to_f64(F), parity.to_f64(Kc), w.T, w.q_start, w.scale)
    worst = parity.check_scores(parity.to_f64(s), ref)
    idx = gpu.topk_blocks(s, w.k)
    banded = parity.check_topk_band(idx.cpu().numpy(), ref, w.k)
    say(f"  worst score rel err {worst:.2e}, rows in tie band {banded}")


@pytest.mark.parametrize("G", [1, 2, 4, 8])
@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
def test_select_multihead_decode_parity(gpu, G, dtype):
    w = small(dtype, Hq=2 * G)
    say("select_multihead", dtype, "G", G)
    _, Kc = _select_inputs(w, gpu)
    Q = gen(w, "Q")
    s = gpu.select_multihead(Q, Kc, w.T, w.q_start)
    torch.cuda.synchronize()
    ref = oracle.select_multihead(parity.to_f64(Q), parity.to_f64(Kc), w.T, w.q_start, w.scale)
    parity.check_scores(parity.to_f64(s), ref)
    parity.check_topk_band(gpu.topk_blocks(s, w.k).cpu().numpy(), ref, w.k)


@pytest.mark.parametrize("w", [wl.C1_TINY, wl.C2_DECODE_32K], ids=lambda w: w.name)
def test_select_multihead_workloads(gpu, w):
    say("select_multihead", w.name)
    _, Kc = _select_inputs(w, gpu)
    Q = gen(w, "Q")
    s = gpu.select_multihead(Q, Kc, w.T, w.q_start)
    torch.cuda.synchronize()
    ref = oracle.select_multihead(parity.to_f64(Q), parity.to_f64(Kc), w.T, w.q_start, w.scale)
    parity.check_scores(parity.to_f64(s), ref)
    parity.check_topk_band(gpu.topk_blocks(s, w.k).cpu().numpy(), ref, w.k)


@pytest.mark.parametrize("scale", [-0.07, 0.0])
def test_decode_path_any_scale(gpu, scale):
    """Both decode selectors, then the fused top-k + attention, with a
    negative and a zero scale (at zero every visible window ties and the
    attention weights are uniform over the selected keys)."""
    w = small("bf16", B=3, T=64 * 40, k=7)
    say("decode path, scale", scale)
    F, K, Q, V = gen(w, "F"), gen(w, "K"), gen(w, "Q"), gen(w, "V")
    Kc = gpu.compress_keys(K)
    s = gpu.select_forecast(F, Kc, w.T, w.q_start, scale=scale)
    m = gpu.select_multihead(Q, Kc, w.T, w.q_start, scale=scale)
    idx, out = gpu.topk_block_sparse_attn(s, Q, K, V, w.k, w.T, w.q_start, scale=scale)
    torch.cuda.synchronize()
    ref = oracle.select_forecast(parity.to_f64(F), parity.to_f64(Kc), w.T, w.q_start, scale)
    parity.check_scores(parity.to_f64(s), ref)
    parity.check_topk_band(idx.cpu().numpy(), ref, w.k)
    ref_m = oracle.select_multihead(parity.to_f64(Q), parity.to_f64(Kc), w.T, w.q_start, scale)
    parity.check_scores(parity.to_f64(m), ref_m)
    ref_o = oracle.block_sparse_attention(parity.to_f64(Q), parity.to_f64(K), parity.to_f64(V), idx.cpu().numpy(),
                                          w.q_start, scale)
    err = parity.check_attention(parity.to_f64(out), ref_o, parity.ATTN_ATOL_BF16)
    say(f"  attention err {err:.2e}")


# ------------------------------------------------------------------ top-k ---
@pytest.mark.parametrize("nB", [1, 7, 64, 255, 256, 257, 512, 2048, 4097, 8192])
def test_topk_exact(gpu, nB):
    rng = np.random.default_rng(nB)
    rows = 37
    s = rng.standard_normal((rows, nB)).astype(np.float32)
    s[0] = 1.0                                            # all tied
    s[1] = rng.integers(-3, 4, size=nB).astype(np.float32)  # heavy ties
    s[2, ::3] = -np.inf                                   # non-candidates
    s[3] = -np.inf
    s[3, nB // 2] = 0.0                                   # one candidate
    s[4] = -s[4] * 0.0                                     # +-0 mixed
    s[5] = np.float32(1e-38) * rng.standard_normal(nB).astype(np.float32)  # tiny values
    st = torch.from_numpy(s).to(DEV)
    for k in sorted(x for x in {1, 3, 16, 64, nB} if x <= nB):
        idx = gpu.topk_blocks(st, k).cpu().numpy()
        ref = oracle.topk_blocks(s.astype(np.float64), k)
        np.testing.assert_array_equal(idx, ref, err_msg=f"nB={nB} k={k}")


def test_topk_signed_zero_tie(gpu):
    # -0.0 and +0.0 are equal scores: the lower index wins, as in the oracle
    s = np.array([[-0.0, 0.0, 1.0, -1.0], [0.0, -0.0, -1.0, -2.0]], dtype=np.float32)
    idx = gpu.topk_blocks(torch.from_numpy(s).to(DEV), 2).cpu().numpy()
    np.testing.assert_array_equal(idx, oracle.topk_blocks(s.astype(np.float64), 2))
    np.testing.assert_array_equal(idx, [[0, 2], [0, 1]])


@pytest.mark.parametrize("nB", [5, 37, 100, 1000])
def test_topk_mixed_sign_lane_groups(gpu, nB):
    """Rows where some 16-lane groups of the wave see only negative scores and
    others see positive ones (the unsigned order of the keys must hold across
    groups), short rows that leave lanes empty, and sentinels after the output
    that no row may overwrite."""
    rng = np.random.default_rng(1000 + nB)
    rows, k = 8, 4
    s = -np.abs(rng.standard_normal((rows, nB))).astype(np.float32) - 0.5
    npt = (nB + 255) // 256
    for r in range(rows):
        # positive scores only in blocks owned by one 16-lane group of one wave
        lanes = np.arange(16) + 16 * (r % 4) + 64 * ((r // 4) % 4)
        blk = (lanes[:, None] * npt + np.arange(npt)[None, :]).ravel()
        blk = blk[blk < nB]
        s[r, blk[: max(1, len(blk) // 2)]] = np.abs(rng.standard_normal(max(1, len(blk) // 2))) + 0.5
    s[1, nB // 3] = -np.inf
    for kk in (1, k, min(nB, 20)):
        out = torch.full((rows + 1, kk), -7, dtype=torch.int32, device=DEV)
        gpu.topk_blocks(torch.from_numpy(s).to(DEV), kk, out=out[:rows])
        got = out.cpu().numpy()
        assert (got[rows] == -7).all(), "top-k wrote past its output"
        np.testing.assert_array_equal(got[:rows], oracle.topk_blocks(s.astype(np.float64), kk), err_msg=f"k={kk}")


# -------------------------------------------------------------- attention ---
def _attention_case(kbs, w, idx_np):
    Q, K, V = gen(w, "Q"), gen(w, "K"), gen(w, "V")
    idx = torch.from_numpy(idx_np.astype(np.int32)).to(DEV)
    out = kbs.block_sparse_attn(Q, K, V, idx, w.T, w.q_start)
    torch.cuda.synchronize()
    ref = oracle.block_sparse_attention(parity.to_f64(Q), parity.to_f64(K), parity.to_f64(V), idx_np, w.q_start,
                                        w.scale)
    tol = parity.ATTN_ATOL_BF16 if w.dtype == "bf16" else 1e-4
    return parity.check_attention(parity.to_f64(out), ref, tol), (Q, K, V, idx, out)


@pytest.mark.parametrize("G", [1, 2, 4, 8])
@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
@pytest.mark.parametrize("k", [1, 5, 37])
def test_attention_decode_parity(gpu, G, dtype, k):
    w = small(dtype, Hq=2 * G, k=k)
    say("attention", dtype, "G", G, "k", k)
    rng = np.random.default_rng(G * 100 + k)
    idx = np.stack([np.sort(rng.choice(w.nB, k, replace=False)) for _ in range(w.B * w.Hkv)]).reshape(w.B, w.Hkv, 1, k)
    if k > 2:
        idx[0, 0, 0, 1] = -1  # an unused slot in the middle
    err, _ = _attention_case(gpu, w, idx)
    say(f"  max abs err {err:.2e}")


@pytest.mark.parametrize("k", [5, 37])
def test_attention_decode_shared_workspace(gpu, k):
    """Successive calls with new queries and selections on one workspace that
    starts filled with garbage: 6 rows, split into 5 and 37 block ranges (the
    merge's variants for at most 16 and for more ranges), each call against
    the oracle."""
    w = small("bf16", B=3, Hq=8, Hkv=2, k=k)
    rows = w.B * w.Hkv
    K, V = gen(w, "K"), gen(w, "V")
    K64, V64 = parity.to_f64(K), parity.to_f64(V)
    nbytes = gpu.workspace_bytes(gpu.OP_BLOCK_SPARSE_ATTN, w.B, w.Hq, w.Hkv, 1, w.T, w.k)
    ws = torch.full((nbytes,), 0x7F, dtype=torch.uint8, device=DEV)
    rng = np.random.default_rng(k)
    for call in range(4):
        Q = sg.tensor(wl.scaled(w, seed=300 + call).recipe("Q"), w.shape("Q"), DEV)
        idx_np = np.stack([np.sort(rng.choice(w.nB, k, replace=False)) for _ in range(rows)])
        idx_np = idx_np.reshape(w.B, w.Hkv, 1, k).astype(np.int32)
        out = gpu.block_sparse_attn(Q, K, V, torch.from_numpy(idx_np).to(DEV), w.T, w.q_start, ws=ws)
        torch.cuda.synchronize()
        ref = oracle.block_sparse_attention(parity.to_f64(Q), K64, V64, idx_np, w.q_start, w.scale)
        err = parity.check_attention(parity.to_f64(out), ref, parity.ATTN_ATOL_BF16)
        say(f"k {k} call {call}: max abs err {err:.2e}")


@pytest.mark.parametrize("w", [wl.C1_TINY, wl.C2_DECODE_32K], ids=lambda w: w.name)
def test_decode_step_end_to_end(gpu, w):
    """select (Forecast) -> top-k -> attention, against the oracle run from K."""
    say("decode step", w.name)
    K, V, Q, F = gen(w, "K"), gen(w, "V"), gen(w, "Q"), gen(w, "F")
    Kc = gpu.compress_keys(K)
    s = gpu.select_forecast(F, Kc, w.T, w.q_start)
    idx = gpu.topk_blocks(s, w.k)
    out = gpu.block_sparse_attn(Q, K, V, idx, w.T, w.q_start)
    torch.cuda.synchronize()
    K64, V64, Q64, F64 = (parity.to_f64(x) for x in (K, V, Q, F))
    # end to end from K: the oracle compresses in fp64; the GPU's Kc is bf16
    s_ref = oracle.select_forecast(F64, oracle.compress_keys(K64), w.T, w.q_start, w.scale)
    parity.check_scores(parity.to_f64(s), s_ref, rtol=1e-2 if w.dtype == "bf16" else 1e-3)
    idx_np = idx.cpu().numpy()
    banded = parity.check_topk_band(idx_np, oracle.select_forecast(F64, parity.to_f64(Kc), w.T, w.q_start, w.scale),
                                    w.k)
    ref = oracle.block_sparse_attention(Q64, K64, V64, idx_np, w.q_start, w.scale)
    tol = parity.ATTN_ATOL_BF16 if w.dtype == "bf16" else 1e-4
    err = parity.check_attention(parity.to_f64(out), ref, tol)
    # and with the oracle's own selection fed to the GPU attention
    idx_ref = oracle.topk_blocks(s_ref, w.k)
    out2 = gpu.block_sparse_attn(Q, K, V, torch.from_numpy(idx_ref).to(DEV), w.T, w.q_start)
    torch.cuda.synchronize()
    parity.check_attention(parity.to_f64(out2), oracle.block_sparse_attention(Q64, K64, V64, idx_ref, w.q_start,
                                                                               w.scale), tol)
    # determinism
    out3 = gpu.block_sparse_attn(Q, K, V, idx, w.T, w.q_start)
    s3 = gpu.select_forecast(F, Kc, w.T, w.q_start)
    torch.cuda.synchronize()
    assert torch.equal(out3.view(torch.int16) if out3.dtype == torch.bfloat16 else out3,
                       out.view(torch.int16) if out.dtype == torch.bfloat16 else out)
    assert torch.equal(s3, s)
    say(f"  attn err {err:.2e}, banded rows {banded}")


# ------------------------------------------------------- prefetch/staging ---
@pytest.mark.parametrize("nwg", [0, 1, 7, 64])
def test_prefetch_gather_and_staging_attention(gpu, nwg):
    w = small("bf16", B=3, k=5)
    say("prefetch", nwg)
    Kh = sg.pinned_tensor(w.recipe("K"), w.shape("K"), DEV)
    Vh = sg.pinned_tensor(w.recipe("V"), w.shape("V"), DEV)
    rng = np.random.default_rng(nwg)
    idx_np = np.stack([rng.choice(w.nB, w.k, replace=False) for _ in range(w.B * w.Hkv)]).reshape(w.B, w.Hkv, w.k)
    idx_np[1, 1, 2] = -1
    idx = torch.from_numpy(idx_np.astype(np.int32)).to(DEV)
    sk = torch.full((w.B, w.Hkv, w.k, 64, 128), float("nan"), dtype=torch.bfloat16, device=DEV)
    sv = torch.full_like(sk, float("nan"))
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    gpu.prefetch_blocks(Kh, Vh, idx, sk, sv, num_workgroups=nwg, stream=side)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    kbits = Kh.view(torch.int16).numpy().view(np.uint16)
    ref_k = oracle.gather_blocks(kbits, idx_np)
    got_k = sk.view(torch.int16).cpu().numpy().view(np.uint16)
    live = idx_np >= 0
    np.testing.assert_array_equal(got_k[live], ref_k[live])
    ref_v = oracle.gather_blocks(Vh.view(torch.int16).numpy().view(np.uint16), idx_np)
    np.testing.assert_array_equal(sv.view(torch.int16).cpu().numpy().view(np.uint16)[live], ref_v[live])
    # staging-mode attention == cache-mode attention, bit for bit
    Q = gen(w, "Q")
    Kd, Vd = Kh.to(DEV), Vh.to(DEV)
    idx4 = idx.view(w.B, w.Hkv, 1, w.k)
    o_cache = gpu.block_sparse_attn(Q, Kd, Vd, idx4, w.T, w.q_start, kv_mode=gpu.KV_CACHE)
    o_stage = gpu.block_sparse_attn(Q, sk, sv, idx4, w.T, w.q_start, kv_mode=gpu.KV_STAGING)
    torch.cuda.synchronize()
    assert torch.equal(o_cache.view(torch.int16), o_stage.view(torch.int16))


def _cache_model(tags, idx_row):
    """Expected slot assignment of one row: a selected block already held keeps
    its (first) slot; each other selected block takes the lowest slot that no
    selected block holds. Returns (slot_of, new tags, fetched js)."""
    tags = list(tags)
    slot_of = [-1] * len(idx_row)
    keep = set()
    for j, b in enumerate(idx_row):
        if b >= 0 and b in tags:
            slot_of[j] = tags.index(b)
            keep.add(slot_of[j])
    free = [s for s in range(len(tags)) if s not in keep]
    fetched = [j for j, b in enumerate(idx_row) if b >= 0 and slot_of[j] < 0]
    for m, j in enumerate(fetched):
        slot_of[j] = free[m]
        tags[free[m]] = idx_row[j]
    return slot_of, tags, fetched


@pytest.mark.parametrize("nwg,extra_slots", [(0, 0), (3, 5), (64, 6)])
def test_prefetch_cached_across_steps(gpu, nwg, extra_slots):
    """Four gathers into a staging buffer kept as a block cache, with selections
    that share blocks from call to call: slot assignment and tags follow the
    host model, every selected block's staged copy equals its host block, kept
    blocks are not fetched again, and attention over the cache equals
    attention over the device cache bit for bit."""
    w = small("bf16", B=3, k=6)
    n_slots = w.k + extra_slots
    say("prefetch cached", nwg, n_slots)
    Kh = sg.pinned_tensor(w.recipe("K"), w.shape("K"), DEV)
    Vh = sg.pinned_tensor(w.recipe("V"), w.shape("V"), DEV)
    rows = w.B * w.Hkv
    rng = np.random.default_rng(40 + nwg)
    first = np.stack([np.sort(rng.choice(w.nB, w.k, replace=False)) for _ in range(rows)])
    calls = [first]
    nxt = first.copy()
    for r in range(rows):  # half the blocks stay
        pool = np.setdiff1d(np.arange(w.nB), nxt[r])
        nxt[r, w.k // 2:] = rng.choice(pool, w.k - w.k // 2, replace=False)
    calls.append(np.sort(nxt, axis=1))
    third = calls[-1][:, ::-1].copy()  # same blocks, other order, one unused slot
    third[0, 1] = -1
    calls.append(third)
    calls.append(np.stack([np.sort(rng.choice(w.nB, w.k, replace=False)) for _ in range(rows)]))
    tags = torch.full((w.B, w.Hkv, n_slots), -1, dtype=torch.int32, device=DEV)
    slot_of = torch.empty((w.B, w.Hkv, w.k), dtype=torch.int32, device=DEV)
    sk = torch.full((w.B, w.Hkv, n_slots, 64, 128), float("nan"), dtype=torch.bfloat16, device=DEV)
    sv = torch.full_like(sk, float("nan"))
    model_tags = [[-1] * n_slots for _ in range(rows)]
    side = torch.cuda.Stream()
    Q = gen(w, "Q")
    fetched_total = 0
    for c, idx_np in enumerate(calls):
        if c == 2:  # change the host copy of a block that stays selected: it must not be fetched again
            b_kept = int(calls[1][0, 0])
            Kh[0, 0, 64 * b_kept:64 * (b_kept + 1)] = 7.0
        idx = torch.from_numpy(idx_np.reshape(w.B, w.Hkv, w.k).astype(np.int32)).to(DEV)
        side.wait_stream(torch.cuda.current_stream())
        gpu.prefetch_blocks_cached(Kh, Vh, idx, tags, slot_of, sk, sv, num_workgroups=nwg, stream=side)
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        got_slot = slot_of.view(rows, w.k).cpu().numpy()
        got_tags = tags.view(rows, n_slots).cpu().numpy()
        kb = sk.view(rows, n_slots, 64 * 128).view(torch.int16).cpu().numpy()
        vb = sv.view(rows, n_slots, 64 * 128).view(torch.int16).cpu().numpy()
        hk = Kh.view(rows, w.nB, 64 * 128).view(torch.int16).numpy()
        hv = Vh.view(rows, w.nB, 64 * 128).view(torch.int16).numpy()
        for r in range(rows):
            exp_slot, model_tags[r], fetched = _cache_model(model_tags[r], list(idx_np[r]))
            fetched_total += len(fetched)
            np.testing.assert_array_equal(got_slot[r], exp_slot, err_msg=f"call {c} row {r}")
            np.testing.assert_array_equal(got_tags[r], model_tags[r], err_msg=f"call {c} row {r}")
            for j, b in enumerate(idx_np[r]):
                if b < 0:
                    continue
                if c >= 2 and r == 0 and b == b_kept:  # kept since call 1: the old host data
                    assert not np.array_equal(kb[r, exp_slot[j]], hk[r, b]), "kept block was fetched again"
                    continue
                np.testing.assert_array_equal(kb[r, exp_slot[j]], hk[r, b], err_msg=f"K call {c} row {r} j {j}")
                np.testing.assert_array_equal(vb[r, exp_slot[j]], hv[r, b], err_msg=f"V call {c} row {r} j {j}")
        if c == 1:  # attention over the cache == over the device cache (host data still untouched here)
            idx4 = idx.view(w.B, w.Hkv, 1, w.k)
            o_cache = gpu.block_sparse_attn(Q, Kh.to(DEV), Vh.to(DEV), idx4, w.T, w.q_start, kv_mode=gpu.KV_CACHE)
            o_slots = gpu.block_sparse_attn(Q, sk, sv, idx4, w.T, w.q_start, kv_mode=gpu.KV_SLOTS, slot_of=slot_of)
            torch.cuda.synchronize()
            assert torch.equal(o_cache.view(torch.int16), o_slots.view(torch.int16))
    say(f"  blocks fetched over 4 calls: {fetched_total} of {4 * rows * w.k} selected")
    assert fetched_total < 4 * rows * w.k


def test_prefetch_rejects_unpinned_host_memory(gpu):
    w = small("bf16", B=1, k=2)
    Kh = torch.zeros(w.shape("K"), dtype=torch.bfloat16)  # pageable
    idx = torch.zeros((1, w.Hkv, 2), dtype=torch.int32, device=DEV)
    sk = torch.empty((1, w.Hkv, 2, 64, 128), dtype=torch.bfloat16, device=DEV)
    lib = gpu.load()
    st = lib.sparda_prefetch_blocks(Kh.data_ptr(), Kh.data_ptr(), idx.data_ptr(), sk.data_ptr(), sk.data_ptr(),
                                    gpu.SPARDA_BF16, 1, w.Hkv, w.nB, 64, 128, 2, 0, None)
    assert st == 1 and b"pinned" in lib.sparda_last_error()


def test_empty_batch_is_a_no_op(gpu):
    e = torch.empty((0, 2, 128, 128), dtype=torch.bfloat16, device=DEV)
    lib = gpu.load()
    assert lib.sparda_compress_keys(None, None, 1, 0, 2, 128, 128, 32, 16, None) == 0
    assert lib.sparda_topk_blocks(None, None, 0, 2, 1, None) == 0
    assert gpu.compress_keys(e).shape == (0, 2, 7, 128)
