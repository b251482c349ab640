"""GPU parity of the two-layer offloaded decode step with lookahead prefetch
(layer 1's KV in pinned host memory, gathered on a side stream while layer 0
attends), against the fp64 oracle through the C ABI."""

import numpy as np
import pytest
import torch

import oracle
from synth import workloads as wl
from synth.offload import offload_layers
from tests import parity

pytestmark = pytest.mark.gpu
DEV = "cuda"


def say(*a):
    print(*a, flush=True)


def small(seed=3, **kw):
    base = dict(B=2, Hq=8, Hkv=2, T=8192, q_start=8191, k=16, seed=seed)
    base.update(kw)
    return wl.scaled(wl.C4_OFFLOAD, **base)


def bits(t):
    return t.view(torch.int16)


def f64_layers(l0, l1):
    a = {n: parity.to_f64(l0[n]) for n in ("Q", "F_self", "F_next", "K", "V", "Kc")}
    b = {"Q": parity.to_f64(l1["Q"]), "Kc": parity.to_f64(l1["Kc"]), "K": parity.to_f64(l1["host_K"]),
         "V": parity.to_f64(l1["host_V"])}
    return a, b


def check_step(w, r0, r1, got):
    """got = (scores0, scores1, idx0, idx1, out0, out1) as numpy; r0/r1 fp64 layers."""
    s0, s1, i0, i1, o0, o1 = got
    q = w.q_start
    ref_s0 = oracle.select_forecast(r0["F_self"], r0["Kc"], w.T, q, w.scale)
    ref_s1 = oracle.select_forecast(r0["F_next"], r1["Kc"], w.T, q, w.scale)
    parity.check_scores(s0, ref_s0)
    parity.check_scores(s1, ref_s1)
    banded = parity.check_topk_band(i0, ref_s0, w.k) + parity.check_topk_band(i1, ref_s1, w.k)
    # attention against the oracle on the GPU's indices
    ref_o0 = oracle.block_sparse_attention(r0["Q"], r0["K"], r0["V"], i0, q, w.scale)
    ref_o1 = oracle.block_sparse_attention(r1["Q"], r1["K"], r1["V"], i1, q, w.scale)
    e0 = parity.check_attention(o0, ref_o0, parity.ATTN_ATOL_BF16)
    e1 = parity.check_attention(o1, ref_o1, parity.ATTN_ATOL_BF16)
    if banded == 0:  # the oracle's own step picks the same blocks: compare end to end
        O0, O1, I0, I1 = oracle.lookahead_decode_step(r0, r1, w.T, w.k, w.scale)
        assert np.array_equal(I0, i0) and np.array_equal(I1, i1)
        parity.check_attention(o0, O0, parity.ATTN_ATOL_BF16)
        parity.check_attention(o1, O1, parity.ATTN_ATOL_BF16)
    say(f"  banded rows {banded}, attention err {e0:.2e} / {e1:.2e}")


@pytest.mark.parametrize("markers", [False, True])
def test_lookahead_step_parity_back_to_back(gpu, markers):
    """Three steps enqueued without a host sync, alternating two input sets, so
    that a missing wait between the side stream's gather and the main stream's
    attention (or the next step's gather) would mix the sets' data; with and
    without the phase marker ranges."""
    from kv_block_selection_amd.lookahead import LookaheadStep
    wa, wb = small(seed=3), small(seed=103)
    sets = [offload_layers(w, gpu.compress_keys, DEV) for w in (wa, wb)]
    st = LookaheadStep(wa.B, wa.Hq, wa.Hkv, wa.T, wa.k, torch.bfloat16, DEV, markers=markers)
    st.stage_k.fill_(float("nan"))  # poisoned staging must not matter
    st.stage_v.fill_(float("nan"))
    order = [0, 1, 0]
    got = []
    for i in order:
        st.step(*sets[i])
        got.append([t.clone() for t in (st.scores0, st.scores1, st.idx0, st.idx1, st.out0, st.out1)])
    torch.cuda.synchronize()
    refs = [f64_layers(*s) for s in sets]
    for n, i in enumerate(order):
        say("step", n, "input set", i)
        g = got[n]
        check_step((wa, wb)[i], *refs[i], [parity.to_f64(t) if t.dtype != torch.int32 else t.cpu().numpy()
                                           for t in g])
    # the repeat of set 0 reproduces the first step bit for bit
    for a, b in zip(got[0], got[2]):
        assert torch.equal(a.view(torch.int16) if a.dtype == torch.bfloat16 else a,
                           b.view(torch.int16) if b.dtype == torch.bfloat16 else b)


@pytest.mark.parametrize("nwg", [8, 128])
def test_lookahead_staging_equals_device_cache(gpu, nwg):
    """Layer 1's output from the gathered staging equals attention on a device
    copy of its KV at the same indices, bit for bit, for any gather grid."""
    from kv_block_selection_amd.lookahead import LookaheadStep
    w = small(seed=7, B=3, k=8)
    l0, l1 = offload_layers(w, gpu.compress_keys, DEV)
    st = LookaheadStep(w.B, w.Hq, w.Hkv, w.T, w.k, torch.bfloat16, DEV, num_workgroups=nwg)
    st.step(l0, l1)
    o1 = st.out1.clone()
    Kd, Vd = l1["host_K"].to(DEV), l1["host_V"].to(DEV)
    ref = gpu.block_sparse_attn(l1["Q"], Kd, Vd, st.idx1, w.T, w.q_start)
    torch.cuda.synchronize()
    assert torch.equal(bits(o1), bits(ref))


def test_lookahead_with_block_cache(gpu):
    """The two-layer step with the staging kept as a block cache: layer 1's KV
    stays put while layer 0's Forecast changes (two input sets alternate), so
    successive selections share some blocks. Three steps enqueued without a
    host sync, staging poisoned at the start; each step's layer-1 output,
    indices and scores equal those of the step with plain staging, and the
    output equals attention on a device copy of layer 1's KV, bit for bit."""
    from kv_block_selection_amd.lookahead import LookaheadStep
    wa, wb = small(seed=3), small(seed=103)
    l0a, l1 = offload_layers(wa, gpu.compress_keys, DEV)
    l0b, _ = offload_layers(wb, gpu.compress_keys, DEV)
    cached = LookaheadStep(wa.B, wa.Hq, wa.Hkv, wa.T, wa.k, torch.bfloat16, DEV, cache_slots=wa.k + 3)
    plain = LookaheadStep(wa.B, wa.Hq, wa.Hkv, wa.T, wa.k, torch.bfloat16, DEV)
    cached.stage_k.fill_(float("nan"))
    cached.stage_v.fill_(float("nan"))
    got, want = [], []
    for l0 in (l0a, l0b, l0a):
        cached.step(l0, l1)
        got.append([t.clone() for t in (cached.out1, cached.idx1, cached.scores1)])
        plain.step(l0, l1)
        want.append([t.clone() for t in (plain.out1, plain.idx1, plain.scores1)])
    Kd, Vd = l1["host_K"].to(DEV), l1["host_V"].to(DEV)
    refs = [gpu.block_sparse_attn(l1["Q"], Kd, Vd, g[1], wa.T, wa.q_start) for g in got]
    torch.cuda.synchronize()
    for n, (g, w_, r) in enumerate(zip(got, want, refs)):
        say("cached step", n)
        assert torch.equal(g[1], w_[1]) and torch.equal(g[2], w_[2])
        assert torch.equal(bits(g[0]), bits(w_[0]))
        assert torch.equal(bits(g[0]), bits(r))
    # the cache holds every block of the last selection, at the slot the map gives
    tags = cached.slot_tags.view(wa.B * wa.Hkv, -1).cpu().numpy()
    sel = got[-1][1].view(wa.B * wa.Hkv, -1).cpu().numpy()
    slot = cached.slot_of.view(wa.B * wa.Hkv, -1).cpu().numpy()
    for r in range(sel.shape[0]):
        live = sel[r] >= 0
        np.testing.assert_array_equal(tags[r][slot[r][live]], sel[r][live])


def test_c4_full_size_parity(gpu):
    """The batch-64, 128K-context offload workload in the launch configuration the
    benchmark times (32 GiB of layer-1 KV in pinned host memory): every one of
    the 512 (sequence, KV head) rows of both layers (scores, selection,
    attention of all 2048 query heads) against the fp64 oracle, layer 1's keys
    and values read from the host copy; compression on three sampled rows."""
    from kv_block_selection_amd.lookahead import LookaheadStep
    w = wl.C4_OFFLOAD
    say("generating", w.name)
    l0, l1 = offload_layers(w, gpu.compress_keys, DEV)
    say("step")
    st = LookaheadStep(w.B, w.Hq, w.Hkv, w.T, w.k, torch.bfloat16, DEV)
    st.step(l0, l1)
    torch.cuda.synchronize()
    q = w.q_start
    for b, h in [(0, 0), (31, 5), (63, 7)]:
        parity.check_compress(parity.to_f64(l1["Kc"][b, h]), oracle.compress_keys(parity.to_f64(l1["host_K"][b, h])),
                              "bf16")
    worst = err = 0.0
    banded = 0
    for layer in (0, 1):
        F = l0["F_self"] if layer == 0 else l0["F_next"]
        Kc = (l0 if layer == 0 else l1)["Kc"]
        scores = parity.to_f64(st.scores0 if layer == 0 else st.scores1)
        idx = (st.idx0 if layer == 0 else st.idx1).cpu().numpy()
        out = parity.to_f64(st.out0 if layer == 0 else st.out1)
        Q = parity.to_f64((l0 if layer == 0 else l1)["Q"])
        Kl, Vl = (l0["K"], l0["V"]) if layer == 0 else (l1["host_K"], l1["host_V"])
        say("layer", layer)
        for b in range(w.B):
            for h in range(w.Hkv):
                ref_s = oracle.select_forecast_tile(parity.to_f64(F[b, h]), parity.to_f64(Kc[b, h]), [q], w.T,
                                                    w.scale)[None]
                worst = max(worst, parity.check_scores(scores[b, h], ref_s))
                banded += parity.check_topk_band(idx[b, h], ref_s, w.k)
                J = oracle.selected_keys(idx[b, h, 0], q)
                Jt = torch.from_numpy(J).to(Kl.device)
                KJ, VJ = parity.to_f64(Kl[b, h].index_select(0, Jt)), parity.to_f64(Vl[b, h].index_select(0, Jt))
                for g in range(w.G):
                    qh = h * w.G + g
                    ref_o = oracle.attend(Q[b, qh, 0], KJ, VJ, w.scale)
                    err = max(err, parity.check_attention(out[b, qh, 0], ref_o, parity.ATTN_ATOL_BF16))
    say(f"c4 all rows, both layers: worst score error {worst:.2e}, banded rows {banded}, attention max abs {err:.2e}")


@pytest.mark.parametrize("L,depth", [(2, 1), (4, 1), (4, 2), (5, 3), (3, 5)])
def test_layer_pipeline_parity(gpu, L, depth):
    """The L-layer step with lookahead of ``depth`` layers and min(depth + 1,
    L - 1) staging buffers used in turn: two steps enqueued back to back;
    every layer's selection, top-k and attention against the oracle. Layer l
    is selected by layer l - depth's Forecast of it, layers 1 .. depth by
    layer 0's."""
    from kv_block_selection_amd.pipeline import LayerPipeline
    from synth.offload import offload_stack
    w = small(seed=11, B=2, k=12)
    layers = offload_stack(w, L, gpu.compress_keys, DEV, depth=depth)
    pipe = LayerPipeline(L, w.B, w.Hq, w.Hkv, w.T, w.k, torch.bfloat16, DEV, depth=depth)
    assert len(pipe.stage) == min(depth + 1, L - 1)

    def forecast_of(l):
        if l == 0:
            return layers[0]["F_self"]
        src = max(0, l - depth)
        if depth == 1:
            return layers[src]["F_next"]
        return layers[0]["F_ahead"][l - 1] if src == 0 else layers[src]["F_ahead"]
    for s in pipe.stage:
        s[0].fill_(float("nan"))
        s[1].fill_(float("nan"))
    pipe.step(layers)
    first = [o.clone() for o in pipe.out]
    pipe.step(layers)  # again, without a host sync in between
    torch.cuda.synchronize()
    q = w.q_start
    for l in range(L):
        lay = layers[l]
        f = parity.to_f64(forecast_of(l))
        kc = parity.to_f64(lay["Kc"])
        ref_s = oracle.select_forecast(f, kc, w.T, q, w.scale)
        parity.check_scores(parity.to_f64(pipe.scores[l]), ref_s)
        idx = pipe.idx[l].cpu().numpy()
        parity.check_topk_band(idx, ref_s, w.k)
        K = parity.to_f64(lay["K"] if l == 0 else lay["host_K"])
        V = parity.to_f64(lay["V"] if l == 0 else lay["host_V"])
        ref_o = oracle.block_sparse_attention(parity.to_f64(lay["Q"]), K, V, idx, q, w.scale)
        err = parity.check_attention(parity.to_f64(pipe.out[l]), ref_o, parity.ATTN_ATOL_BF16)
        assert torch.equal(bits(first[l]), bits(pipe.out[l]))
        say(f"  layer {l}: attention err {err:.2e}")
