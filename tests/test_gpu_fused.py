"""GPU parity of the fused decode call sparda_topk_block_sparse_attn (the
row's top-k computed by each attention workgroup, then block-sparse
attention, in one launch): its selection and output must hold the same bits
as sparda_topk_blocks followed by sparda_block_sparse_attn, and match the
fp64 oracle. Covers the three top-k widths (nB <= 256, <= 2048, <= 8192),
GQA groups 1/2/4/8, fp32 and bf16, block ranges per row that do not fill the
last workgroup, ties and non-candidates in the scores, ragged positions."""

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


def bits(t):
    return t.view(torch.int16) if t.dtype == torch.bfloat16 else t.view(torch.int32)


def small(dtype="bf16", **kw):
    base = dict(name="small", description="small decode", dtype=dtype, B=2, Hq=8, Hkv=2, T=64 * 37, d=128, Tq=1,
                q_start=64 * 37 - 1, k=5, seed=17, block_offsets=dtype == "bf16",
                value_scale=wl.INV_SQRT_128 if dtype == "fp32" else None)
    base.update(kw)
    if "T" in kw and "q_start" not in kw:
        base["q_start"] = kw["T"] - 1
    return wl.Workload(**base)


def _case(gpu, w, scores=None, q_pos=None, check_oracle=True):
    Q, K, V = (sg.tensor(w.recipe(n), w.shape(n), DEV) for n in ("Q", "K", "V"))
    if scores is None:
        Kc = gpu.compress_keys(K)
        F = sg.tensor(w.recipe("F"), w.shape("F"), DEV)
        scores = gpu.select_forecast(F, Kc, w.T, w.q_start, q_pos=q_pos)
    idx_ref = gpu.topk_blocks(scores, w.k)
    out_ref = gpu.block_sparse_attn(Q, K, V, idx_ref, w.T, w.q_start, q_pos=q_pos)
    idx, out = gpu.topk_block_sparse_attn(scores, Q, K, V, w.k, w.T, w.q_start, q_pos=q_pos)
    torch.cuda.synchronize()
    assert torch.equal(idx, idx_ref), "fused top-k differs from sparda_topk_blocks"
    assert torch.equal(bits(out), bits(out_ref)), "fused attention differs from sparda_block_sparse_attn"
    if check_oracle:
        idx_np = idx.cpu().numpy()
        np.testing.assert_array_equal(idx_np, oracle.topk_blocks(parity.to_f64(scores), w.k))
        pos = w.q_start if q_pos is None else None
        if pos is not None:
            ref = oracle.block_sparse_attention(parity.to_f64(Q), parity.to_f64(K), parity.to_f64(V), idx_np, pos,
                                                w.scale)
            tol = parity.ATTN_ATOL_BF16 if w.dtype == "bf16" else 1e-4
            return parity.check_attention(parity.to_f64(out), ref, tol)
    return 0.0


@pytest.mark.parametrize("G", [1, 2, 4, 8])
@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
def test_fused_matches_separate_calls(gpu, G, dtype):
    w = small(dtype, Hq=2 * G, k=5)
    say("fused", dtype, "G", G)
    err = _case(gpu, w)
    say(f"  max abs err {err:.2e}")


@pytest.mark.parametrize("T,k", [(64, 1), (64 * 200, 7), (64 * 256, 64), (64 * 257, 33), (64 * 2048, 64),
                                 (64 * 2049, 100), (64 * 5000, 64)])
def test_fused_topk_widths_and_split_counts(gpu, T, k):
    """nB across the three top-k widths; k values whose block ranges leave the
    last workgroup of a row partly idle."""
    w = small("bf16", B=1, T=T, k=k)
    say("fused T", T, "k", k)
    _case(gpu, w, check_oracle=T <= 64 * 2048)


def test_fused_ties_and_non_candidates(gpu):
    """Integer scores full of ties (lower index wins) and -inf blocks that must
    never be taken, with rows that have fewer candidates than k (-1 padding)."""
    w = small("bf16", B=2, Hq=8, Hkv=2, k=20)
    rng = np.random.default_rng(5)
    s = rng.integers(-3, 4, size=(w.B, w.Hkv, 1, w.nB)).astype(np.float32)
    s[0, 0, 0, ::2] = -np.inf
    s[1, 1, 0, :] = -np.inf
    s[1, 1, 0, [3, 9, 30]] = 1.0  # 3 candidates < k
    _case(gpu, w, scores=torch.from_numpy(s).to(DEV))


def test_fused_ragged_positions(gpu):
    """Per-sequence query positions, one of them before its first complete
    window (no candidate block: all -1, output 0): the same bits as the
    separate calls."""
    w = small("bf16", B=5, Hq=8, Hkv=2, k=6)
    q_pos = torch.tensor([w.T - 1, 70, 64 * 20 + 5, 31, 5], dtype=torch.int32, device=DEV)
    _case(gpu, w, q_pos=q_pos)


# ------------------------------------------- merge deferred to the next layer ----
def _layers(gpu, w, n, seed0=40):
    """n layers' inputs of one decode shape: Q, K, V, F, compressed keys."""
    out = []
    for l in range(n):
        wl_ = wl.scaled(w, seed=seed0 + l)
        Q, K, V, F = (sg.tensor(wl_.recipe(nm), wl_.shape(nm), DEV) for nm in ("Q", "K", "V", "F"))
        out.append(dict(Q=Q, K=K, V=V, F=F, Kc=gpu.compress_keys(K)))
    return out


@pytest.mark.parametrize("dtype,G,k", [("bf16", 4, 5), ("bf16", 4, 37), ("bf16", 8, 20), ("fp32", 2, 9),
                                       ("bf16", 4, 1)])
def test_merge_deferred_to_next_selection(gpu, dtype, G, k):
    """Layer 0 attends without merging; layer 1's selection merges it in the
    same launch; layer 1 attends and is merged on its own. Every output, score
    and selection holds the bits of the unpipelined calls (k = 1: rows are
    not split, the attention writes its output and the merge does nothing)."""
    w = small(dtype, B=3, Hq=2 * G, Hkv=2, k=k)
    L = _layers(gpu, w, 2)
    ref = []
    for l in range(2):
        s = gpu.select_forecast(L[l]["F"], L[l]["Kc"], w.T, w.q_start)
        i, o = gpu.topk_block_sparse_attn(s, L[l]["Q"], L[l]["K"], L[l]["V"], w.k, w.T, w.q_start)
        ref.append((s, i, o))
    nbytes = gpu.workspace_bytes(gpu.OP_BLOCK_SPARSE_ATTN, w.B, w.Hq, w.Hkv, 1, w.T, w.k)
    ws = torch.full((max(nbytes, 1),), 0x55, dtype=torch.uint8, device=DEV) if nbytes else None
    outs = [torch.full_like(L[l]["Q"], 7.0) for l in range(2)]
    s0 = gpu.select_forecast(L[0]["F"], L[0]["Kc"], w.T, w.q_start)
    i0, _ = gpu.topk_block_sparse_attn(s0, L[0]["Q"], L[0]["K"], L[0]["V"], w.k, w.T, w.q_start, out=outs[0], ws=ws,
                                       merge=False)
    s1 = gpu.select_forecast(L[1]["F"], L[1]["Kc"], w.T, w.q_start, merge_from=(ws, outs[0], w.T, w.k))
    i1, _ = gpu.topk_block_sparse_attn(s1, L[1]["Q"], L[1]["K"], L[1]["V"], w.k, w.T, w.q_start, out=outs[1], ws=ws,
                                       merge=False)
    gpu.merge_partials(ws, outs[1], w.T, w.k, w.Hkv)
    torch.cuda.synchronize()
    for l, (s, i) in enumerate(((s0, i0), (s1, i1))):
        assert torch.equal(s, ref[l][0]), f"layer {l}: scores"
        assert torch.equal(i, ref[l][1]), f"layer {l}: selection"
        assert torch.equal(bits(outs[l]), bits(ref[l][2])), f"layer {l}: attention output"
    say(f"deferred merge {dtype} G {G} k {k}: same bits")


def test_merge_deferred_with_positions(gpu):
    """Per-sequence positions in both layers, one sequence with no candidate
    block yet: the same bits as without deferral."""
    w = small("bf16", B=5, Hq=8, Hkv=2, k=6)
    L = _layers(gpu, w, 2, seed0=60)
    q_pos = torch.tensor([w.T - 1, 70, 64 * 20 + 5, 300, 5], dtype=torch.int32, device=DEV)
    ref = []
    for l in range(2):
        s = gpu.select_forecast(L[l]["F"], L[l]["Kc"], w.T, 0, q_pos=q_pos)
        ref.append(gpu.topk_block_sparse_attn(s, L[l]["Q"], L[l]["K"], L[l]["V"], w.k, w.T, 0, q_pos=q_pos)[1])
    ws = torch.zeros(gpu.workspace_bytes(gpu.OP_BLOCK_SPARSE_ATTN, w.B, w.Hq, w.Hkv, 1, w.T, w.k), dtype=torch.uint8,
                     device=DEV)
    outs = [torch.empty_like(L[l]["Q"]) for l in range(2)]
    s0 = gpu.select_forecast(L[0]["F"], L[0]["Kc"], w.T, 0, q_pos=q_pos)
    gpu.topk_block_sparse_attn(s0, L[0]["Q"], L[0]["K"], L[0]["V"], w.k, w.T, 0, out=outs[0], ws=ws, q_pos=q_pos,
                               merge=False)
    s1 = gpu.select_forecast(L[1]["F"], L[1]["Kc"], w.T, 0, q_pos=q_pos, merge_from=(ws, outs[0], w.T, w.k))
    gpu.topk_block_sparse_attn(s1, L[1]["Q"], L[1]["K"], L[1]["V"], w.k, w.T, 0, out=outs[1], ws=ws, q_pos=q_pos,
                               merge=False)
    gpu.merge_partials(ws, outs[1], w.T, w.k, w.Hkv)
    torch.cuda.synchronize()
    for l in range(2):
        assert torch.equal(bits(outs[l]), bits(ref[l])), f"layer {l}"
        assert not outs[l][4].float().any(), "a sequence with no visible block attends to nothing"


def test_merge_deferred_graph_replay(gpu):
    """Two pipelined layers captured in a HIP graph give the eager bits on every
    replay, with eager work and synchronisations between replays."""
    w = wl.C2_DECODE_32K
    L = _layers(gpu, w, 2, seed0=80)
    ws = torch.zeros(gpu.workspace_bytes(gpu.OP_BLOCK_SPARSE_ATTN, w.B, w.Hq, w.Hkv, 1, w.T, w.k), dtype=torch.uint8,
                     device=DEV)
    sc = [torch.empty((w.B, w.Hkv, 1, w.nB), dtype=torch.float32, device=DEV) for _ in range(2)]
    ix = [torch.empty((w.B, w.Hkv, 1, w.k), dtype=torch.int32, device=DEV) for _ in range(2)]
    outs = [torch.empty_like(L[l]["Q"]) for l in range(2)]

    def run():
        gpu.select_forecast(L[0]["F"], L[0]["Kc"], w.T, w.q_start, out=sc[0])
        gpu.topk_block_sparse_attn(sc[0], L[0]["Q"], L[0]["K"], L[0]["V"], w.k, w.T, w.q_start, idx=ix[0],
                                   out=outs[0], ws=ws, merge=False)
        gpu.select_forecast(L[1]["F"], L[1]["Kc"], w.T, w.q_start, out=sc[1], merge_from=(ws, outs[0], w.T, w.k))
        gpu.topk_block_sparse_attn(sc[1], L[1]["Q"], L[1]["K"], L[1]["V"], w.k, w.T, w.q_start, idx=ix[1],
                                   out=outs[1], ws=ws, merge=False)
        gpu.merge_partials(ws, outs[1], w.T, w.k, w.Hkv)

    run()
    torch.cuda.synchronize()
    ref = [t.clone() for t in sc + ix + outs]
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        run()
    torch.cuda.current_stream().wait_stream(side)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        run()
    for rep in range(4):
        for t in sc + outs:
            t.zero_()
        for t in ix:
            t.fill_(-7)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for got, want in zip(sc + ix + outs, ref):
            assert torch.equal(bits(got) if got.dtype == torch.bfloat16 else got,
                               bits(want) if want.dtype == torch.bfloat16 else want), f"replay {rep}"
        run()  # eager work between replays
        torch.cuda.synchronize()


# ------------------------------------------------ one launch per decode layer ----
def _attn_rows_oracle(Q, K, V, idx_np, positions, scale):
    """fp64 oracle attention of every (sequence, query head) at decode, reading
    only the selected keys of each row (the big caches stay on the GPU)."""
    B, Hq = Q.shape[0], Q.shape[1]
    Hkv = K.shape[1]
    G = Hq // Hkv
    out = np.zeros((B, Hq, 1, Q.shape[-1]))
    Q64 = parity.to_f64(Q)
    for b in range(B):
        for h in range(Hkv):
            J = oracle.selected_keys(idx_np[b, h, 0], positions[b])
            if J.size == 0:
                continue
            Jt = torch.from_numpy(J).to(K.device)
            KJ, VJ = parity.to_f64(K[b, h].index_select(0, Jt)), parity.to_f64(V[b, h].index_select(0, Jt))
            for g in range(G):
                out[b, h * G + g, 0] = oracle.attend(Q64[b, h * G + g, 0], KJ, VJ, scale)
    return out


@pytest.mark.parametrize("B,Hkv,G,k,ragged", [(3, 2, 4, 5, False), (3, 2, 4, 37, False), (3, 2, 2, 20, True),
                                              (3, 2, 8, 9, False), (3, 2, 4, 1, False),
                                              (12, 8, 4, 5, False), (12, 8, 4, 37, True), (12, 8, 8, 9, False),
                                              (16, 8, 1, 3, False), (12, 8, 2, 1, False)])
def test_decode_layer_chain(gpu, B, Hkv, G, k, ragged):
    """Three layers, each one sparda_decode_layer call (this layer's top-k +
    attention, finished, and the next layer's selection in the same launch).
    Every layer's scores and selection hold the bits of the separate calls;
    the outputs match the oracle run with that selection, and, for batches
    of fewer than 96 rows (block ranges merged by a second launch, as the
    separate calls do), also the separate calls' bits. 96 rows and more take
    one workgroup per row, merged in LDS."""
    w = small("bf16", B=B, Hq=G * Hkv, Hkv=Hkv, k=k)
    rows = B * Hkv
    L = _layers(gpu, w, 3, seed0=90)
    pos = [w.T - 1, 64 * 9 + 3, 300] + [w.T - 1 - 7 * i for i in range(3, B)] if ragged else [w.q_start] * B
    q_pos = torch.tensor(pos, dtype=torch.int32, device=DEV) if ragged else None
    qs = 0 if ragged else w.q_start
    ref = []
    for l in range(3):
        s = gpu.select_forecast(L[l]["F"], L[l]["Kc"], w.T, qs, q_pos=q_pos)
        i, o = gpu.topk_block_sparse_attn(s, L[l]["Q"], L[l]["K"], L[l]["V"], w.k, w.T, qs, q_pos=q_pos)
        ref.append((s, i, o))
    nbytes = gpu.workspace_bytes(gpu.OP_DECODE_LAYER, w.B, w.Hq, w.Hkv, 1, w.T, w.k)
    assert nbytes == 0 or rows < 96  # (a row of one block range needs none either)
    ws = torch.full((max(nbytes, 1),), 0x33, dtype=torch.uint8, device=DEV) if nbytes else None
    sc = [torch.full((w.B, w.Hkv, 1, w.nB), 7.0, dtype=torch.float32, device=DEV) for _ in range(3)]
    outs = [torch.full_like(L[l]["Q"], 3.0) for l in range(3)]
    ix = [torch.full((w.B, w.Hkv, 1, w.k), -9, dtype=torch.int32, device=DEV) for _ in range(3)]
    gpu.select_forecast(L[0]["F"], L[0]["Kc"], w.T, qs, out=sc[0], q_pos=q_pos)
    for l in range(3):
        nxt = (L[l + 1]["F"], L[l + 1]["Kc"], sc[l + 1], w.T, qs, q_pos) if l < 2 else None
        gpu.decode_layer(sc[l], L[l]["Q"], L[l]["K"], L[l]["V"], w.k, w.T, qs, ws, idx=ix[l], out=outs[l],
                         q_pos=q_pos, select_next=nxt)
    torch.cuda.synchronize()
    worst = 0.0
    for l in range(3):
        assert torch.equal(sc[l], ref[l][0]), f"layer {l}: scores"
        assert torch.equal(ix[l], ref[l][1]), f"layer {l}: selection"
        if rows < 96:
            assert torch.equal(bits(outs[l]), bits(ref[l][2])), f"layer {l}: attention output"
        want = _attn_rows_oracle(L[l]["Q"], L[l]["K"], L[l]["V"], ix[l].cpu().numpy(), pos, w.scale)
        worst = max(worst, parity.check_attention(parity.to_f64(outs[l]), want, parity.ATTN_ATOL_BF16))
    say(f"decode_layer chain rows {rows} G {G} k {k} ragged {ragged}: max abs err {worst:.2e}")


def test_decode_layer_c3_shape(gpu):
    """The batch-16 128K shape the benchmark times, two layers: the first
    call's selection of the second layer and both layers' top-k hold the bits
    of the separate calls; every one of the 512 query heads' outputs matches
    the oracle run with that selection."""
    w = wl.C3_DECODE_128K
    L = _layers(gpu, w, 2, seed0=5)
    ref = []
    for l in range(2):
        s = gpu.select_forecast(L[l]["F"], L[l]["Kc"], w.T, w.q_start)
        ref.append((s,) + gpu.topk_block_sparse_attn(s, L[l]["Q"], L[l]["K"], L[l]["V"], w.k, w.T, w.q_start))
    assert gpu.workspace_bytes(gpu.OP_DECODE_LAYER, w.B, w.Hq, w.Hkv, 1, w.T, w.k) == 0
    s0 = gpu.select_forecast(L[0]["F"], L[0]["Kc"], w.T, w.q_start)
    s1 = torch.empty_like(s0)
    i0, o0 = gpu.decode_layer(s0, L[0]["Q"], L[0]["K"], L[0]["V"], w.k, w.T, w.q_start,
                              select_next=(L[1]["F"], L[1]["Kc"], s1, w.T, w.q_start))
    i1, o1 = gpu.decode_layer(s1, L[1]["Q"], L[1]["K"], L[1]["V"], w.k, w.T, w.q_start)
    torch.cuda.synchronize()
    for l, (s, i, o) in enumerate(((s0, i0, o0), (s1, i1, o1))):
        assert torch.equal(s, ref[l][0]) and torch.equal(i, ref[l][1]), f"layer {l}: scores/selection"
        want = _attn_rows_oracle(L[l]["Q"], L[l]["K"], L[l]["V"], i.cpu().numpy(), [w.q_start] * w.B, w.scale)
        err = parity.check_attention(parity.to_f64(o), want, parity.ATTN_ATOL_BF16)
        # against the split-and-merge call: the same terms summed in another order
        diff = float((o.float() - ref[l][2].float()).abs().max())
        say(f"c3 layer {l}: max abs err vs oracle {err:.2e}, vs split call {diff:.2e}")
        assert diff <= parity.ATTN_ATOL_BF16


def test_decode_layer_rejects_overlapping_scores(gpu):
    """The next layer's scores are written in the launch that reads this
    layer's: one buffer for both is refused before anything runs."""
    w = small("bf16", B=12, Hq=32, Hkv=8, k=5)
    L = _layers(gpu, w, 1, seed0=3)
    s = gpu.select_forecast(L[0]["F"], L[0]["Kc"], w.T, w.q_start)
    with pytest.raises(gpu.SpardaError, match="must not overlap"):
        gpu.decode_layer(s, L[0]["Q"], L[0]["K"], L[0]["V"], w.k, w.T, w.q_start,
                         select_next=(L[0]["F"], L[0]["Kc"], s, w.T, w.q_start))
