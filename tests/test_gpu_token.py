"""GPU parity of the token-level Forecast variant (token scores, the top-k of
long rows, attention over the kept tokens) against the fp64 oracle, through the
C ABI of libsparda.so. Inputs come from the seeded generator; the oracle sees
the exact stored bits."""

import numpy as np
import pytest
import torch

import kv_block_selection_amd as kbs
import oracle
import synth.gpu as sg
from synth import workloads as wl
from tests import parity

pytestmark = pytest.mark.gpu
DEV = "cuda"


def say(*a):
    print(*a, flush=True)


def gen(w: wl.Workload, name: str, shape=None):
    return sg.tensor(w.recipe(name, 0), shape or w.shape(name), DEV)


def small(dtype="bf16", **kw):
    base = dict(name="small_tokens", description="token-level decode", dtype=dtype, B=2, Hq=8, Hkv=2, T=64 * 37,
                d=128, Tq=1, q_start=64 * 37 - 1, k=5, seed=21, block_offsets=dtype == "bf16",
                value_scale=wl.INV_SQRT_128 if dtype == "fp32" else None)
    base.update(kw)
    if "T" in kw and "q_start" not in kw:
        base["q_start"] = kw["T"] - 1
    return wl.Workload(**base)


def tol(dtype):
    return parity.ATTN_ATOL_BF16 if dtype == "bf16" else 1e-4


@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
@pytest.mark.parametrize("ragged", [False, True])
def test_select_tokens_parity(gpu, dtype, ragged):
    w = small(dtype, T=64 * 37 + 20)  # a ragged tail of key rows
    say("select_tokens", dtype, "ragged", ragged)
    F, K = gen(w, "F"), gen(w, "K")
    pos = [w.T - 1, 300] if ragged else None
    q_pos = torch.tensor(pos, dtype=torch.int32, device=DEV) if ragged else None
    s = kbs.select_tokens(F, K, w.q_start, scale=w.scale, q_pos=q_pos)
    torch.cuda.synchronize()
    ref = oracle.forecast_token_scores(parity.to_f64(F), parity.to_f64(K), w.q_start, w.scale, positions=pos)
    parity.check_scores(parity.to_f64(s), ref)


@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
def test_select_tokens_unaligned_rows(gpu, dtype):
    """Rows of an odd length T, and an output that starts 4 bytes past a
    16-byte boundary: the scores that cannot leave as aligned 16-byte pieces
    take the kernel's 4-byte stores. The floats around the output stay
    untouched."""
    w = small(dtype, T=64 * 9 + 13)
    say("select_tokens unaligned", dtype, "T", w.T)
    F, K = gen(w, "F"), gen(w, "K")
    n = w.B * w.Hkv * w.T
    buf = torch.full((n + 2,), 7.0, dtype=torch.float32, device=DEV)
    out = buf[1 : n + 1].view(w.B, w.Hkv, 1, w.T)
    assert out.data_ptr() % 16 != 0
    kbs.select_tokens(F, K, w.q_start, scale=w.scale, out=out)
    torch.cuda.synchronize()
    ref = oracle.forecast_token_scores(parity.to_f64(F), parity.to_f64(K), w.q_start, w.scale)
    parity.check_scores(parity.to_f64(out), ref)
    assert float(buf[0]) == 7.0 and float(buf[-1]) == 7.0


def test_select_tokens_nothing_visible(gpu):
    w = small()
    F, K = gen(w, "F"), gen(w, "K")
    q_pos = torch.tensor([-1, 0], dtype=torch.int32, device=DEV)
    s = kbs.select_tokens(F, K, w.q_start, q_pos=q_pos).cpu().numpy()
    assert np.all(np.isneginf(s[0])) and np.isfinite(s[1, :, 0, 0]).all() and np.all(np.isneginf(s[1, :, 0, 1:]))


def _tie_rows(rng, rows, n, n_ninf):
    """Scores on a coarse grid (many exact ties) with some -inf entries."""
    x = (np.round(rng.standard_normal((rows, n)) * 8) / 8).astype(np.float32)
    for r in range(rows):
        x[r, rng.choice(n, size=min(n_ninf, n), replace=False)] = -np.inf
    return x


@pytest.mark.parametrize("n", [8193, 20000, 131072])
def test_topk_long_rows_exact(gpu, n):
    rng = np.random.default_rng(n)
    x = _tie_rows(rng, 4, n, n // 7)
    n_cand = int(np.isfinite(x[0]).sum())
    dev = torch.from_numpy(x).to(DEV)
    for k in (1, 100, 4096, n_cand - 1, n_cand, n_cand + 5, n):
        say("topk long", n, "k", k)
        got = kbs.topk_blocks(dev, k).cpu().numpy()
        want = oracle.topk_blocks(x.astype(np.float64), k)
        np.testing.assert_array_equal(got, want)


@pytest.mark.parametrize("n,k", [(131072, 4096), (50000, 1000), (8193, 64)])
def test_topk_long_rows_sampled_path(gpu, n, k):
    """Distinct scores, so the candidates above the sampled threshold are
    enough and fit: exact against the oracle (one row a third -inf)."""
    rng = np.random.default_rng(n + k)
    x = rng.standard_normal((3, n)).astype(np.float32)
    x[1, rng.choice(n, size=n // 3, replace=False)] = -np.inf
    say("topk long sampled", n, "k", k)
    got = kbs.topk_blocks(torch.from_numpy(x).to(DEV), k).cpu().numpy()
    np.testing.assert_array_equal(got, oracle.topk_blocks(x.astype(np.float64), k))


def test_topk_long_rows_degenerate(gpu):
    n = 10000
    x = np.full((3, n), -np.inf, dtype=np.float32)
    x[1, 7] = 1.0                      # one candidate
    x[2, :] = 0.5                      # all equal: the lowest indices win
    x[2, 9000] = -0.0                  # -0 ranks with +0, below 0.5
    got = kbs.topk_blocks(torch.from_numpy(x).to(DEV), 64).cpu().numpy()
    np.testing.assert_array_equal(got, oracle.topk_blocks(x.astype(np.float64), 64))
    assert np.all(got[0] == -1) and got[1, 0] == 7 and np.all(got[1, 1:] == -1)
    assert np.array_equal(got[2], np.arange(64))


@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
@pytest.mark.parametrize("G", [1, 4, 8])
def test_token_path_parity(gpu, dtype, G):
    """Scores, top-k and attention chained on the GPU; attention against the
    oracle run with the GPU's own selection, the selection by the band rule."""
    w = small(dtype, Hq=2 * G)
    k_tok = 320
    say("token path", dtype, "G", G)
    F, K, V, Q = gen(w, "F"), gen(w, "K"), gen(w, "V"), gen(w, "Q")
    s = kbs.select_tokens(F, K, w.q_start, scale=w.scale)
    idx = kbs.topk_blocks(s, k_tok)
    out = kbs.token_sparse_attn(Q, K, V, idx, w.q_start, scale=w.scale)
    torch.cuda.synchronize()
    ref_s = oracle.forecast_token_scores(parity.to_f64(F), parity.to_f64(K), w.q_start, w.scale)
    parity.check_topk_band(idx.cpu().numpy(), ref_s, k_tok)
    gi = idx.cpu().numpy()
    ref = oracle.token_sparse_attention(parity.to_f64(Q), parity.to_f64(K), parity.to_f64(V), gi, w.q_start, w.scale)
    err = parity.check_attention(parity.to_f64(out), ref, tol(dtype))
    say(f"  max abs err {err:.2e}")


def test_token_attention_ragged_positions_and_padding(gpu):
    """Per-sequence positions (one sequence sees nothing, one sees fewer tokens
    than k_tok), padding in the middle of a row and tokens in any order."""
    w = small("bf16", B=3)
    k_tok = 192
    Q, K, V = gen(w, "Q"), gen(w, "K"), gen(w, "V")
    rng = np.random.default_rng(5)
    idx = np.stack([rng.permutation(w.T)[:k_tok] for _ in range(w.B * w.Hkv)]).astype(np.int32)
    idx[:, 10:20] = -1
    idx[1, 50] = w.T - 1
    idx = idx.reshape(w.B, w.Hkv, 1, k_tok)
    pos = [w.T - 1, -1, 100]
    q_pos = torch.tensor(pos, dtype=torch.int32, device=DEV)
    out = kbs.token_sparse_attn(Q, K, V, torch.from_numpy(idx).to(DEV), w.q_start, scale=w.scale, q_pos=q_pos)
    torch.cuda.synchronize()
    ref = oracle.token_sparse_attention(parity.to_f64(Q), parity.to_f64(K), parity.to_f64(V), idx, w.q_start,
                                        w.scale, positions=pos)
    parity.check_attention(parity.to_f64(out), ref, tol("bf16"))
    assert np.all(parity.to_f64(out)[1] == 0)


def test_token_attention_short_cache(gpu):
    """A cache shorter than one 64-token block (T = 40, 1 and 63): the kept
    list (written by hand: the top-k needs k <= T) is padded with -1, and the
    64-entry list is one range, so the call needs no workspace."""
    for T in (40, 1, 63):
        w = small("bf16", T=T)
        k_tok = 64
        say("token attention, short cache T =", T)
        Q, K, V = gen(w, "Q"), gen(w, "K"), gen(w, "V")
        need = kbs.workspace_bytes(kbs.OP_TOKEN_ATTN, w.B, w.Hq, w.Hkv, 1, T, k_tok)
        assert need == 0
        rng = np.random.default_rng(T)
        idx = np.full((w.B, w.Hkv, 1, k_tok), -1, dtype=np.int32)
        for b in range(w.B):
            for h in range(w.Hkv):
                keep = rng.permutation(T)[: max(1, T // 2)]
                idx[b, h, 0, rng.choice(k_tok, keep.size, replace=False)] = keep
        out = kbs.token_sparse_attn(Q, K, V, torch.from_numpy(idx).to(DEV), w.q_start, scale=w.scale)
        torch.cuda.synchronize()
        ref = oracle.token_sparse_attention(parity.to_f64(Q), parity.to_f64(K), parity.to_f64(V), idx, w.q_start,
                                            w.scale)
        parity.check_attention(parity.to_f64(out), ref, tol("bf16"))


def test_token_attention_reused_workspace(gpu):
    """Two calls on one workspace, the second with fewer kept tokens visible:
    no staging slot of the first call leaks into the second."""
    w = small("bf16")
    k_tok = 256
    Q, K, V = gen(w, "Q"), gen(w, "K"), gen(w, "V")
    need = kbs.workspace_bytes(kbs.OP_TOKEN_ATTN, w.B, w.Hq, w.Hkv, 1, w.T, k_tok)
    ws = torch.empty(need, dtype=torch.uint8, device=DEV)
    idx1 = torch.arange(k_tok, dtype=torch.int32, device=DEV).repeat(w.B, w.Hkv, 1, 1)
    kbs.token_sparse_attn(Q, K, V, idx1, w.q_start, scale=w.scale, ws=ws)
    idx2 = idx1.clone()
    idx2[..., 40:] = -1
    out2 = kbs.token_sparse_attn(Q, K, V, idx2, w.q_start, scale=w.scale, ws=ws)
    torch.cuda.synchronize()
    ref = oracle.token_sparse_attention(parity.to_f64(Q), parity.to_f64(K), parity.to_f64(V), idx2.cpu().numpy(),
                                        w.q_start, w.scale)
    parity.check_attention(parity.to_f64(out2), ref, tol("bf16"))


def test_token_path_128k_rows(gpu):
    """The benchmark's shape per row (T = 131072, k_tok = 4096, 4 heads per
    group) on one sequence: scores and attention against the oracle, the top-k
    of the GPU's scores exactly as the oracle takes it."""
    w = wl.C3_DECODE_128K
    B, k_tok = 1, 4096
    say("token path 128K, B", B)
    F = gen(w, "F", shape=(B, w.Hkv, 1, w.d))
    K = gen(w, "K", shape=(B, w.Hkv, w.T, w.d))
    V = gen(w, "V", shape=(B, w.Hkv, w.T, w.d))
    Q = gen(w, "Q", shape=(B, w.Hq, 1, w.d))
    s = kbs.select_tokens(F, K, w.q_start, scale=w.scale)
    idx = kbs.topk_blocks(s, k_tok)
    out = kbs.token_sparse_attn(Q, K, V, idx, w.q_start, scale=w.scale)
    torch.cuda.synchronize()
    s64 = s.cpu().numpy().astype(np.float64)
    np.testing.assert_array_equal(idx.cpu().numpy(), oracle.topk_blocks(s64, k_tok))
    for h in (0, 5):  # sampled rows of the scores
        ref_s = oracle.forecast_token_scores(parity.to_f64(F[:, h:h + 1]), parity.to_f64(K[:, h:h + 1]), w.q_start,
                                             w.scale)
        parity.check_scores(s64[:, h:h + 1], ref_s)
    gi = idx.cpu().numpy()
    G = w.Hq // w.Hkv
    for h in (0, 7):  # attention of two KV heads' groups
        Kh = parity.to_f64(K[:, h:h + 1, :, :][:, :, torch.from_numpy(np.sort(gi[0, h, 0])).to(DEV).long()])
        Vh = parity.to_f64(V[:, h:h + 1, :, :][:, :, torch.from_numpy(np.sort(gi[0, h, 0])).to(DEV).long()])
        local = np.arange(k_tok, dtype=np.int32).reshape(1, 1, 1, k_tok)
        ref = oracle.token_sparse_attention(parity.to_f64(Q[:, G * h:G * h + G]), Kh, Vh, local, k_tok - 1, w.scale)
        parity.check_attention(parity.to_f64(out[:, G * h:G * h + G]), ref, tol("bf16"))


def test_token_path_graph_replay(gpu):
    """Scores, top-k of long rows and attention over the kept tokens captured
    in one HIP graph: every replay (with eager work and synchronisations in
    between, and the outputs overwritten first) gives the eager bits."""
    w = small("bf16", T=64 * 160)  # rows of 10240 scores: the streaming top-k
    k_tok = 512
    F, K, V, Q = gen(w, "F"), gen(w, "K"), gen(w, "V"), gen(w, "Q")
    scores = torch.empty((w.B, w.Hkv, 1, w.T), dtype=torch.float32, device=DEV)
    idx = torch.empty((w.B, w.Hkv, 1, k_tok), dtype=torch.int32, device=DEV)
    out = torch.empty_like(Q)
    ws = torch.empty(kbs.workspace_bytes(kbs.OP_TOKEN_ATTN, w.B, w.Hq, w.Hkv, 1, w.T, k_tok), dtype=torch.uint8,
                     device=DEV)

    def step():
        kbs.select_tokens(F, K, w.q_start, scale=w.scale, out=scores)
        kbs.topk_blocks(scores, k_tok, out=idx)
        kbs.token_sparse_attn(Q, K, V, idx, w.q_start, scale=w.scale, out=out, ws=ws)

    step()
    torch.cuda.synchronize()
    ref_s, ref_i, ref_o = scores.clone(), idx.clone(), out.clone()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    for rep in range(3):
        scores.fill_(-1.0)
        idx.fill_(-7)
        out.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(scores, ref_s), f"replay {rep}: scores"
        assert torch.equal(idx, ref_i), f"replay {rep}: idx"
        assert torch.equal(out.view(torch.int16), ref_o.view(torch.int16)), f"replay {rep}: attention"
        step()  # eager work between replays
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int16), ref_o.view(torch.int16))
