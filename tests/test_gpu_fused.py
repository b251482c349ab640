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
    """Per-sequence query positions: the same bits as the separate calls."""
    w = small("bf16", B=4, Hq=8, Hkv=2, k=6)
    q_pos = torch.tensor([w.T - 1, 70, 64 * 20 + 5, 31], dtype=torch.int32, device=DEV)
    _case(gpu, w, q_pos=q_pos)
