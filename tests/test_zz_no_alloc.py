"""The decode top-k + attention call that allocates nothing
(sparda_topk_block_sparse_attn_noalloc: its block ranges' results in the
library's static device array) against the call with a caller-owned
workspace, through the C ABI: two calls in a row, the second on a smaller
batch, each with the same selection and output bits."""

import pytest
import torch

import kv_block_selection_amd as kbs
import synth.gpu as sg
from synth import workloads as wl

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _inputs(gpu, w):
    Q, K, V, F = (sg.tensor(w.recipe(n), w.shape(n), DEV) for n in ("Q", "K", "V", "F"))
    scores = gpu.select_forecast(F, gpu.compress_keys(K), w.T, w.q_start)
    return scores, Q, K, V


def _bits(t):
    return t.view(torch.int16) if t.dtype == torch.bfloat16 else t.view(torch.int32)


@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
def test_noalloc_matches_workspace_call_twice(gpu, dtype):
    big = wl.Workload(name="noalloc_big", description="", dtype=dtype, B=16, Hq=32, Hkv=8, T=64 * 37, d=128, Tq=1,
                      q_start=64 * 37 - 1, k=9, seed=71, block_offsets=dtype == "bf16",
                      value_scale=wl.INV_SQRT_128 if dtype == "fp32" else None)
    small = wl.scaled(big, B=3, Hq=16, Hkv=2, T=64 * 20, q_start=64 * 20 - 1, k=5, seed=72)
    for w in (big, small):  # the second call's rows sit where the first left its results
        print("noalloc", dtype, "B", w.B, "Hkv", w.Hkv, "T", w.T, "k", w.k, flush=True)
        assert kbs.workspace_bytes(kbs.OP_BLOCK_SPARSE_ATTN, w.B, w.Hq, w.Hkv, 1, w.T, w.k) > 0
        scores, Q, K, V = _inputs(gpu, w)
        idx_ref, out_ref = gpu.topk_block_sparse_attn(scores, Q, K, V, w.k, w.T, w.q_start)
        idx, out = gpu.topk_block_sparse_attn_noalloc(scores, Q, K, V, w.k, w.T, w.q_start)
        torch.cuda.synchronize()
        assert torch.equal(idx, idx_ref)
        assert torch.equal(_bits(out), _bits(out_ref))
