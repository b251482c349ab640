"""GPU parity of the Q/K/V/Forecast projection GEMM against the fp64 oracle,
through the C ABI of libsparda.so: the decode batch of the 128K configuration
(B = 16), the offload batch (B = 64) with the first layer's two Forecast sets,
batches that end inside a 16-sequence tile or span two 64-sequence grid rows,
no Forecast (n_f = 0), and no write outside the outputs. Hidden states and
random weights come from the seeded generator."""

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


def _case(gpu, w, B, D, n_f, sentinel=False):
    wB = wl.scaled(w, B=B)
    x = sg.tensor(wl.hidden_recipe(wB), (B, D), DEV)
    W = sg.tensor(wl.qkvf_weight_recipe(wB, D), (wl.qkvf_rows(wB, n_f), D), DEV)
    shapes = [(B, w.Hq, 1, w.d), (B, w.Hkv, 1, w.d), (B, w.Hkv, 1, w.d), (n_f, B, w.Hkv, 1, w.d)]
    if sentinel:
        # each output is the front of a larger buffer whose tail must stay untouched
        bufs = [torch.full((int(np.prod(s)) + 4096,), 512.0, dtype=torch.bfloat16, device=DEV) for s in shapes]
        out = [b[: int(np.prod(s))].view(s) for b, s in zip(bufs, shapes)]
        if n_f == 0:
            out[3] = None
        q, k, v, f = gpu.project_qkvf(x, W, w.Hq, w.Hkv, n_f, out=tuple(out))
    else:
        q, k, v, f = gpu.project_qkvf(x, W, w.Hq, w.Hkv, n_f)
    torch.cuda.synchronize()
    x64, W64 = parity.to_f64(x), parity.to_f64(W)
    ref = oracle.project_qkvf(x64, W64, w.Hq, w.Hkv, n_f, w.d)
    abs_ref = oracle.project_qkvf(np.abs(x64), np.abs(W64), w.Hq, w.Hkv, n_f, w.d)
    worst = 0.0
    for got, r, a in zip((q, k, v, f), ref, abs_ref):
        if r is None:
            assert got is None
            continue
        worst = max(worst, parity.check_projection(parity.to_f64(got), r, a, D))
    if sentinel:
        for b, s in zip(bufs, shapes):
            tail = b[int(np.prod(s)):]
            assert (tail == 512.0).all().item(), "projection wrote past an output"
    return worst


@pytest.mark.parametrize("B,D,n_f", [(16, wl.MODEL_DIM, 1), (64, wl.MODEL_DIM, 2), (3, 512, 0), (70, 1024, 1),
                                     (17, 2048, 1), (40, 1536, 1), (33, 512, 1)])
def test_projection_parity(gpu, B, D, n_f):
    say("project_qkvf B", B, "D", D, "n_f", n_f)
    worst = _case(gpu, wl.C3_DECODE_128K, B, D, n_f)
    say(f"  worst error / bound {worst:.3f}")


def test_projection_writes_only_its_outputs(gpu):
    for B, n_f in ((3, 0), (33, 2)):
        say("project_qkvf sentinels B", B, "n_f", n_f)
        _case(gpu, wl.C3_DECODE_128K, B, 512, n_f, sentinel=True)


def test_projection_gqa_groups(gpu):
    """Group sizes 1 and 8 (the head counts move the K/V/Forecast row offsets)."""
    for Hq, Hkv in ((8, 8), (16, 2)):
        w = wl.scaled(wl.C3_DECODE_128K, Hq=Hq, Hkv=Hkv)
        say("project_qkvf Hq", Hq, "Hkv", Hkv)
        _case(gpu, w, 5, 512, 2)


def test_projection_feeds_forecast_selection(gpu):
    """The Forecast vectors the projection emits drive selection as inputs of
    their own would: select + top-k on the GPU's F against the oracle chain."""
    w = wl.scaled(wl.C3_DECODE_128K, B=2, T=64 * 37, q_start=64 * 37 - 1, k=5)
    D = 1024
    x = sg.tensor(wl.hidden_recipe(w), (w.B, D), DEV)
    W = sg.tensor(wl.qkvf_weight_recipe(w, D), (wl.qkvf_rows(w, 1), D), DEV)
    q, k, v, f = gpu.project_qkvf(x, W, w.Hq, w.Hkv, 1)
    K = sg.tensor(w.recipe("K"), w.shape("K"), DEV)
    Kc = gpu.compress_keys(K)
    F = f[0]
    s = gpu.select_forecast(F, Kc, w.T, w.q_start)
    idx = gpu.topk_blocks(s, w.k)
    torch.cuda.synchronize()
    ref = oracle.select_forecast(parity.to_f64(F), parity.to_f64(Kc), w.T, w.q_start, w.scale)
    parity.check_scores(parity.to_f64(s), ref)
    parity.check_topk_band(idx.cpu().numpy(), ref, w.k)
