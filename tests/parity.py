"""Comparison rules between the HIP path and the fp64 oracle.

* Block scores: the -inf pattern must match exactly; each finite score must be
  within 1e-3 * max(|ref|, rho) of the oracle, rho = RMS of the row's finite
  oracle scores (relative error stays meaningful for scores near zero).
* Block indices: let s_k be the oracle's k-th best score of the row and
  delta = 1e-3 * max(|s_k|, rho). Every block scoring above s_k + delta must be
  selected, every selected block must score at least s_k - delta, the row holds
  exactly min(k, #candidates) distinct ascending indices then -1 padding.
  Outside that band the sets are identical.
* Attention: max |O_gpu - O_ref| <= 2e-2 for bf16 inputs (fp32 accumulation).
* Compressed keys, bf16: within one bf16 ulp of the exact mean; fp32: within
  the recursive-summation bound 32 * 2^-24 * mean|k| of the window.
"""

from __future__ import annotations

import numpy as np

import oracle
import synth

SCORE_RTOL = 1e-3
ATTN_ATOL_BF16 = 2e-2


def to_f64(t) -> np.ndarray:
    """fp64 copy of a torch tensor (bf16/fp32/int) on any device."""
    import torch
    if t.dtype == torch.bfloat16:
        bits = t.detach().contiguous().view(torch.int16).cpu().numpy().view(np.uint16)
        return synth.bf16_bits_to_f32(bits).astype(np.float64)
    return t.detach().cpu().numpy().astype(np.float64)


def _rho(ref_row: np.ndarray) -> float:
    fin = ref_row[np.isfinite(ref_row)]
    return float(np.sqrt(np.mean(fin ** 2))) if fin.size else 0.0


def check_scores(gpu: np.ndarray, ref: np.ndarray, rtol: float = SCORE_RTOL) -> float:
    """Returns the worst |err| / max(|ref|, rho); raises on failure."""
    g = gpu.reshape(-1, gpu.shape[-1])
    r = ref.reshape(-1, ref.shape[-1])
    worst = 0.0
    for i in range(r.shape[0]):
        ninf_r = np.isneginf(r[i])
        ninf_g = np.isneginf(g[i])
        assert np.array_equal(ninf_r, ninf_g), f"row {i}: -inf pattern differs"
        assert np.isfinite(g[i][~ninf_g]).all(), f"row {i}: NaN/inf in GPU scores"
        fin = ~ninf_r
        if not fin.any():
            continue
        denom = np.maximum(np.abs(r[i][fin]), _rho(r[i]))
        denom = np.where(denom > 0, denom, 1.0)
        rel = np.abs(g[i][fin] - r[i][fin]) / denom
        worst = max(worst, float(rel.max()))
        assert rel.max() <= rtol, f"row {i}: score error {rel.max():.3g} > {rtol}"
    return worst


def check_topk_band(gpu_idx: np.ndarray, ref_scores: np.ndarray, k: int, rtol: float = SCORE_RTOL) -> int:
    """Band rule for selected sets; returns the number of rows whose set differs
    from the oracle's own top-k (all within the band)."""
    gi = gpu_idx.reshape(-1, gpu_idx.shape[-1])
    rs = ref_scores.reshape(-1, ref_scores.shape[-1])
    banded = 0
    for i in range(rs.shape[0]):
        row = rs[i]
        n_cand = int(np.count_nonzero(np.isfinite(row)))
        kk = min(k, n_cand)
        sel = gi[i][:kk]
        assert np.all(gi[i][kk:] == -1), f"row {i}: padding"
        assert np.all(sel >= 0) and np.all(np.diff(sel) > 0), f"row {i}: not ascending/distinct: {sel}"
        if kk == 0:
            continue
        assert np.isfinite(row[sel]).all(), f"row {i}: selected a non-candidate"
        ref_sel = oracle.topk_row(row, k)[:kk]
        if np.array_equal(ref_sel, sel):
            continue
        banded += 1
        s_k = np.sort(row[np.isfinite(row)])[::-1][kk - 1]
        delta = rtol * max(abs(s_k), _rho(row))
        must = np.nonzero(row > s_k + delta)[0]
        assert set(must.tolist()) <= set(sel.tolist()), f"row {i}: missed a block clearly above the k-th score"
        assert np.all(row[sel] >= s_k - delta), f"row {i}: selected a block clearly below the k-th score"
    return banded


def check_attention(gpu: np.ndarray, ref: np.ndarray, atol: float) -> float:
    err = float(np.max(np.abs(gpu - ref))) if gpu.size else 0.0
    assert np.isfinite(gpu).all(), "non-finite attention output"
    assert err <= atol, f"attention max abs error {err:.3g} > {atol}"
    return err


def bf16_ulp(x: np.ndarray) -> np.ndarray:
    ax = np.abs(x)
    e = np.floor(np.log2(np.where(ax > 0, ax, 1.0)))
    ulp = np.exp2(e - 7)
    return np.where(ax > 0, ulp, 2.0 ** -133)


def check_compress(gpu: np.ndarray, ref: np.ndarray, dtype: str, mean_abs: np.ndarray | None = None) -> float:
    err = np.abs(gpu - ref)
    if dtype == "bf16":
        tol = bf16_ulp(ref)
        assert np.all(err <= tol), f"compressed keys off by more than 1 bf16 ulp: max {float((err / tol).max())} ulp"
        return float((err / tol).max())
    assert mean_abs is not None
    tol = 32 * 2.0 ** -24 * mean_abs + 1e-30
    assert np.all(err <= tol), f"fp32 compressed keys beyond the summation bound: {float((err / tol).max())}"
    return float((err / tol).max())


def check_projection(gpu: np.ndarray, ref: np.ndarray, abs_sum: np.ndarray, D: int) -> float:
    """bf16 projections accumulated in fp32: each output may differ from the
    exact fp64 dot product by the fp32 summation bound D * 2^-24 * sum|x w|
    plus the final rounding to bf16 (half an ulp, 2^-9 |value|; 2^-8 |ref|
    allows for the value itself being off by the summation error). Returns the
    largest error as a fraction of its bound."""
    bound = 2.0 ** -8 * np.abs(ref) + D * 2.0 ** -24 * abs_sum
    err = np.abs(gpu - ref)
    worst = float((err / bound).max()) if err.size else 0.0
    assert worst <= 1.0, f"projection error {err.max():.3e} exceeds its bound (worst ratio {worst:.2f})"
    return worst
