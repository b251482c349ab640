"""Python binding of libsparda.so: SparDA block selection and block-sparse
attention on MI355X.

Argument marshalling only: every step runs in the HIP kernels of libsparda.so,
reached through its C ABI (include/sparda.h). torch supplies device memory and
the current stream. There is no fallback: if the library is missing, ``load()``
raises.
"""

from __future__ import annotations

import ctypes
import os

# SPARDA_LIB names another build of the same library (the host-sanitized one
# of the CPU tests); by default the in-tree build
LIB_PATH = os.environ.get("SPARDA_LIB") or os.path.join(os.path.dirname(os.path.abspath(__file__)), "libsparda.so")

SPARDA_OK = 0
SPARDA_F32 = 0
SPARDA_BF16 = 1
KV_CACHE = 0
KV_STAGING = 1
KV_SLOTS = 2
OP_SELECT_FORECAST = 1
OP_SELECT_MULTIHEAD = 2
OP_BLOCK_SPARSE_ATTN = 3
OP_TOKEN_ATTN = 4
OP_DECODE_LAYER = 5

HEAD_DIM = 128
BLOCK = 64
KERNEL = 32
STRIDE = 16
TILE = 64

_c = ctypes
_vp, _i, _f, _sz = _c.c_void_p, _c.c_int, _c.c_float, _c.c_size_t

# name -> (restype, argtypes), exactly as declared in include/sparda.h
SIGNATURES = {
    "sparda_compress_keys": (_i, [_vp, _vp, _i, _i, _i, _i, _i, _i, _i, _vp]),
    "sparda_compress_windows": (_i, [_vp, _vp, _i, _i, _i, _i, _i, _i, _i, _i, _i, _i, _vp]),
    "sparda_append_kv": (_i, [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _i, _i, _i, _i, _i, _i, _i, _i, _i, _vp]),
    "sparda_select_forecast": (_i, [_vp, _vp, _vp, _i, _i, _i, _i, _i, _vp, _i, _i, _i, _i, _i, _i, _f, _vp, _sz,
                                    _vp]),
    "sparda_select_multihead": (_i, [_vp, _vp, _vp, _i, _i, _i, _i, _i, _i, _vp, _i, _i, _i, _i, _i, _i, _f, _vp,
                                     _sz, _vp]),
    "sparda_topk_blocks": (_i, [_vp, _vp, _i, _i, _i, _vp]),
    "sparda_block_sparse_attn": (_i, [_vp, _vp, _vp, _i, _vp, _vp, _i, _vp, _i, _i, _i, _i, _i, _i, _vp, _i, _i, _i,
                                      _i, _i, _f, _vp, _sz, _vp]),
    "sparda_prefetch_blocks": (_i, [_vp, _vp, _vp, _vp, _vp, _i, _i, _i, _i, _i, _i, _i, _i, _vp]),
    "sparda_prefetch_blocks_cached": (_i, [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _i, _i, _i, _i, _i, _i, _i, _i, _i,
                                           _vp]),
    "sparda_project_qkvf": (_i, [_vp, _vp, _vp, _vp, _vp, _vp, _i, _i, _i, _i, _i, _i, _i, _vp]),
    "sparda_topk_block_sparse_attn": (_i, [_vp, _vp, _vp, _vp, _vp, _vp, _i, _i, _i, _i, _i, _vp, _i, _i, _i, _i, _f,
                                           _vp, _sz, _vp]),
    "sparda_topk_block_sparse_attn_noalloc": (_i, [_vp, _vp, _vp, _vp, _vp, _vp, _i, _i, _i, _i, _i, _vp, _i, _i, _i,
                                                   _i, _f, _vp]),
    "sparda_topk_block_sparse_attn_partial": (_i, [_vp, _vp, _vp, _vp, _vp, _vp, _i, _i, _i, _i, _i, _vp, _i, _i, _i,
                                                   _i, _f, _vp, _sz, _vp]),
    "sparda_merge_partials": (_i, [_vp, _sz, _vp, _i, _i, _i, _i, _i, _i, _i, _vp]),
    "sparda_decode_layer": (_i, [_vp, _vp, _vp, _vp, _vp, _vp, _i, _i, _vp, _i, _i, _f, _vp, _sz, _vp, _vp, _vp, _i,
                                 _vp, _i, _f, _i, _i, _i, _i, _i, _i, _i, _vp]),
    "sparda_select_forecast_merge": (_i, [_vp, _vp, _vp, _i, _i, _i, _i, _vp, _i, _i, _i, _i, _i, _f, _vp, _sz, _vp,
                                          _i, _i, _i, _vp]),
    "sparda_select_tokens": (_i, [_vp, _vp, _vp, _i, _i, _i, _i, _i, _vp, _i, _f, _vp]),
    "sparda_token_sparse_attn": (_i, [_vp, _vp, _vp, _vp, _vp, _i, _i, _i, _i, _i, _i, _vp, _i, _i, _f, _vp, _sz,
                                      _vp]),
    "sparda_workspace_bytes": (_sz, [_i, _i, _i, _i, _i, _i, _i, _i]),
    "sparda_status_string": (_c.c_char_p, [_i]),
    "sparda_last_error": (_c.c_char_p, []),
    "sparda_version": (_i, []),
}

_LIB = None


class SpardaError(RuntimeError):
    def __init__(self, status: int, call: str, message: str):
        self.status = status
        super().__init__(f"{call}: {_LIB.sparda_status_string(status).decode()}: {message}")


def load() -> ctypes.CDLL:
    """Load libsparda.so (built in-tree); raises if it is not built."""
    global _LIB
    if _LIB is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is not built; run `python -m kv_block_selection_amd.build`")
        lib = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            fn = getattr(lib, name)
            fn.restype = res
            fn.argtypes = args
        _LIB = lib
    return _LIB


def _call(name: str, *args) -> None:
    lib = load()
    st = getattr(lib, name)(*args)
    if st != SPARDA_OK:
        raise SpardaError(st, name, lib.sparda_last_error().decode())


# ------------------------------------------------------------ torch glue ----
def _torch():
    import torch
    return torch


def _dtype_code(t) -> int:
    torch = _torch()
    if t.dtype == torch.float32:
        return SPARDA_F32
    if t.dtype == torch.bfloat16:
        return SPARDA_BF16
    raise TypeError(f"unsupported dtype {t.dtype}; use float32 or bfloat16")


def _ptr(t):
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError("tensor must be on the GPU")
    if not t.is_contiguous():
        raise ValueError("tensor must be contiguous")
    return t.data_ptr()


def _stream(t, stream=None):
    torch = _torch()
    s = stream if stream is not None else torch.cuda.current_stream(t.device)
    return s.cuda_stream


def num_windows(T: int) -> int:
    return (T - KERNEL) // STRIDE + 1


def workspace_bytes(op: int, B: int, Hq: int, Hkv: int, Tq: int, T: int, k: int = 0) -> int:
    return int(load().sparda_workspace_bytes(op, B, Hq, Hkv, Tq, T, HEAD_DIM, k))


def _workspace(ws, nbytes: int, like):
    torch = _torch()
    if nbytes == 0:
        return None, 0
    if ws is None:
        # no initial contents are needed (every byte read is written first by the same call)
        ws = torch.empty(nbytes, dtype=torch.uint8, device=like.device)
    if ws.numel() * ws.element_size() < nbytes:
        raise ValueError(f"workspace has {ws.numel() * ws.element_size()} bytes, needs {nbytes}")
    return ws, ws.numel() * ws.element_size()


# ------------------------------------------------------------- the calls ----
def compress_keys(k, out=None, stream=None):
    """K [B, Hkv, T, 128] -> mean-pooled windows [B, Hkv, W, 128] (kernel 32, stride 16)."""
    torch = _torch()
    B, Hkv, T, d = k.shape
    if out is None:
        out = torch.empty((B, Hkv, num_windows(T), d), dtype=k.dtype, device=k.device)
    _call("sparda_compress_keys", _ptr(k), _ptr(out), _dtype_code(k), B, Hkv, T, d, KERNEL, STRIDE,
          _stream(k, stream))
    return out


def compress_windows(k, k_cmp, w_begin: int, w_end: int, stream=None):
    """Windows [w_begin, w_end) of K cache rows [B, Hkv, T_cap, 128] into k_cmp
    [B, Hkv, W_cap, 128] (the other windows are left as they are)."""
    B, Hkv, T_cap, d = k.shape
    W_cap = k_cmp.shape[2]
    if k_cmp.shape[:2] != (B, Hkv) or k_cmp.dtype != k.dtype:
        raise ValueError("k_cmp must be [B, Hkv, W_cap, 128] in k's dtype")
    _call("sparda_compress_windows", _ptr(k), _ptr(k_cmp), _dtype_code(k), B, Hkv, T_cap, W_cap, d, KERNEL, STRIDE,
          w_begin, w_end, _stream(k, stream))
    return k_cmp


def _positions(q_pos, B: int):
    """Per-sequence query positions: None, or an int32 device tensor [B]."""
    torch = _torch()
    if q_pos is None:
        return None
    if q_pos.dtype != torch.int32 or q_pos.numel() != B:
        raise ValueError(f"q_pos must be an int32 tensor of {B} positions")
    return _ptr(q_pos)


def append_kv(k_new, v_new, k_cache, v_cache, seq_len, k_cmp=None, status=None, stream=None):
    """Write k_new/v_new [B, Hkv, n_new, 128] into the caches [B, Hkv, T_cap, 128]
    at positions seq_len[b] .. seq_len[b] + n_new - 1 (seq_len: int32 device [B],
    not changed) and compress into k_cmp [B, Hkv, W_cap, 128] every window the
    new tokens complete. status (int32 device [1], optional) gets 1 OR-ed in when
    a sequence's tokens do not fit; that sequence is left untouched."""
    torch = _torch()
    B, Hkv, n_new, d = k_new.shape
    T_cap = k_cache.shape[2]
    W_cap = k_cmp.shape[2] if k_cmp is not None else 0
    for t in (v_new, k_cache, v_cache) + ((k_cmp,) if k_cmp is not None else ()):
        if t.dtype != k_new.dtype or t.shape[:2] != (B, Hkv) or t.shape[3] != d:
            raise ValueError("k_new, v_new, caches and k_cmp must share dtype, [B, Hkv] and d")
    if v_new.shape != k_new.shape or v_cache.shape != k_cache.shape:
        raise ValueError("k_new/v_new and k_cache/v_cache must have equal shapes")
    if seq_len.dtype != torch.int32 or seq_len.numel() != B:
        raise ValueError(f"seq_len must be an int32 tensor of {B} lengths")
    if status is not None and status.dtype != torch.int32:
        raise ValueError("status must be int32")
    _call("sparda_append_kv", _ptr(k_new), _ptr(v_new), _ptr(k_cache), _ptr(v_cache), _ptr(k_cmp), _ptr(seq_len),
          _ptr(status), _dtype_code(k_new), B, Hkv, n_new, T_cap, W_cap, d, KERNEL, STRIDE, _stream(k_new, stream))


def select_forecast(f, k_cmp, T: int, q_start: int, scale: float | None = None, out=None, stream=None, q_pos=None,
                    merge_from=None):
    """Forecast block scores [B, Hkv, nTiles, nB] (float32) for F [B, Hkv, Tq, 128].
    q_pos (int32 device [B], decode only) gives each sequence its own position.
    merge_from = (ws, out, T, k_sel) of a topk_block_sparse_attn(..., merge=False)
    call with the same B and Hkv (decode only): that attention's merge runs in
    the same launch."""
    torch = _torch()
    B, Hkv, Tq, d = f.shape
    scale = d ** -0.5 if scale is None else scale
    n_tiles = -(-Tq // TILE)
    if out is None:
        out = torch.empty((B, Hkv, n_tiles, T // BLOCK), dtype=torch.float32, device=f.device)
    if merge_from is not None:
        m_ws, m_out, m_T, m_k = merge_from
        m_bytes = m_ws.numel() * m_ws.element_size() if m_ws is not None else 0
        _call("sparda_select_forecast_merge", _ptr(f), _ptr(k_cmp), _ptr(out), _dtype_code(f), B, Hkv, q_start,
              _positions(q_pos, B), T, d, KERNEL, STRIDE, BLOCK, scale, _ptr(m_ws), m_bytes, _ptr(m_out),
              m_out.shape[1], m_T, m_k, _stream(f, stream))
        return out
    _call("sparda_select_forecast", _ptr(f), _ptr(k_cmp), _ptr(out), _dtype_code(f), B, Hkv, Tq, q_start,
          _positions(q_pos, B), T, d, KERNEL, STRIDE, BLOCK, TILE, scale, None, 0, _stream(f, stream))
    return out


def select_multihead(q, k_cmp, T: int, q_start: int, scale: float | None = None, out=None, ws=None,
                     stream=None, q_pos=None):
    """Multi-head-selector block scores [B, Hkv, nTiles, nB] (float32) for Q [B, Hq, Tq, 128]."""
    torch = _torch()
    B, Hq, Tq, d = q.shape
    Hkv = k_cmp.shape[1]
    scale = d ** -0.5 if scale is None else scale
    n_tiles = -(-Tq // TILE)
    if out is None:
        out = torch.empty((B, Hkv, n_tiles, T // BLOCK), dtype=torch.float32, device=q.device)
    ws, nbytes = _workspace(ws, workspace_bytes(OP_SELECT_MULTIHEAD, B, Hq, Hkv, Tq, T), q)
    _call("sparda_select_multihead", _ptr(q), _ptr(k_cmp), _ptr(out), _dtype_code(q), B, Hq, Hkv, Tq, q_start,
          _positions(q_pos, B), T, d, KERNEL, STRIDE, BLOCK, TILE, scale, _ptr(ws), nbytes, _stream(q, stream))
    return out


def topk_blocks(scores, k: int, out=None, stream=None):
    """Top-k block indices [..., k] int32 (ascending, -1 padded) of float32 scores [..., nB]."""
    torch = _torch()
    nB = scores.shape[-1]
    rows = scores.numel() // nB if nB else 0
    if out is None:
        out = torch.empty(tuple(scores.shape[:-1]) + (k,), dtype=torch.int32, device=scores.device)
    _call("sparda_topk_blocks", _ptr(scores), _ptr(out), rows, nB, k, _stream(scores, stream))
    return out


def block_sparse_attn(q, k, v, idx, T: int, q_start: int, scale: float | None = None, kv_mode: int = KV_CACHE,
                      out=None, ws=None, stream=None, q_pos=None, slot_of=None):
    """GQA block-sparse attention; O [B, Hq, Tq, 128] in q's dtype. With
    kv_mode KV_SLOTS, k/v are the cached staging [B, Hkv, n_slots, 64, 128]
    and slot_of [B, Hkv, k] (int32) says where each selected block sits."""
    torch = _torch()
    B, Hq, Tq, d = q.shape
    Hkv = k.shape[1]
    k_sel = idx.shape[-1]
    scale = d ** -0.5 if scale is None else scale
    if out is None:
        out = torch.empty_like(q)
    ws, nbytes = _workspace(ws, workspace_bytes(OP_BLOCK_SPARSE_ATTN, B, Hq, Hkv, Tq, T, k_sel), q)
    n_slots = k.shape[2] if kv_mode == KV_SLOTS else 0
    _call("sparda_block_sparse_attn", _ptr(q), _ptr(k), _ptr(v), kv_mode, _ptr(idx), _ptr(slot_of), n_slots,
          _ptr(out), _dtype_code(q), B, Hq, Hkv, Tq, q_start, _positions(q_pos, B), T, d, BLOCK, TILE, k_sel, scale,
          _ptr(ws), nbytes, _stream(q, stream))
    return out


def select_tokens(f, k, q_start: int, scale: float | None = None, out=None, stream=None, q_pos=None):
    """Token-level Forecast scores [B, Hkv, 1, T] float32 of every key token
    (scale * f . k[t] up to the query's position, -inf after it)."""
    torch = _torch()
    B, Hkv, T, d = k.shape
    scale = d ** -0.5 if scale is None else scale
    if out is None:
        out = torch.empty((B, Hkv, 1, T), dtype=torch.float32, device=k.device)
    _call("sparda_select_tokens", _ptr(f), _ptr(k), _ptr(out), _dtype_code(k), B, Hkv, T, q_start,
          _positions(q_pos, B), d, scale, _stream(k, stream))
    return out


def token_sparse_attn(q, k, v, tok_idx, q_start: int, scale: float | None = None, out=None, ws=None, stream=None,
                      q_pos=None):
    """GQA attention at decode over the kept tokens tok_idx [B, Hkv, 1, k_tok]
    (int32, -1 padded); O [B, Hq, 1, 128] in q's dtype."""
    torch = _torch()
    B, Hq, Tq, d = q.shape
    Hkv, T = k.shape[1], k.shape[2]
    k_tok = tok_idx.shape[-1]
    scale = d ** -0.5 if scale is None else scale
    if out is None:
        out = torch.empty_like(q)
    ws, nbytes = _workspace(ws, workspace_bytes(OP_TOKEN_ATTN, B, Hq, Hkv, 1, T, k_tok), q)
    _call("sparda_token_sparse_attn", _ptr(q), _ptr(k), _ptr(v), _ptr(tok_idx), _ptr(out), _dtype_code(q), B, Hq,
          Hkv, T, q_start, _positions(q_pos, B), d, k_tok, scale, _ptr(ws), nbytes, _stream(q, stream))
    return out


def project_qkvf(x, w, Hq: int, Hkv: int, n_f: int = 1, out=None, stream=None):
    """Q, K, V and n_f Forecast sets from hidden states x [B, D] and the
    concatenated weight rows w [(Hq + 2 Hkv + n_f Hkv) * 128, D] (bf16).
    Returns (q [B, Hq, 1, 128], k [B, Hkv, 1, 128], v [B, Hkv, 1, 128],
    f [n_f, B, Hkv, 1, 128] or None); ``out`` may give those four tensors."""
    torch = _torch()
    B, D = x.shape
    d = HEAD_DIM
    if w.shape != ((Hq + 2 * Hkv + n_f * Hkv) * d, D):
        raise ValueError(f"w has shape {tuple(w.shape)}, expected {((Hq + 2 * Hkv + n_f * Hkv) * d, D)}")
    if out is None:
        out = (torch.empty((B, Hq, 1, d), dtype=x.dtype, device=x.device),
               torch.empty((B, Hkv, 1, d), dtype=x.dtype, device=x.device),
               torch.empty((B, Hkv, 1, d), dtype=x.dtype, device=x.device),
               torch.empty((n_f, B, Hkv, 1, d), dtype=x.dtype, device=x.device) if n_f else None)
    q, k, v, f = out
    _call("sparda_project_qkvf", _ptr(x), _ptr(w), _ptr(q), _ptr(k), _ptr(v), _ptr(f), _dtype_code(x), B, D, Hq,
          Hkv, n_f, d, _stream(x, stream))
    return q, k, v, f


def topk_block_sparse_attn(scores, q, k, v, k_sel: int, T: int, q_start: int, scale: float | None = None,
                           idx=None, out=None, ws=None, stream=None, q_pos=None, merge: bool = True):
    """Top-k blocks of the decode scores [B, Hkv, 1, nB] and attention of q
    [B, Hq, 1, 128] over them, in one launch. Returns (idx [B, Hkv, 1, k_sel]
    int32, O [B, Hq, 1, 128]), the same bits as topk_blocks + block_sparse_attn.
    merge=False leaves the block ranges' results in ``ws`` (pass one): O is
    complete after merge_partials or select_forecast(..., merge_from=...)."""
    torch = _torch()
    B, Hq, Tq, d = q.shape
    Hkv = k.shape[1]
    if Tq != 1:
        raise ValueError("topk_block_sparse_attn is a decode call (one query per sequence)")
    scale = d ** -0.5 if scale is None else scale
    if idx is None:
        idx = torch.empty((B, Hkv, 1, k_sel), dtype=torch.int32, device=q.device)
    if out is None:
        out = torch.empty_like(q)
    need = workspace_bytes(OP_BLOCK_SPARSE_ATTN, B, Hq, Hkv, 1, T, k_sel)
    if not merge and ws is None and need > 0:
        raise ValueError("merge=False needs the workspace that will be merged later")
    ws, nbytes = _workspace(ws, need, q)
    name = "sparda_topk_block_sparse_attn" if merge else "sparda_topk_block_sparse_attn_partial"
    _call(name, _ptr(scores), _ptr(q), _ptr(k), _ptr(v), _ptr(idx), _ptr(out),
          _dtype_code(q), B, Hq, Hkv, q_start, _positions(q_pos, B), T, d, BLOCK, k_sel, scale, _ptr(ws), nbytes,
          _stream(q, stream))
    return idx, out


def topk_block_sparse_attn_noalloc(scores, q, k, v, k_sel: int, T: int, q_start: int, idx=None, out=None,
                                    scale=None, q_pos=None, stream=None):
    """topk_block_sparse_attn without a workspace: the library's static
    device array holds the block ranges' results (calls on one GPU share it
    and must not overlap). Returns (idx, out)."""
    torch = _torch()
    B, Hq, Tq, d = q.shape
    Hkv = k.shape[1]
    scale = d ** -0.5 if scale is None else scale
    if idx is None:
        idx = torch.empty((B, Hkv, 1, k_sel), dtype=torch.int32, device=q.device)
    if out is None:
        out = torch.empty_like(q)
    _call("sparda_topk_block_sparse_attn_noalloc", _ptr(scores), _ptr(q), _ptr(k), _ptr(v), _ptr(idx), _ptr(out),
          _dtype_code(q), B, Hq, Hkv, q_start, _positions(q_pos, B), T, d, BLOCK, k_sel, scale, _stream(q, stream))
    return idx, out


def decode_layer(scores, q, k, v, k_sel: int, T: int, q_start: int, ws=None, idx=None, out=None, scale=None,
                 q_pos=None, select_next=None, stream=None):
    """One decode layer (bf16): this layer's top-k of scores [B, Hkv, 1, nB]
    and attention of q [B, Hq, 1, 128], finished in ``out``, and optionally
    the next layer's Forecast selection in the same launch (select_next =
    (f_next, k_cmp_next, scores_next, T_next, q_start_next[, q_pos_next])).
    ``ws`` is needed only for batches of fewer than 96 (sequence, KV head)
    rows. Returns (idx, out)."""
    torch = _torch()
    B, Hq, Tq, d = q.shape
    Hkv = k.shape[1]
    scale = d ** -0.5 if scale is None else scale
    if idx is None:
        idx = torch.empty((B, Hkv, 1, k_sel), dtype=torch.int32, device=q.device)
    if out is None:
        out = torch.empty_like(q)
    ws, nbytes = _workspace(ws, workspace_bytes(OP_DECODE_LAYER, B, Hq, Hkv, 1, T, k_sel), q)
    f_n = kc_n = s_n = qp_n = None
    T_n = q_n = 0
    if select_next is not None:
        f_n, kc_n, s_n, T_n, q_n = select_next[:5]
        qp_n = select_next[5] if len(select_next) > 5 else None
    _call("sparda_decode_layer", _ptr(scores), _ptr(q), _ptr(k), _ptr(v), _ptr(idx), _ptr(out), Hq, q_start,
          _positions(q_pos, B), T, k_sel, scale, _ptr(ws), nbytes, _ptr(f_n), _ptr(kc_n), _ptr(s_n), q_n,
          _positions(qp_n, B), T_n, scale, _dtype_code(q), B, Hkv, d, BLOCK, KERNEL, STRIDE, _stream(q, stream))
    return idx, out


def merge_partials(ws, out, T: int, k_sel: int, Hkv: int, stream=None):
    """Merge the block-range results a topk_block_sparse_attn(..., merge=False)
    call left in ws into its output out [B, Hq, 1, 128]."""
    B, Hq = out.shape[0], out.shape[1]
    nbytes = ws.numel() * ws.element_size() if ws is not None else 0
    _call("sparda_merge_partials", _ptr(ws), nbytes, _ptr(out), _dtype_code(out), B, Hq, Hkv, T, HEAD_DIM, k_sel,
          _stream(out, stream))
    return out


def prefetch_blocks(host_k, host_v, idx, stage_k, stage_v, num_workgroups: int = 0, stream=None):
    """Gather the blocks idx [B, Hkv, k] of pinned host K/V [B, Hkv, T, 128] into
    device staging [B, Hkv, k, 64, 128], on ``stream`` (default: current)."""
    B, Hkv, T, d = host_k.shape
    if not (host_k.is_pinned() and host_v.is_pinned()):
        raise ValueError("host_k / host_v must be pinned host tensors")
    k_sel = idx.shape[-1]
    _call("sparda_prefetch_blocks", host_k.data_ptr(), host_v.data_ptr(), _ptr(idx), _ptr(stage_k), _ptr(stage_v),
          _dtype_code(host_k), B, Hkv, T // BLOCK, BLOCK, d, k_sel, num_workgroups, _stream(idx, stream))
    return stage_k, stage_v


def prefetch_blocks_cached(host_k, host_v, idx, slot_tags, slot_of, stage_k, stage_v, num_workgroups: int = 0,
                           stream=None):
    """Fetch into the cached staging [B, Hkv, n_slots, 64, 128] only the
    blocks of idx [B, Hkv, k] that its slot_tags [B, Hkv, n_slots] (int32,
    -1 = empty; updated) do not hold; slot_of [B, Hkv, k] (int32) receives
    each selected block's slot."""
    torch = _torch()
    B, Hkv, T, d = host_k.shape
    if not (host_k.is_pinned() and host_v.is_pinned()):
        raise ValueError("host_k / host_v must be pinned host tensors")
    k_sel = idx.shape[-1]
    n_slots = stage_k.shape[2]
    if slot_tags.dtype != torch.int32 or slot_tags.numel() != B * Hkv * n_slots:
        raise ValueError("slot_tags must be int32 [B, Hkv, n_slots]")
    if slot_of.dtype != torch.int32 or slot_of.numel() != B * Hkv * k_sel:
        raise ValueError("slot_of must be int32 [B, Hkv, k]")
    _call("sparda_prefetch_blocks_cached", host_k.data_ptr(), host_v.data_ptr(), _ptr(idx), _ptr(slot_tags),
          _ptr(slot_of), _ptr(stage_k), _ptr(stage_v), _dtype_code(host_k), B, Hkv, T // BLOCK, BLOCK, d, k_sel,
          n_slots, num_workgroups, _stream(idx, stream))
    return slot_of
