// C ABI of libsparda.so: argument validation on the host, then dispatch to the
// kernels. Nothing is enqueued when validation fails; no C++ exception leaves
// this file.
#include <hip/hip_runtime.h>
#include <stdarg.h>
#include <stdio.h>

#include <cmath>
#include <string>

#include "launch.h"
#include "sparda.h"

#define SPARDA_EXPORT extern "C" __attribute__((visibility("default")))

namespace {

thread_local std::string g_last_error;

int fail(int status, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return status;
}

int ok() {
  g_last_error.clear();
  return SPARDA_OK;
}

int hip_status(hipError_t e, const char* what) {
  if (e != hipSuccess) return fail(SPARDA_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
  return ok();
}

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

#define CHECK(cond, status, ...) \
  do {                           \
    if (!(cond)) return fail(status, __VA_ARGS__); \
  } while (0)

#define CHECK_PTR(p)                                                                 \
  do {                                                                               \
    if ((p) == nullptr) return fail(SPARDA_ERR_INVALID_ARG, "%s is NULL", #p);       \
    if (!aligned16(p)) return fail(SPARDA_ERR_INVALID_ARG, "%s is not 16-byte aligned", #p); \
  } while (0)

int check_dtype(int dtype) {
  if (dtype != SPARDA_F32 && dtype != SPARDA_BF16)
    return fail(SPARDA_ERR_INVALID_ARG, "dtype %d is neither SPARDA_F32 nor SPARDA_BF16", dtype);
  return SPARDA_OK;
}

// Geometry shared by selection and attention.
int check_geometry(int B, int Hq, int Hkv, int Tq, int q_start, int T, int d) {
  CHECK(B >= 0, SPARDA_ERR_INVALID_ARG, "B = %d < 0", B);
  CHECK(Hkv >= 1 && Hq >= 1, SPARDA_ERR_INVALID_ARG, "head counts must be >= 1 (Hq %d, Hkv %d)", Hq, Hkv);
  CHECK(Hq % Hkv == 0, SPARDA_ERR_INVALID_ARG, "Hq %d is not a multiple of Hkv %d", Hq, Hkv);
  const int G = Hq / Hkv;
  CHECK(G == 1 || G == 2 || G == 4 || G == 8, SPARDA_ERR_UNSUPPORTED, "GQA group %d not in {1,2,4,8}", G);
  CHECK(d == sparda::kHeadDim, SPARDA_ERR_UNSUPPORTED, "head dim %d != 128", d);
  CHECK(T >= sparda::kBlock && T % sparda::kBlock == 0, SPARDA_ERR_UNSUPPORTED,
        "T = %d must be a positive multiple of 64", T);
  CHECK(Tq >= 1, SPARDA_ERR_INVALID_ARG, "Tq = %d < 1", Tq);
  CHECK(Tq == 1 || Tq % sparda::kTile == 0, SPARDA_ERR_UNSUPPORTED, "Tq = %d is neither 1 nor a multiple of 64", Tq);
  CHECK(q_start >= 0 && (long)q_start + Tq <= T, SPARDA_ERR_INVALID_ARG,
        "the query chunk must lie inside the cache: q_start %d + Tq %d > T %d", q_start, Tq, T);
  CHECK((long)B * Hkv <= 65535, SPARDA_ERR_UNSUPPORTED, "B*Hkv = %ld exceeds 65535", (long)B * Hkv);
  return SPARDA_OK;
}

int check_select_params(int kernel, int stride, int block, int tile, float scale) {
  CHECK(kernel == sparda::kKernel && stride == sparda::kStride, SPARDA_ERR_UNSUPPORTED,
        "compression kernel/stride %d/%d != 32/16", kernel, stride);
  CHECK(block == sparda::kBlock, SPARDA_ERR_UNSUPPORTED, "block %d != 64", block);
  CHECK(tile == sparda::kTile, SPARDA_ERR_UNSUPPORTED, "tile %d != 64", tile);
  CHECK(std::isfinite(scale), SPARDA_ERR_INVALID_ARG, "scale is not finite");
  return SPARDA_OK;
}

// Default workgroups of the host-memory gathers. The techwalker.com article
// (section 三) sizes the grid by batch for H100 (16 below batch 32, else 32);
// on MI355X the host link
// saturates from 32 workgroups at any batch measured (16 and 64 sequences),
// and 128 sits in the middle of that plateau.
constexpr int kGatherWorkgroups = 128;

int check_q_pos(const int* q_pos, int Tq) {
  if (q_pos == nullptr) return SPARDA_OK;
  CHECK(Tq == 1, SPARDA_ERR_UNSUPPORTED, "per-sequence positions (q_pos) need Tq = 1, got Tq = %d", Tq);
  CHECK(((uintptr_t)q_pos & 3u) == 0, SPARDA_ERR_INVALID_ARG, "q_pos is not 4-byte aligned");
  return SPARDA_OK;
}

sparda::SelectDims select_dims(int B, int Hq, int Hkv, int Tq, int q_start, int T, float scale) {
  sparda::SelectDims s;
  s.B = B;
  s.Hq = Hq;
  s.Hkv = Hkv;
  s.Tq = Tq;
  s.q_start = q_start;
  s.T = T;
  s.W = (T - sparda::kKernel) / sparda::kStride + 1;
  s.q_pos = nullptr;
  s.nB = T / sparda::kBlock;
  s.n_tiles = (Tq + sparda::kTile - 1) / sparda::kTile;
  s.scale = scale;
  return s;
}

sparda::AttnDims attn_dims(int B, int Hq, int Hkv, int Tq, int q_start, int T, int k, float scale,
                           int kv_mode) {
  sparda::AttnDims a;
  a.B = B;
  a.Hq = Hq;
  a.Hkv = Hkv;
  a.Tq = Tq;
  a.q_start = q_start;
  a.T = T;
  a.q_pos = nullptr;
  a.slot_of = nullptr;
  a.n_slots = 0;
  a.nB = T / sparda::kBlock;
  a.n_tiles = (Tq + sparda::kTile - 1) / sparda::kTile;
  a.k = k;
  a.scale = scale;
  a.kv_mode = kv_mode;
  return a;
}

size_t ws_bytes_for(int op, int B, int Hq, int Hkv, int Tq, int T, int k) {
  if (B <= 0 || Hkv <= 0 || Hq <= 0) return 0;
  if (op == SPARDA_OP_TOKEN_ATTN) {  // k = k_tok: the attention's block-range results over k_tok / 64 slots; any T >= 1
    if (Tq != 1 || T < 1 || k < sparda::kBlock || k % sparda::kBlock != 0) return 0;
    return sparda::decode_attn_ws_bytes(attn_dims(B, Hq, Hkv, 1, T - 1, T, k / sparda::kBlock, 1.f, 0));
  }
  if (T < sparda::kBlock) return 0;
  const int q_start = T - Tq;
  switch (op) {
    case SPARDA_OP_SELECT_FORECAST:
      return 0;
    case SPARDA_OP_SELECT_MULTIHEAD:
      if (Tq == 1) return sparda::multihead_decode_ws_bytes(select_dims(B, Hq, Hkv, Tq, q_start, T, 1.f));
      return 0;
    case SPARDA_OP_BLOCK_SPARSE_ATTN:
      if (Tq == 1) return sparda::decode_attn_ws_bytes(attn_dims(B, Hq, Hkv, Tq, q_start, T, k, 1.f, 0));
      return 0;
    case SPARDA_OP_DECODE_LAYER: {  // none when every row has a workgroup of its own
      const sparda::AttnDims ad = attn_dims(B, Hq, Hkv, 1, T - 1, T, k, 1.f, 0);
      return sparda::decode_layer_row_form(ad) ? 0 : sparda::decode_attn_ws_bytes(ad);
    }
    default:
      return 0;
  }
}

}  // namespace

SPARDA_EXPORT int sparda_version(void) { return 100; }  // 0.1.0

SPARDA_EXPORT const char* sparda_status_string(int status) {
  switch (status) {
    case SPARDA_OK: return "SPARDA_OK";
    case SPARDA_ERR_INVALID_ARG: return "SPARDA_ERR_INVALID_ARG";
    case SPARDA_ERR_UNSUPPORTED: return "SPARDA_ERR_UNSUPPORTED";
    case SPARDA_ERR_WORKSPACE: return "SPARDA_ERR_WORKSPACE";
    case SPARDA_ERR_HIP: return "SPARDA_ERR_HIP";
    default: return "SPARDA_ERR_UNKNOWN";
  }
}

SPARDA_EXPORT const char* sparda_last_error(void) { return g_last_error.c_str(); }

SPARDA_EXPORT size_t sparda_workspace_bytes(int op, int B, int Hq, int Hkv, int Tq, int T, int d, int k_sel) {
  (void)d;
  return ws_bytes_for(op, B, Hq, Hkv, Tq, T, k_sel);
}

SPARDA_EXPORT int sparda_compress_keys(const void* k, void* k_cmp, int dtype, int B, int Hkv, int T, int d,
                                       int kernel, int stride, void* stream) {
  if (int e = check_dtype(dtype)) return e;
  CHECK(B >= 0 && Hkv >= 1, SPARDA_ERR_INVALID_ARG, "B %d / Hkv %d out of range", B, Hkv);
  CHECK(d == sparda::kHeadDim, SPARDA_ERR_UNSUPPORTED, "head dim %d != 128", d);
  CHECK(kernel == sparda::kKernel && stride == sparda::kStride, SPARDA_ERR_UNSUPPORTED,
        "compression kernel/stride %d/%d != 32/16", kernel, stride);
  CHECK(T >= sparda::kBlock && T % sparda::kBlock == 0, SPARDA_ERR_UNSUPPORTED,
        "T = %d must be a positive multiple of 64", T);
  if (B == 0) return ok();
  CHECK_PTR(k);
  CHECK_PTR(k_cmp);
  const int W = (T - kernel) / stride + 1;
  return hip_status(sparda::launch_compress(k, k_cmp, dtype == SPARDA_BF16, B * Hkv, T, W, 0, W, (hipStream_t)stream),
                    "compress_keys launch");
}

SPARDA_EXPORT int sparda_compress_windows(const void* k, void* k_cmp, int dtype, int B, int Hkv, int T_cap, int W_cap,
                                          int d, int kernel, int stride, int w_begin, int w_end, void* stream) {
  if (int e = check_dtype(dtype)) return e;
  CHECK(B >= 0 && Hkv >= 1, SPARDA_ERR_INVALID_ARG, "B %d / Hkv %d out of range", B, Hkv);
  CHECK(d == sparda::kHeadDim, SPARDA_ERR_UNSUPPORTED, "head dim %d != 128", d);
  CHECK(kernel == sparda::kKernel && stride == sparda::kStride, SPARDA_ERR_UNSUPPORTED,
        "compression kernel/stride %d/%d != 32/16", kernel, stride);
  CHECK(T_cap >= kernel && W_cap >= 1, SPARDA_ERR_INVALID_ARG, "T_cap %d / W_cap %d too small", T_cap, W_cap);
  CHECK(0 <= w_begin && w_begin <= w_end && w_end <= W_cap, SPARDA_ERR_INVALID_ARG,
        "window range [%d, %d) not inside [0, W_cap = %d)", w_begin, w_end, W_cap);
  CHECK(w_end == 0 || (long)stride * (w_end - 1) + kernel <= T_cap, SPARDA_ERR_INVALID_ARG,
        "window %d needs tokens up to %ld, beyond T_cap = %d", w_end - 1, (long)stride * (w_end - 1) + kernel - 1,
        T_cap);
  if (B == 0 || w_begin == w_end) return ok();
  CHECK_PTR(k);
  CHECK_PTR(k_cmp);
  return hip_status(sparda::launch_compress(k, k_cmp, dtype == SPARDA_BF16, B * Hkv, T_cap, W_cap, w_begin, w_end,
                                            (hipStream_t)stream),
                    "compress_windows launch");
}

SPARDA_EXPORT int sparda_append_kv(const void* k_new, const void* v_new, void* k_cache, void* v_cache, void* k_cmp,
                                   const int* seq_len, int* status, int dtype, int B, int Hkv, int n_new, int T_cap,
                                   int W_cap, int d, int kernel, int stride, void* stream) {
  if (int e = check_dtype(dtype)) return e;
  CHECK(B >= 0 && Hkv >= 1, SPARDA_ERR_INVALID_ARG, "B %d / Hkv %d out of range", B, Hkv);
  CHECK(d == sparda::kHeadDim, SPARDA_ERR_UNSUPPORTED, "head dim %d != 128", d);
  CHECK(kernel == sparda::kKernel && stride == sparda::kStride, SPARDA_ERR_UNSUPPORTED,
        "compression kernel/stride %d/%d != 32/16", kernel, stride);
  CHECK(T_cap >= 1, SPARDA_ERR_INVALID_ARG, "T_cap = %d < 1", T_cap);
  CHECK(n_new >= 0 && n_new <= T_cap, SPARDA_ERR_INVALID_ARG, "n_new = %d outside 0..T_cap (%d)", n_new, T_cap);
  CHECK(k_cmp == nullptr || W_cap >= 1, SPARDA_ERR_INVALID_ARG, "W_cap = %d < 1 with k_cmp given", W_cap);
  CHECK((long)B * Hkv <= 2147483647L, SPARDA_ERR_UNSUPPORTED, "B*Hkv too large");
  CHECK(sparda::append_grid_y(dtype == SPARDA_BF16, n_new, k_cmp != nullptr) <= 65535, SPARDA_ERR_UNSUPPORTED,
        "n_new = %d too large for one call", n_new);
  if (B == 0 || n_new == 0) return ok();
  CHECK_PTR(k_new);
  CHECK_PTR(v_new);
  CHECK_PTR(k_cache);
  CHECK_PTR(v_cache);
  if (k_cmp != nullptr) CHECK_PTR(k_cmp);
  CHECK(seq_len != nullptr && ((uintptr_t)seq_len & 3u) == 0, SPARDA_ERR_INVALID_ARG,
        "seq_len is NULL or not 4-byte aligned");
  CHECK(((uintptr_t)status & 3u) == 0, SPARDA_ERR_INVALID_ARG, "status is not 4-byte aligned");
  return hip_status(sparda::launch_append_kv(k_new, v_new, k_cache, v_cache, k_cmp, seq_len, status,
                                             dtype == SPARDA_BF16, B, Hkv, n_new, T_cap, W_cap, (hipStream_t)stream),
                    "append_kv launch");
}

SPARDA_EXPORT int sparda_select_forecast(const void* f, const void* k_cmp, float* blk_scores, int dtype, int B,
                                         int Hkv, int Tq, int q_start, const int* q_pos, int T, int d, int kernel,
                                         int stride, int block, int tile, float scale, void* ws, size_t ws_bytes,
                                         void* stream) {
  (void)ws;
  (void)ws_bytes;
  if (int e = check_dtype(dtype)) return e;
  if (int e = check_geometry(B, Hkv, Hkv, Tq, q_start, T, d)) return e;
  if (int e = check_select_params(kernel, stride, block, tile, scale)) return e;
  if (B == 0) return ok();
  CHECK_PTR(f);
  CHECK_PTR(k_cmp);
  CHECK_PTR(blk_scores);
  if (int e = check_q_pos(q_pos, Tq)) return e;
  sparda::SelectDims sd = select_dims(B, Hkv, Hkv, Tq, q_start, T, scale);
  sd.q_pos = q_pos;
  if (Tq != 1) {
    CHECK(dtype == SPARDA_BF16, SPARDA_ERR_UNSUPPORTED, "select_forecast: a query chunk (Tq > 1) needs bf16 inputs");
    CHECK((long)B * Hkv <= 2147483647L && sd.n_tiles <= 65535, SPARDA_ERR_UNSUPPORTED, "grid too large");
    return hip_status(sparda::launch_select_forecast_prefill(f, k_cmp, blk_scores, sd, (hipStream_t)stream),
                      "select_forecast launch");
  }
  return hip_status(sparda::launch_select_forecast_decode(f, k_cmp, blk_scores, dtype == SPARDA_BF16, sd,
                                                          (hipStream_t)stream),
                    "select_forecast launch");
}

SPARDA_EXPORT int sparda_select_multihead(const void* q, const void* k_cmp, float* blk_scores, int dtype, int B,
                                          int Hq, int Hkv, int Tq, int q_start, const int* q_pos, int T, int d,
                                          int kernel, int stride, int block, int tile, float scale, void* ws,
                                          size_t ws_bytes, void* stream) {
  if (int e = check_dtype(dtype)) return e;
  if (int e = check_geometry(B, Hq, Hkv, Tq, q_start, T, d)) return e;
  if (int e = check_select_params(kernel, stride, block, tile, scale)) return e;
  if (B == 0) return ok();
  CHECK_PTR(q);
  CHECK_PTR(k_cmp);
  CHECK_PTR(blk_scores);
  const size_t need = ws_bytes_for(SPARDA_OP_SELECT_MULTIHEAD, B, Hq, Hkv, Tq, T, 0);
  CHECK(ws_bytes >= need, SPARDA_ERR_WORKSPACE, "select_multihead needs %zu workspace bytes, got %zu", need, ws_bytes);
  if (need) CHECK_PTR(ws);
  if (int e = check_q_pos(q_pos, Tq)) return e;
  sparda::SelectDims sd = select_dims(B, Hq, Hkv, Tq, q_start, T, scale);
  sd.q_pos = q_pos;
  if (Tq != 1) {
    CHECK(dtype == SPARDA_BF16, SPARDA_ERR_UNSUPPORTED, "select_multihead: a query chunk (Tq > 1) needs bf16 inputs");
    CHECK(sd.n_tiles <= 65535, SPARDA_ERR_UNSUPPORTED, "grid too large");
    return hip_status(sparda::launch_select_multihead_prefill(q, k_cmp, blk_scores, sd, (hipStream_t)stream),
                      "select_multihead launch");
  }
  return hip_status(sparda::launch_select_multihead_decode(q, k_cmp, blk_scores, dtype == SPARDA_BF16, sd, ws,
                                                           (hipStream_t)stream),
                    "select_multihead launch");
}

SPARDA_EXPORT int sparda_topk_blocks(const float* blk_scores, int32_t* idx, int rows, int nB, int k, void* stream) {
  CHECK(rows >= 0, SPARDA_ERR_INVALID_ARG, "rows = %d < 0", rows);
  CHECK(nB >= 1 && nB <= (1 << 26), SPARDA_ERR_UNSUPPORTED, "row length %d outside 1..2^26", nB);
  CHECK(k >= 1 && k <= nB, SPARDA_ERR_INVALID_ARG, "k = %d outside 1..nB (%d)", k, nB);
  CHECK(rows <= 2147483647, SPARDA_ERR_UNSUPPORTED, "too many rows");
  if (rows == 0) return ok();
  CHECK(blk_scores != nullptr && ((uintptr_t)blk_scores & 3u) == 0, SPARDA_ERR_INVALID_ARG,
        "blk_scores is NULL or not 4-byte aligned");
  CHECK(idx != nullptr && ((uintptr_t)idx & 3u) == 0, SPARDA_ERR_INVALID_ARG, "idx is NULL or not 4-byte aligned");
  if (nB > 8192)  // long rows (token scores): the streaming top-k
    return hip_status(sparda::launch_topk_long(blk_scores, idx, rows, nB, k, (hipStream_t)stream), "topk launch");
  return hip_status(sparda::launch_topk(blk_scores, idx, rows, nB, k, (hipStream_t)stream), "topk launch");
}

SPARDA_EXPORT int sparda_block_sparse_attn(const void* q, const void* k, const void* v, int kv_mode,
                                           const int32_t* idx, const int32_t* slot_of, int n_slots, void* out,
                                           int dtype, int B, int Hq, int Hkv,
                                           int Tq, int q_start, const int* q_pos, int T, int d, int block, int tile,
                                           int k_sel, float scale, void* ws, size_t ws_bytes, void* stream) {
  if (int e = check_dtype(dtype)) return e;
  if (int e = check_geometry(B, Hq, Hkv, Tq, q_start, T, d)) return e;
  CHECK(block == sparda::kBlock, SPARDA_ERR_UNSUPPORTED, "block %d != 64", block);
  CHECK(tile == sparda::kTile, SPARDA_ERR_UNSUPPORTED, "tile %d != 64", tile);
  CHECK(std::isfinite(scale), SPARDA_ERR_INVALID_ARG, "scale is not finite");
  CHECK(kv_mode == SPARDA_KV_CACHE || kv_mode == SPARDA_KV_STAGING || kv_mode == SPARDA_KV_SLOTS,
        SPARDA_ERR_INVALID_ARG, "kv_mode %d", kv_mode);
  CHECK(k_sel >= 1 && k_sel <= T / sparda::kBlock, SPARDA_ERR_INVALID_ARG, "k = %d outside 1..nB (%d)", k_sel,
        T / sparda::kBlock);
  CHECK(kv_mode == SPARDA_KV_CACHE || Tq == 1, SPARDA_ERR_UNSUPPORTED, "staging mode is decode-only (Tq = 1)");
  if (kv_mode == SPARDA_KV_SLOTS) {
    CHECK(n_slots >= k_sel && n_slots <= sparda::kCacheMaxSlots, SPARDA_ERR_INVALID_ARG,
          "n_slots = %d outside k (%d) .. %d", n_slots, k_sel, sparda::kCacheMaxSlots);
    CHECK(B == 0 || (slot_of != nullptr && ((uintptr_t)slot_of & 3u) == 0), SPARDA_ERR_INVALID_ARG,
          "slot_of is NULL or not 4-byte aligned");
  }
  if (B == 0) return ok();
  CHECK_PTR(q);
  CHECK_PTR(k);
  CHECK_PTR(v);
  CHECK_PTR(out);
  CHECK(idx != nullptr && ((uintptr_t)idx & 3u) == 0, SPARDA_ERR_INVALID_ARG, "idx is NULL or not 4-byte aligned");
  const size_t need = ws_bytes_for(SPARDA_OP_BLOCK_SPARSE_ATTN, B, Hq, Hkv, Tq, T, k_sel);
  CHECK(ws_bytes >= need, SPARDA_ERR_WORKSPACE, "block_sparse_attn needs %zu workspace bytes, got %zu", need,
        ws_bytes);
  if (need) CHECK_PTR(ws);
  if (int e = check_q_pos(q_pos, Tq)) return e;
  sparda::AttnDims ad = attn_dims(B, Hq, Hkv, Tq, q_start, T, k_sel, scale, kv_mode);
  ad.q_pos = q_pos;
  ad.slot_of = kv_mode == SPARDA_KV_SLOTS ? slot_of : nullptr;
  ad.n_slots = kv_mode == SPARDA_KV_SLOTS ? n_slots : 0;
  if (Tq != 1) {
    CHECK(dtype == SPARDA_BF16, SPARDA_ERR_UNSUPPORTED, "block_sparse_attn: a query chunk (Tq > 1) needs bf16 inputs");
    CHECK(ad.n_tiles <= 65535, SPARDA_ERR_UNSUPPORTED, "too many query tiles");
    return hip_status(sparda::launch_attn_prefill(q, k, v, idx, out, ad, (hipStream_t)stream),
                      "block_sparse_attn launch");
  }
  return hip_status(sparda::launch_attn_decode(q, k, v, idx, out, dtype == SPARDA_BF16, ad, ws, (hipStream_t)stream),
                    "block_sparse_attn launch");
}

namespace {
int topk_attn_impl(const float* blk_scores, const void* q, const void* k, const void* v, int32_t* idx, void* out,
                   int dtype, int B, int Hq, int Hkv, int q_start, const int* q_pos, int T, int d, int block,
                   int k_sel, float scale, void* ws, size_t ws_bytes, bool merge, void* stream, const char* name) {
  if (int e = check_dtype(dtype)) return e;
  if (int e = check_geometry(B, Hq, Hkv, 1, q_start, T, d)) return e;
  CHECK(block == sparda::kBlock, SPARDA_ERR_UNSUPPORTED, "block %d != 64", block);
  CHECK(std::isfinite(scale), SPARDA_ERR_INVALID_ARG, "scale is not finite");
  const int nB = T / sparda::kBlock;
  CHECK(nB <= 8192, SPARDA_ERR_UNSUPPORTED, "%s: nB = %d above 8192", name, nB);
  CHECK(k_sel >= 1 && k_sel <= nB, SPARDA_ERR_INVALID_ARG, "k = %d outside 1..nB (%d)", k_sel, nB);
  CHECK(k_sel <= 1024, SPARDA_ERR_UNSUPPORTED, "%s: k = %d above 1024", name, k_sel);
  if (B == 0) return ok();
  CHECK(blk_scores != nullptr && ((uintptr_t)blk_scores & 3u) == 0, SPARDA_ERR_INVALID_ARG,
        "blk_scores is NULL or not 4-byte aligned");
  CHECK_PTR(q);
  CHECK_PTR(k);
  CHECK_PTR(v);
  CHECK_PTR(out);
  CHECK(idx != nullptr && ((uintptr_t)idx & 3u) == 0, SPARDA_ERR_INVALID_ARG, "idx is NULL or not 4-byte aligned");
  const size_t need = ws_bytes_for(SPARDA_OP_BLOCK_SPARSE_ATTN, B, Hq, Hkv, 1, T, k_sel);
  CHECK(ws_bytes >= need, SPARDA_ERR_WORKSPACE, "%s needs %zu workspace bytes, got %zu", name, need, ws_bytes);
  if (need) CHECK_PTR(ws);
  if (int e = check_q_pos(q_pos, 1)) return e;
  sparda::AttnDims ad = attn_dims(B, Hq, Hkv, 1, q_start, T, k_sel, scale, SPARDA_KV_CACHE);
  ad.q_pos = q_pos;
  return hip_status(sparda::launch_topk_attn_decode(blk_scores, q, k, v, idx, out, dtype == SPARDA_BF16, ad, ws,
                                                    merge, (hipStream_t)stream),
                    name);
}

// The partial results a decode attention of these sizes left in ws, checked.
int pending_merge(const void* ws, size_t ws_bytes, int dtype, int B, int Hq, int Hkv, int T, int d, int k_sel,
                  sparda::AttnDims* ad) {
  if (int e = check_dtype(dtype)) return e;
  if (int e = check_geometry(B, Hq, Hkv, 1, T - 1, T, d)) return e;
  CHECK(k_sel >= 1 && k_sel <= T / sparda::kBlock, SPARDA_ERR_INVALID_ARG, "k = %d outside 1..nB (%d)", k_sel,
        T / sparda::kBlock);
  const size_t need = ws_bytes_for(SPARDA_OP_BLOCK_SPARSE_ATTN, B, Hq, Hkv, 1, T, k_sel);
  CHECK(ws_bytes >= need, SPARDA_ERR_WORKSPACE, "the merged attention's workspace needs %zu bytes, got %zu", need,
        ws_bytes);
  *ad = attn_dims(B, Hq, Hkv, 1, T - 1, T, k_sel, 1.f, SPARDA_KV_CACHE);
  return SPARDA_OK;
}
}  // namespace

SPARDA_EXPORT int sparda_topk_block_sparse_attn(const float* blk_scores, const void* q, const void* k, const void* v,
                                                int32_t* idx, void* out, int dtype, int B, int Hq, int Hkv,
                                                int q_start, const int* q_pos, int T, int d, int block, int k_sel,
                                                float scale, void* ws, size_t ws_bytes, void* stream) {
  return topk_attn_impl(blk_scores, q, k, v, idx, out, dtype, B, Hq, Hkv, q_start, q_pos, T, d, block, k_sel, scale,
                        ws, ws_bytes, true, stream, "topk_block_sparse_attn");
}

SPARDA_EXPORT int sparda_topk_block_sparse_attn_noalloc(const float* blk_scores, const void* q, const void* k,
                                                        const void* v, int32_t* idx, void* out, int dtype, int B,
                                                        int Hq, int Hkv, int q_start, const int* q_pos, int T, int d,
                                                        int block, int k_sel, float scale, void* stream) {
  // validated against the static array's size first, so nothing is looked up
  // or launched for a request that does not fit
  if (int e = check_dtype(dtype)) return e;
  if (int e = check_geometry(B, Hq, Hkv, 1, q_start, T, d)) return e;
  const int nB = T / sparda::kBlock;
  CHECK(k_sel >= 1 && k_sel <= nB, SPARDA_ERR_INVALID_ARG, "k = %d outside 1..nB (%d)", k_sel, nB);
  const size_t need = ws_bytes_for(SPARDA_OP_BLOCK_SPARSE_ATTN, B, Hq, Hkv, 1, T, k_sel);
  CHECK(need <= sparda::kStaticScratchBytes, SPARDA_ERR_UNSUPPORTED,
        "topk_block_sparse_attn_noalloc: these sizes need %zu bytes of scratch, the static array holds %zu; use "
        "sparda_topk_block_sparse_attn with a workspace",
        need, sparda::kStaticScratchBytes);
  if (B == 0) return ok();
  void* ws = nullptr;
  if (need) {
    const hipError_t e = sparda::static_scratch(&ws);
    if (e != hipSuccess) return hip_status(e, "topk_block_sparse_attn_noalloc: static scratch address");
  }
  return topk_attn_impl(blk_scores, q, k, v, idx, out, dtype, B, Hq, Hkv, q_start, q_pos, T, d, block, k_sel, scale,
                        ws, need, true, stream, "topk_block_sparse_attn_noalloc");
}

SPARDA_EXPORT int sparda_topk_block_sparse_attn_partial(const float* blk_scores, const void* q, const void* k,
                                                        const void* v, int32_t* idx, void* out, int dtype, int B,
                                                        int Hq, int Hkv, int q_start, const int* q_pos, int T, int d,
                                                        int block, int k_sel, float scale, void* ws, size_t ws_bytes,
                                                        void* stream) {
  return topk_attn_impl(blk_scores, q, k, v, idx, out, dtype, B, Hq, Hkv, q_start, q_pos, T, d, block, k_sel, scale,
                        ws, ws_bytes, false, stream, "topk_block_sparse_attn_partial");
}

SPARDA_EXPORT int sparda_merge_partials(void* ws, size_t ws_bytes, void* out, int dtype, int B, int Hq, int Hkv,
                                        int T, int d, int k_sel, void* stream) {
  sparda::AttnDims ad;
  if (int e = pending_merge(ws, ws_bytes, dtype, B, Hq, Hkv, T, d, k_sel, &ad)) return e;
  if (B == 0) return ok();
  CHECK_PTR(out);
  if (ws_bytes) CHECK_PTR(ws);
  return hip_status(sparda::launch_merge_partials(ws, out, dtype == SPARDA_BF16, ad, (hipStream_t)stream),
                    "merge_partials launch");
}

SPARDA_EXPORT int sparda_select_forecast_merge(const void* f, const void* k_cmp, float* blk_scores, int dtype, int B,
                                               int Hkv, int q_start, const int* q_pos, int T, int d, int kernel,
                                               int stride, int block, float scale, void* m_ws, size_t m_ws_bytes,
                                               void* m_out, int m_Hq, int m_T, int m_k_sel, void* stream) {
  if (int e = check_dtype(dtype)) return e;
  if (int e = check_geometry(B, Hkv, Hkv, 1, q_start, T, d)) return e;
  if (int e = check_select_params(kernel, stride, block, sparda::kTile, scale)) return e;
  sparda::AttnDims ad;
  if (int e = pending_merge(m_ws, m_ws_bytes, dtype, B, m_Hq, Hkv, m_T, d, m_k_sel, &ad)) return e;
  if (B == 0) return ok();
  CHECK_PTR(f);
  CHECK_PTR(k_cmp);
  CHECK_PTR(blk_scores);
  CHECK_PTR(m_out);
  if (m_ws_bytes) CHECK_PTR(m_ws);
  if (int e = check_q_pos(q_pos, 1)) return e;
  sparda::SelectDims sd = select_dims(B, Hkv, Hkv, 1, q_start, T, scale);
  sd.q_pos = q_pos;
  const sparda::DecodePartials p = sparda::decode_attn_partials(m_ws, ad);
  return hip_status(sparda::launch_select_forecast_decode(f, k_cmp, blk_scores, dtype == SPARDA_BF16, sd,
                                                          (hipStream_t)stream, &p, m_out),
                    "select_forecast_merge launch");
}

namespace {
// Byte ranges [a, a + na) and [b, b + nb) share a byte.
bool overlaps(const void* a, size_t na, const void* b, size_t nb) {
  const uintptr_t x = (uintptr_t)a, y = (uintptr_t)b;
  return na && nb && x < y + nb && y < x + na;
}
}  // namespace

SPARDA_EXPORT int sparda_decode_layer(const float* blk_scores, const void* q, const void* k, const void* v,
                                      int32_t* idx, void* out, int Hq, int q_start, const int* q_pos, int T, int k_sel,
                                      float scale, void* ws, size_t ws_bytes, const void* f_next,
                                      const void* k_cmp_next, float* blk_scores_next, int q_start_next,
                                      const int* q_pos_next, int T_next, float scale_next, int dtype, int B, int Hkv,
                                      int d, int block, int kernel, int stride, void* stream) {
  if (int e = check_dtype(dtype)) return e;
  CHECK(dtype == SPARDA_BF16, SPARDA_ERR_UNSUPPORTED, "decode_layer: only bf16 inputs are supported");
  // this layer's top-k + attention
  if (int e = check_geometry(B, Hq, Hkv, 1, q_start, T, d)) return e;
  CHECK(block == sparda::kBlock, SPARDA_ERR_UNSUPPORTED, "block %d != 64", block);
  CHECK(std::isfinite(scale), SPARDA_ERR_INVALID_ARG, "scale is not finite");
  const int nB = T / sparda::kBlock;
  CHECK(nB <= 8192, SPARDA_ERR_UNSUPPORTED, "decode_layer: nB = %d above 8192", nB);
  CHECK(k_sel >= 1 && k_sel <= nB, SPARDA_ERR_INVALID_ARG, "k = %d outside 1..nB (%d)", k_sel, nB);
  CHECK(k_sel <= 1024, SPARDA_ERR_UNSUPPORTED, "decode_layer: k = %d above 1024", k_sel);
  const size_t need = ws_bytes_for(SPARDA_OP_DECODE_LAYER, B, Hq, Hkv, 1, T, k_sel);
  CHECK(ws_bytes >= need, SPARDA_ERR_WORKSPACE, "decode_layer needs %zu workspace bytes, got %zu", need, ws_bytes);
  // the next layer's selection
  const bool next = f_next != nullptr;
  if (next) {
    if (int e = check_geometry(B, Hkv, Hkv, 1, q_start_next, T_next, d)) return e;
    if (int e = check_select_params(kernel, stride, block, sparda::kTile, scale_next)) return e;
  }
  if (B == 0) return ok();
  CHECK(blk_scores != nullptr && ((uintptr_t)blk_scores & 3u) == 0, SPARDA_ERR_INVALID_ARG,
        "blk_scores is NULL or not 4-byte aligned");
  CHECK_PTR(q);
  CHECK_PTR(k);
  CHECK_PTR(v);
  CHECK_PTR(out);
  CHECK(idx != nullptr && ((uintptr_t)idx & 3u) == 0, SPARDA_ERR_INVALID_ARG, "idx is NULL or not 4-byte aligned");
  if (need) CHECK_PTR(ws);
  if (int e = check_q_pos(q_pos, 1)) return e;
  const size_t rows = (size_t)B * Hkv;
  const size_t scores_b = rows * nB * 4, idx_b = rows * k_sel * 4, out_b = (size_t)B * Hq * d * 2;
  CHECK(!overlaps(out, out_b, blk_scores, scores_b) && !overlaps(out, out_b, idx, idx_b) &&
            !overlaps(idx, idx_b, blk_scores, scores_b),
        SPARDA_ERR_INVALID_ARG, "decode_layer: out, idx and blk_scores must not overlap");
  if (next) {
    if (int e = check_q_pos(q_pos_next, 1)) return e;
    CHECK_PTR(k_cmp_next);
    CHECK_PTR(blk_scores_next);
    // the next layer's scores are written while this layer's are read, its
    // selection and top-k running in the same grid
    const size_t next_b = rows * (T_next / sparda::kBlock) * 4;
    CHECK(!overlaps(blk_scores_next, next_b, blk_scores, scores_b) && !overlaps(blk_scores_next, next_b, idx, idx_b) &&
              !overlaps(blk_scores_next, next_b, out, out_b) && !overlaps(blk_scores_next, next_b, ws, need),
          SPARDA_ERR_INVALID_ARG,
          "decode_layer: blk_scores_next must not overlap blk_scores, idx, out or the workspace (they are read or "
          "written in the same launch)");
  }
  sparda::LayerLaunch L{};
  L.attn = attn_dims(B, Hq, Hkv, 1, q_start, T, k_sel, scale, SPARDA_KV_CACHE);
  L.attn.q_pos = q_pos;
  L.scores = blk_scores;
  L.q = q;
  L.k = k;
  L.v = v;
  L.idx = idx;
  L.out = out;
  L.ws = ws;
  if (next) {
    L.sel = select_dims(B, Hkv, Hkv, 1, q_start_next, T_next, scale_next);
    L.sel.q_pos = q_pos_next;
    L.f_next = f_next;
    L.kc_next = k_cmp_next;
    L.scores_next = blk_scores_next;
  }
  return hip_status(sparda::launch_decode_layer(L, true, (hipStream_t)stream), "decode_layer launch");
}

namespace {
// Pinned, mapped host memory: returns the device-side address or nullptr.
const void* mapped_host_ptr(const void* p) {
  hipPointerAttribute_t attr;
  const hipError_t e = hipPointerGetAttributes(&attr, p);
  if (e != hipSuccess) {
    (void)hipGetLastError();
    return nullptr;
  }
  if (attr.type != hipMemoryTypeHost) return nullptr;
  return attr.devicePointer;
}
}  // namespace

SPARDA_EXPORT int sparda_project_qkvf(const void* x, const void* w, void* q, void* k, void* v, void* f, int dtype,
                                      int B, int D, int Hq, int Hkv, int n_f, int d, void* stream) {
  if (int e = check_dtype(dtype)) return e;
  CHECK(dtype == SPARDA_BF16, SPARDA_ERR_UNSUPPORTED, "project_qkvf: only bf16 inputs are supported");
  CHECK(d == 128, SPARDA_ERR_UNSUPPORTED, "project_qkvf: head dim %d (only 128 supported)", d);
  CHECK(B >= 0 && Hkv >= 1 && Hq >= 1 && Hq % Hkv == 0, SPARDA_ERR_INVALID_ARG,
        "project_qkvf: need B >= 0, Hq and Hkv >= 1, Hq %% Hkv == 0 (B=%d Hq=%d Hkv=%d)", B, Hq, Hkv);
  CHECK(D > 0 && D % 512 == 0 && D <= (1 << 24), SPARDA_ERR_UNSUPPORTED,
        "project_qkvf: D=%d must be a positive multiple of 512 up to 2^24", D);
  CHECK(n_f >= 0 && n_f <= 8, SPARDA_ERR_INVALID_ARG, "project_qkvf: n_f=%d outside 0..8", n_f);
  const long rows = (long)(Hq + 2L * Hkv + (long)n_f * Hkv) * d;
  CHECK(rows / 16 <= 2147483647L && (long)B * D < (1L << 40) && rows * (long)D < (1L << 40), SPARDA_ERR_UNSUPPORTED,
        "project_qkvf: sizes too large");
  if (B == 0) return ok();
  CHECK_PTR(x);
  CHECK_PTR(w);
  CHECK_PTR(q);
  CHECK_PTR(k);
  CHECK_PTR(v);
  if (n_f > 0) CHECK_PTR(f);
  return hip_status(sparda::launch_project_qkvf(x, w, q, k, v, f, B, D, Hq, Hkv, n_f, (hipStream_t)stream),
                    "project_qkvf launch");
}

SPARDA_EXPORT int sparda_prefetch_blocks(const void* host_k, const void* host_v, const int32_t* idx,
                                         void* stage_k, void* stage_v, int dtype, int B, int Hkv, int nB,
                                         int block, int d, int k_sel, int num_workgroups, void* side_stream) {
  if (int e = check_dtype(dtype)) return e;
  CHECK(B >= 0 && Hkv >= 1, SPARDA_ERR_INVALID_ARG, "B %d / Hkv %d out of range", B, Hkv);
  CHECK(block == sparda::kBlock, SPARDA_ERR_UNSUPPORTED, "block %d != 64", block);
  CHECK(d == sparda::kHeadDim, SPARDA_ERR_UNSUPPORTED, "head dim %d != 128", d);
  CHECK(nB >= 1, SPARDA_ERR_INVALID_ARG, "nB = %d < 1", nB);
  CHECK(k_sel >= 1 && k_sel <= nB, SPARDA_ERR_INVALID_ARG, "k = %d outside 1..nB (%d)", k_sel, nB);
  CHECK(num_workgroups >= 0 && num_workgroups <= 4096, SPARDA_ERR_INVALID_ARG, "num_workgroups %d outside 0..4096",
        num_workgroups);
  if (B == 0) return ok();
  CHECK_PTR(host_k);
  CHECK_PTR(host_v);
  CHECK_PTR(stage_k);
  CHECK_PTR(stage_v);
  CHECK(idx != nullptr && ((uintptr_t)idx & 3u) == 0, SPARDA_ERR_INVALID_ARG, "idx is NULL or not 4-byte aligned");
  const void* dk = mapped_host_ptr(host_k);
  const void* dv = mapped_host_ptr(host_v);
  CHECK(dk != nullptr, SPARDA_ERR_INVALID_ARG, "host_k is not pinned host memory (use hipHostMalloc)");
  CHECK(dv != nullptr, SPARDA_ERR_INVALID_ARG, "host_v is not pinned host memory (use hipHostMalloc)");
  const int nwg = num_workgroups ? num_workgroups : kGatherWorkgroups;
  return hip_status(sparda::launch_prefetch(dk, dv, idx, stage_k, stage_v, dtype == SPARDA_BF16 ? 2 : 4, B, Hkv,
                                            nB, k_sel, nwg, (hipStream_t)side_stream),
                    "prefetch_blocks launch");
}

SPARDA_EXPORT int sparda_prefetch_blocks_cached(const void* host_k, const void* host_v, const int32_t* idx,
                                                int32_t* slot_tags, int32_t* slot_of, void* stage_k, void* stage_v,
                                                int dtype, int B, int Hkv, int nB, int block, int d, int k_sel,
                                                int n_slots, int num_workgroups, void* side_stream) {
  if (int e = check_dtype(dtype)) return e;
  CHECK(B >= 0 && Hkv >= 1, SPARDA_ERR_INVALID_ARG, "B %d / Hkv %d out of range", B, Hkv);
  CHECK(block == sparda::kBlock, SPARDA_ERR_UNSUPPORTED, "block %d != 64", block);
  CHECK(d == sparda::kHeadDim, SPARDA_ERR_UNSUPPORTED, "head dim %d != 128", d);
  CHECK(nB >= 1, SPARDA_ERR_INVALID_ARG, "nB = %d < 1", nB);
  CHECK(k_sel >= 1 && k_sel <= nB, SPARDA_ERR_INVALID_ARG, "k = %d outside 1..nB (%d)", k_sel, nB);
  CHECK(k_sel <= sparda::kCacheMaxK, SPARDA_ERR_UNSUPPORTED, "k = %d above %d for the cached gather", k_sel,
        sparda::kCacheMaxK);
  CHECK(n_slots >= k_sel && n_slots <= sparda::kCacheMaxSlots, SPARDA_ERR_INVALID_ARG,
        "n_slots = %d outside k (%d) .. %d", n_slots, k_sel, sparda::kCacheMaxSlots);
  CHECK(num_workgroups >= 0 && num_workgroups <= 4096, SPARDA_ERR_INVALID_ARG, "num_workgroups %d outside 0..4096",
        num_workgroups);
  if (B == 0) return ok();
  CHECK_PTR(host_k);
  CHECK_PTR(host_v);
  CHECK_PTR(stage_k);
  CHECK_PTR(stage_v);
  CHECK(idx != nullptr && ((uintptr_t)idx & 3u) == 0, SPARDA_ERR_INVALID_ARG, "idx is NULL or not 4-byte aligned");
  CHECK(slot_tags != nullptr && ((uintptr_t)slot_tags & 3u) == 0, SPARDA_ERR_INVALID_ARG,
        "slot_tags is NULL or not 4-byte aligned");
  CHECK(slot_of != nullptr && ((uintptr_t)slot_of & 3u) == 0, SPARDA_ERR_INVALID_ARG,
        "slot_of is NULL or not 4-byte aligned");
  const void* dk = mapped_host_ptr(host_k);
  const void* dv = mapped_host_ptr(host_v);
  CHECK(dk != nullptr, SPARDA_ERR_INVALID_ARG, "host_k is not pinned host memory (use hipHostMalloc)");
  CHECK(dv != nullptr, SPARDA_ERR_INVALID_ARG, "host_v is not pinned host memory (use hipHostMalloc)");
  const int nwg = num_workgroups ? num_workgroups : kGatherWorkgroups;
  return hip_status(sparda::launch_prefetch_cached(dk, dv, idx, slot_tags, slot_of, stage_k, stage_v,
                                                   dtype == SPARDA_BF16 ? 2 : 4, B, Hkv, nB, k_sel, n_slots, nwg,
                                                   (hipStream_t)side_stream),
                    "prefetch_blocks_cached launch");
}

// ---- token-level Forecast variant ----

SPARDA_EXPORT int sparda_select_tokens(const void* f, const void* k, float* tok_scores, int dtype, int B, int Hkv,
                                       int T, int q_start, const int* q_pos, int d, float scale, void* stream) {
  if (int e = check_dtype(dtype)) return e;
  CHECK(B >= 0 && Hkv >= 1, SPARDA_ERR_INVALID_ARG, "B %d / Hkv %d out of range", B, Hkv);
  CHECK(d == sparda::kHeadDim, SPARDA_ERR_UNSUPPORTED, "head dim %d != 128", d);
  CHECK(T >= 1 && T <= (1 << 26), SPARDA_ERR_UNSUPPORTED, "T = %d outside 1..2^26", T);
  CHECK(q_start >= -1 && q_start < T, SPARDA_ERR_INVALID_ARG, "q_start %d outside -1..T-1", q_start);
  CHECK(std::isfinite(scale), SPARDA_ERR_INVALID_ARG, "scale is not finite");
  CHECK((long)B * Hkv <= 65535, SPARDA_ERR_UNSUPPORTED, "B * Hkv = %ld rows > 65535", (long)B * Hkv);
  if (int e = check_q_pos(q_pos, 1)) return e;
  if (B == 0) return ok();
  CHECK_PTR(f);
  CHECK_PTR(k);
  CHECK(tok_scores != nullptr && ((uintptr_t)tok_scores & 3u) == 0, SPARDA_ERR_INVALID_ARG,
        "tok_scores is NULL or not 4-byte aligned");
  return hip_status(sparda::launch_token_scores(f, k, tok_scores, dtype == SPARDA_BF16, B * Hkv, T, q_start, q_pos,
                                                Hkv, scale, (hipStream_t)stream),
                    "select_tokens launch");
}

SPARDA_EXPORT int sparda_token_sparse_attn(const void* q, const void* k, const void* v, const int32_t* tok_idx,
                                           void* out, int dtype, int B, int Hq, int Hkv, int T, int q_start,
                                           const int* q_pos, int d, int k_tok, float scale, void* ws,
                                           size_t ws_bytes, void* stream) {
  if (int e = check_dtype(dtype)) return e;
  CHECK(B >= 0 && Hkv >= 1 && Hq >= Hkv, SPARDA_ERR_INVALID_ARG, "B %d / Hq %d / Hkv %d out of range", B, Hq, Hkv);
  CHECK(Hq % Hkv == 0, SPARDA_ERR_INVALID_ARG, "Hq = %d is not a multiple of Hkv = %d", Hq, Hkv);
  const int G = Hq / Hkv;
  CHECK(G == 1 || G == 2 || G == 4 || G == 8, SPARDA_ERR_UNSUPPORTED, "group size %d not in {1, 2, 4, 8}", G);
  CHECK(d == sparda::kHeadDim, SPARDA_ERR_UNSUPPORTED, "head dim %d != 128", d);
  CHECK(T >= 1 && T <= (1 << 26), SPARDA_ERR_UNSUPPORTED, "T = %d outside 1..2^26", T);
  CHECK(q_start >= -1 && q_start < T, SPARDA_ERR_INVALID_ARG, "q_start %d outside -1..T-1", q_start);
  CHECK(k_tok >= sparda::kBlock && k_tok % sparda::kBlock == 0 && k_tok <= (1 << 20), SPARDA_ERR_UNSUPPORTED,
        "k_tok = %d must be a multiple of 64 in 64..2^20", k_tok);
  CHECK(std::isfinite(scale), SPARDA_ERR_INVALID_ARG, "scale is not finite");
  CHECK((long)B * Hkv <= 65535, SPARDA_ERR_UNSUPPORTED, "B * Hkv = %ld rows > 65535", (long)B * Hkv);
  if (int e = check_q_pos(q_pos, 1)) return e;
  if (B == 0) return ok();
  CHECK_PTR(q);
  CHECK_PTR(k);
  CHECK_PTR(v);
  CHECK_PTR(out);
  CHECK(tok_idx != nullptr && ((uintptr_t)tok_idx & 3u) == 0, SPARDA_ERR_INVALID_ARG,
        "tok_idx is NULL or not 4-byte aligned");
  const bool bf16 = dtype == SPARDA_BF16;
  // the split attention over k_tok / 64 slots of 64 list entries, each key
  // read where it sits in the cache
  sparda::AttnDims td = attn_dims(B, Hq, Hkv, 1, q_start, T, k_tok / sparda::kBlock, scale, SPARDA_KV_CACHE);
  td.q_pos = q_pos;
  const size_t need = sparda::decode_attn_ws_bytes(td);
  CHECK(need == 0 || (ws != nullptr && ((uintptr_t)ws & 255u) == 0 && ws_bytes >= need), SPARDA_ERR_INVALID_ARG,
        "workspace: need %zu bytes, 256-byte aligned (got %zu)", need, ws_bytes);
  return hip_status(sparda::launch_attn_tokens(q, k, v, tok_idx, out, bf16, td, ws, (hipStream_t)stream),
                    "token attention launch");
}
