// Internal launchers (host side) called by the C ABI layer in api.cpp, which
// has already validated every argument.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace sparda {

// Supported geometry: head dim, KV block, compression window and stride, query tile.
constexpr int kHeadDim = 128;
constexpr int kBlock = 64;
constexpr int kKernel = 32;
constexpr int kStride = 16;
constexpr int kTile = 64;

struct SelectDims {
  int B, Hq, Hkv, Tq, q_start, T, W, nB, n_tiles;
  float scale;
  const int* q_pos;  // decode only: per-sequence query positions [B], or NULL
};

struct AttnDims {
  int B, Hq, Hkv, Tq, q_start, T, nB, n_tiles, k;
  float scale;
  int kv_mode;
  const int* q_pos;  // decode only: per-sequence query positions [B], or NULL
  const int32_t* slot_of;  // kv_mode 2: staging slot of each selected block [B*Hkv, k]
  int n_slots;             // kv_mode 2: staging slots per row
  bool q_pos_per_row = false;  // q_pos holds one position per (sequence, KV head) row
};

// where a decode attention's block-range results sit in its workspace
struct DecodePartials {
  float* part_o;    // [rows, splits, G, 128]
  float2* part_ml;  // [rows, splits, G] (max, sum)
  int splits, G, rows;
};

// compress.hip: windows [w_begin, w_end) of rows holding T tokens and W windows
hipError_t launch_compress(const void* k, void* kc, bool bf16, int rows, int T, int W, int w_begin, int w_end,
                           hipStream_t s);

// append.hip: write n_new tokens per row at the sequence's length and
// compress the windows they complete (k_cmp may be NULL)
hipError_t launch_append_kv(const void* k_new, const void* v_new, void* k_cache, void* v_cache, void* k_cmp,
                            const int* seq_len, int* status, bool bf16, int B, int Hkv, int n_new, int T_cap,
                            int W_cap, hipStream_t s);

int append_grid_y(bool bf16, int n_new, bool with_windows);  // workgroups per row

// select_decode.hip
hipError_t launch_select_forecast_decode(const void* f, const void* kc, float* scores, bool bf16,
                                         const SelectDims& d, hipStream_t s,
                                         const DecodePartials* merge = nullptr, void* merge_out = nullptr);
size_t multihead_decode_ws_bytes(const SelectDims& d);
hipError_t launch_select_multihead_decode(const void* q, const void* kc, float* scores, bool bf16,
                                          const SelectDims& d, void* ws, hipStream_t s);

// select_prefill.hip (bf16, Tq % 64 == 0)
hipError_t launch_select_forecast_prefill(const void* f, const void* kc, float* scores, const SelectDims& d,
                                          hipStream_t s);

// mhsel_prefill.hip (bf16, Tq % 64 == 0)
hipError_t launch_select_multihead_prefill(const void* q, const void* kc, float* scores, const SelectDims& d,
                                           hipStream_t s);

// topk.hip
hipError_t launch_topk(const float* scores, int32_t* idx, int rows, int nB, int k, hipStream_t s);

// attn_decode.hip
int decode_attn_splits(const AttnDims& d);
size_t decode_attn_ws_bytes(const AttnDims& d);
// The decode attention over a list of d.k * 64 tokens per row [rows, d.k * 64]
// (-1 and entries after the row's position are skipped), read in place from
// the cache; ws as for launch_attn_decode.
hipError_t launch_attn_tokens(const void* q, const void* k, const void* v, const int32_t* tok_idx, void* out,
                              bool bf16, const AttnDims& d, void* ws, hipStream_t s);
hipError_t launch_attn_decode(const void* q, const void* k, const void* v, const int32_t* idx,
                              void* out, bool bf16, const AttnDims& d, void* ws, hipStream_t s);
// the same after the row's top-k of scores [rows, nB] (written to idx), in one
// launch; needs nB <= 8192 and k <= 1024. merge = false leaves the block
// ranges' results in ws (the output is complete once they are merged).
hipError_t launch_topk_attn_decode(const float* scores, const void* q, const void* k, const void* v, int32_t* idx,
                                   void* out, bool bf16, const AttnDims& d, void* ws, bool merge, hipStream_t s);
DecodePartials decode_attn_partials(void* ws, const AttnDims& d);
// A static device array (one per GPU) that can stand in for a decode
// attention's workspace: its device address on the current device.
constexpr size_t kStaticScratchBytes = size_t(16) << 20;
hipError_t static_scratch(void** ptr);
hipError_t launch_merge_partials(void* ws, void* out, bool bf16, const AttnDims& d, hipStream_t s);
// one decode layer: top-k + attention of this layer (finished output) and
// the selection of the next layer (f_next may be NULL) in one launch, plus a
// merge launch when the batch has too few rows for a workgroup per row (ws
// then holds the block ranges' results)
bool decode_layer_row_form(const AttnDims& d);
struct LayerLaunch {
  AttnDims attn;
  const float* scores;
  const void *q, *k, *v;
  int32_t* idx;
  void* out;
  void* ws;
  SelectDims sel;
  const void *f_next, *kc_next;
  float* scores_next;
};
hipError_t launch_decode_layer(const LayerLaunch& L, bool bf16, hipStream_t s);

// attn_prefill.hip (bf16, cache mode, Tq % 64 == 0)
hipError_t launch_attn_prefill(const void* q, const void* k, const void* v, const int32_t* idx, void* out,
                               const AttnDims& d, hipStream_t s);

// project.hip (bf16; D % 512 == 0): x [B, D] times the rows of W [N, D]
hipError_t launch_project_qkvf(const void* x, const void* w, void* q, void* k, void* v, void* f, int B, int D, int Hq,
                               int Hkv, int n_f, hipStream_t s);

// prefetch.hip (the cached variant: k <= kCacheMaxK, k <= n_slots <= kCacheMaxSlots)
constexpr int kCacheMaxK = 256;
constexpr int kCacheMaxSlots = 1024;
hipError_t launch_prefetch_cached(const void* host_k, const void* host_v, const int32_t* idx, int32_t* slot_tags,
                                  int32_t* slot_of, void* stage_k, void* stage_v, int elem_bytes, int B, int Hkv,
                                  int nB, int k, int n_slots, int num_workgroups, hipStream_t s);
hipError_t launch_prefetch(const void* host_k, const void* host_v, const int32_t* idx, void* stage_k,
                           void* stage_v, int elem_bytes, int B, int Hkv, int nB, int k,
                           int num_workgroups, hipStream_t s);

// token.hip: the token-level Forecast variant. Token scores of rows [rows, T]
// at the query position (per sequence: q_pos, else p); the top-k of rows
// longer than 8192 (any length). The attention over the kept tokens is
// launch_attn_tokens (attn_decode.hip).
hipError_t launch_token_scores(const void* f, const void* k, float* scores, bool bf16, int rows, int T, int p,
                               const int* q_pos, int hkv, float scale, hipStream_t s);
hipError_t launch_topk_long(const float* scores, int32_t* idx, int rows, int n, int k, hipStream_t s);

}  // namespace sparda
