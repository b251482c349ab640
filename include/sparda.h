/*
 * sparda.h - C ABI of libsparda.so: SparDA's decoupled KV-block selection and
 * block-sparse attention on one AMD Instinct MI355X (gfx950).
 *
 * Sources of the operations (cited by page and section):
 *  [P1] bittide.aicompass.dev - summary post on SparDA and the arXiv abstract of
 *       "SparDA: Sparse Decoupled Attention for Efficient Long-Context LLM
 *       Inference" (arXiv:2606.04511).
 *  [P2] techwalker.com - article on SparDA; sections 一 (problem), 二 (Forecast),
 *       三 (implementation), 四 (training), 五 (experiments).
 *  [P3] 10100.com - commentary on arXiv:2606.04511; sections 痛点, 解法.
 *
 * Conventions shared by every call
 *  - Pointers are device pointers unless named host_*. Tensors are dense,
 *    row-major, 16-byte aligned. Shapes are given in brackets, outermost first.
 *  - dtype: SPARDA_F32 or SPARDA_BF16 for q/k/v/f/k_cmp/out (block scores are
 *    always float32, indices int32). Arithmetic accumulates in float32.
 *  - Supported geometry (v1): d = 128, block = 64, kernel = 32, stride = 16,
 *    tile = 64, T % 64 == 0, T >= 64, Hq % Hkv == 0, Tq == 1 or Tq % 64 == 0,
 *    q_start + Tq <= T. W = (T - kernel)/stride + 1 windows, nB = T/block
 *    blocks, nTiles = ceil(Tq/tile) query tiles (1 for decode).
 *  - T is the extent of the KV cache rows (tokens stored per row); queries sit
 *    at positions q_start .. q_start + Tq - 1. Everything is causal by
 *    position: windows, blocks and keys after a query's position take no part
 *    in its scores or its attention, so a cache may be allocated with room to
 *    grow and filled as decoding proceeds (the chunk need not end at T).
 *    Positions after the newest query may hold any finite values: their
 *    scores are masked, and their values enter only with weight 0.
 *  - Ragged decode batches: the decode calls (Tq = 1) of steps 2, 2' and 4
 *    take q_pos, NULL or a device int32 array [B] holding each sequence's own
 *    query position; q_start is then not used. Positions are read on the
 *    device and clamped to [-1, T - 1]; -1 (or less) means an empty sequence
 *    (no candidate block, output 0). With q_pos NULL every sequence sits at
 *    q_start. A chunk of queries (Tq > 1) needs q_pos NULL.
 *  - Every call is asynchronous on `stream` (a hipStream_t; NULL = the null
 *    stream). Arguments are validated on the host before anything is
 *    enqueued; on error nothing is launched. Device faults surface at the
 *    caller's next synchronisation.
 *  - Ownership: the caller owns every buffer, including the workspace `ws`
 *    (size from sparda_workspace_bytes); the library keeps no pointer after a
 *    call returns and allocates no device memory. Buffers must stay alive
 *    until the enqueued work completes. Calls on different streams that share
 *    a workspace race; ordering across streams is the caller's (events).
 *  - Return: SPARDA_OK (0) or an error status; sparda_last_error() then
 *    holds a message for the calling thread. No C++ exception crosses the ABI.
 */
#ifndef SPARDA_H
#define SPARDA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum sparda_status {
  SPARDA_OK = 0,
  SPARDA_ERR_INVALID_ARG = 1,  /* null/misaligned pointer, inconsistent sizes */
  SPARDA_ERR_UNSUPPORTED = 2,  /* valid request outside the supported set */
  SPARDA_ERR_WORKSPACE = 3,    /* ws_bytes smaller than sparda_workspace_bytes */
  SPARDA_ERR_HIP = 4           /* a HIP runtime call failed at enqueue time */
};

enum sparda_dtype { SPARDA_F32 = 0, SPARDA_BF16 = 1 };

enum sparda_kv_mode {
  SPARDA_KV_CACHE = 0,   /* k, v: the layer's cache [B, Hkv, T, d]; blocks read at idx */
  SPARDA_KV_STAGING = 1, /* k, v: staging [B, Hkv, k, block, d]; slot j holds block idx[.., j] */
  SPARDA_KV_SLOTS = 2    /* k, v: staging kept as a block cache [B, Hkv, n_slots, block, d];
                            block idx[.., j] sits in slot slot_of[.., j] */
};

enum sparda_op {
  SPARDA_OP_SELECT_FORECAST = 1,
  SPARDA_OP_SELECT_MULTIHEAD = 2,
  SPARDA_OP_BLOCK_SPARSE_ATTN = 3,
  SPARDA_OP_TOKEN_ATTN = 4, /* k_sel = k_tok: the block-range results of the attention over the kept tokens */
  SPARDA_OP_DECODE_LAYER = 5 /* sparda_decode_layer (Tq = 1): 0 when each row gets a workgroup */
};

/*
 * Step 1 - compressed keys. [P2] 四: at inference the keys are compressed
 * into windows of kernel 32 and stride 16; the pooling is the arithmetic mean.
 *   k      [B, Hkv, T, d]   keys of one layer
 *   k_cmp  [B, Hkv, W, d]   out: k_cmp[w] = mean of k[stride*w .. stride*w + kernel - 1]
 * Only complete windows are formed. float32 sums; bf16 output rounds to
 * nearest-even.
 */
int sparda_compress_keys(const void* k, void* k_cmp, int dtype, int B, int Hkv, int T, int d,
                         int kernel, int stride, void* stream);

/*
 * Step 1, incremental: the windows [w_begin, w_end) only, for a KV cache that
 * grows while decoding ([P2] 四 for the windows; the cache grows by one token
 * per step, so window w becomes complete once the sequence holds
 * stride*w + kernel tokens).
 *   k      [B, Hkv, T_cap, d]  cache rows of capacity T_cap tokens
 *   k_cmp  [B, Hkv, W_cap, d]  out; windows outside [w_begin, w_end) are left untouched
 * Window w needs tokens stride*w .. stride*w + kernel - 1, so
 * stride*(w_end - 1) + kernel <= T_cap is required. The arithmetic is that of
 * sparda_compress_keys: on the same tokens the two give the same bits.
 * Errors: SPARDA_ERR_INVALID_ARG for a range outside the capacities; the rest
 * as sparda_compress_keys. An empty range or batch is a valid no-op.
 */
int sparda_compress_windows(const void* k, void* k_cmp, int dtype, int B, int Hkv, int T_cap, int W_cap,
                            int d, int kernel, int stride, int w_begin, int w_end, void* stream);

/*
 * Decode-time state maintenance: append tokens to the caches and compress the
 * windows they complete, in one launch ([P2] 四 for the windows; the cache
 * grows by one token per decode step).
 *   k_new, v_new      [B, Hkv, n_new, d]   the new tokens' keys and values
 *   k_cache, v_cache  [B, Hkv, T_cap, d]   caches of capacity T_cap tokens
 *   k_cmp             [B, Hkv, W_cap, d]   compressed keys, or NULL (no windows)
 *   seq_len           device int32 [B]: tokens each sequence holds before the
 *                     call; its new tokens go to positions seq_len[b] ..
 *                     seq_len[b] + n_new - 1. The call does not change it.
 *   status            device int32, or NULL: 1 is OR-ed in when a sequence's
 *                     tokens do not fit (seq_len[b] < 0 or seq_len[b] + n_new >
 *                     T_cap); that sequence's rows are then left untouched.
 * Window w is written when position stride*w + kernel - 1 is among the new
 * ones (and w < W_cap), with the bits sparda_compress_keys would give for the
 * same keys; its earlier keys come from the cache. Rows of the caches outside
 * the new positions and the other windows are not touched.
 * Errors: as sparda_compress_windows for geometry; n_new outside 0..T_cap is
 * SPARDA_ERR_INVALID_ARG; B = 0 or n_new = 0 is a valid no-op.
 */
int sparda_append_kv(const void* k_new, const void* v_new, void* k_cache, void* v_cache, void* k_cmp,
                     const int* seq_len, int* status, int dtype, int B, int Hkv, int n_new, int T_cap,
                     int W_cap, int d, int kernel, int stride, void* stream);

/*
 * Step 2 - Forecast block scoring. [P1] paragraph on one Forecast head per GQA
 * group; [P2] 二; [P3] 解法: one Forecast vector per GQA group scores the
 * compressed keys directly - no per-query-head loop, no softmax.
 *   f           [B, Hkv, Tq, d]        Forecast vectors (query i at position q_start + i)
 *   k_cmp       [B, Hkv, W, d]
 *   blk_scores  [B, Hkv, nTiles, nB]   out (float32)
 * Window score s[i, w] = scale * f[i] . k_cmp[w]. Window w is visible to the
 * query at position p when stride*w + kernel - 1 <= p. Block score of a query
 * = max of s over the visible windows whose token span meets the block; a
 * tile's score = max over its queries; -inf marks a block with no visible
 * window (not a candidate). Decode is Tq = 1 at position q_start (or each
 * sequence's q_pos entry, see the conventions above). A chunk of
 * queries (Tq a multiple of 64) runs on the matrix cores and needs bf16.
 * ws: none needed (ws may be NULL, ws_bytes 0).
 */
int sparda_select_forecast(const void* f, const void* k_cmp, float* blk_scores, int dtype, int B,
                           int Hkv, int Tq, int q_start, const int* q_pos, int T, int d, int kernel,
                           int stride, int block, int tile, float scale, void* ws, size_t ws_bytes,
                           void* stream);

/*
 * Step 2' - the original multi-head selector (comparison path). [P1]
 * paragraph on the standard selector; [P3] 痛点: every query head of the GQA
 * group scores every candidate, softmax per head, then the sum over the group.
 *   q           [B, Hq, Tq, d]       query heads; head qh belongs to KV head qh / (Hq/Hkv)
 *   k_cmp       [B, Hkv, W, d]
 *   blk_scores  [B, Hkv, nTiles, nB] out (float32), pooled and tiled as for the Forecast
 * Per query and head, softmax over that query's visible windows of
 * scale * q . k_cmp[w]; S[w] = sum over the group's heads; block and tile
 * pooling by max as above.
 * ws: sparda_workspace_bytes(SPARDA_OP_SELECT_MULTIHEAD, ...) bytes (decode:
 * the logits and per-chunk softmax statistics; no initial contents needed).
 * A chunk of queries (Tq a multiple of 64) runs on the matrix cores, needs
 * bf16 and no workspace: it sweeps k_cmp twice (normalisers, then group sums).
 */
int sparda_select_multihead(const void* q, const void* k_cmp, float* blk_scores, int dtype, int B,
                            int Hq, int Hkv, int Tq, int q_start, const int* q_pos, int T, int d,
                            int kernel, int stride, int block, int tile, float scale, void* ws,
                            size_t ws_bytes, void* stream);

/*
 * Step 3 - top-k blocks. [P1] paragraph on block-sparse attention: score the
 * KV cache by block and keep the top-k blocks.
 *   blk_scores [rows, nB] float32 (rows = B*Hkv*nTiles), idx [rows, k] int32 out.
 * Candidates are the finite scores; ranked by score (higher first), ties to the
 * lower block index; the first min(k, #candidates) are written in ascending
 * block order, the rest of the row is -1. Scores must not be NaN.
 * Supported: 1 <= k <= nB <= 2^26. Rows longer than 8192 (token scores) go
 * through a top-k that streams the row from memory (one workgroup per row):
 * the same rule, the same result.
 */
int sparda_topk_blocks(const float* blk_scores, int32_t* idx, int rows, int nB, int k,
                       void* stream);

/*
 * Step 4 - GQA block-sparse attention. [P1] paragraphs on block-sparse
 * attention and on the next layer attending with its own queries over the
 * blocks chosen for it; [P3] 解法.
 *   q     [B, Hq, Tq, d]
 *   k, v  kv_mode SPARDA_KV_CACHE:   [B, Hkv, T, d]
 *         kv_mode SPARDA_KV_STAGING: [B, Hkv, k, block, d], slot j = block idx[b, h, 0, j] (Tq = 1 only)
 *         kv_mode SPARDA_KV_SLOTS:   [B, Hkv, n_slots, block, d], block idx[b, h, 0, j] in slot
 *                                    slot_of[b, h, j] (Tq = 1 only; as sparda_prefetch_blocks_cached
 *                                    leaves it); slot_of and n_slots are ignored in the other modes
 *   idx   [B, Hkv, nTiles, k] int32, -1 = unused slot
 *   out   [B, Hq, Tq, d] (dtype of q)
 * Query i (position p = q_start + i) of head qh attends, with softmax of
 * scale * q . k_j, over every key j <= p of the blocks listed for its KV head
 * and tile. Duplicate indices are not allowed. A query with no key gets 0.
 * A chunk of queries (Tq a multiple of 64) runs on the matrix cores and needs
 * bf16 in cache mode.
 * ws: sparda_workspace_bytes(SPARDA_OP_BLOCK_SPARSE_ATTN, ...) bytes (partial
 * results of the block ranges a row is split into; no initial contents needed).
 */
int sparda_block_sparse_attn(const void* q, const void* k, const void* v, int kv_mode,
                             const int32_t* idx, const int32_t* slot_of, int n_slots, void* out,
                             int dtype, int B, int Hq, int Hkv,
                             int Tq, int q_start, const int* q_pos, int T, int d, int block, int tile,
                             int k_sel, float scale, void* ws, size_t ws_bytes, void* stream);

/*
 * Steps 3 and 4 of a decode step in one launch: the top-k blocks of each
 * (sequence, KV head) row of blk_scores, exactly as sparda_topk_blocks picks
 * them, then the attention of sparda_block_sparse_attn (cache mode, one query
 * per sequence) over those blocks. [P1] paragraph on block-sparse attention:
 * keep the top-k scored blocks and attend over them.
 *   blk_scores [B, Hkv, 1, nB] float32, nB = T / block
 *   idx        [B, Hkv, 1, k]  out: the selection (ascending, -1 padded)
 *   q, k, v, out, q_pos, scale: as sparda_block_sparse_attn with Tq = 1
 * idx and out hold the same bits as sparda_topk_blocks followed by
 * sparda_block_sparse_attn. Needs nB <= 8192 and k <= 1024.
 * ws: sparda_workspace_bytes(SPARDA_OP_BLOCK_SPARSE_ATTN, B, Hq, Hkv, 1, T,
 * d, k) bytes, as for the attention call.
 */
int sparda_topk_block_sparse_attn(const float* blk_scores, const void* q, const void* k, const void* v,
                                  int32_t* idx, void* out, int dtype, int B, int Hq, int Hkv, int q_start,
                                  const int* q_pos, int T, int d, int block, int k_sel, float scale, void* ws,
                                  size_t ws_bytes, void* stream);

/*
 * sparda_topk_block_sparse_attn without a workspace argument, for callers
 * that cannot allocate device memory (code under HIP graph capture, serving
 * loops or harnesses that forbid hipMalloc). Same arguments minus ws and
 * ws_bytes, same selection and the same output bits. The block ranges'
 * results go to a static device array of the library (16 MiB, one copy per
 * GPU, held until the process ends); its address on the current device is
 * looked up on the first call there. The call itself allocates nothing.
 * The stream must belong to the current device. Every call on one GPU
 * shares that array and leaves its contents behind (nothing in it needs
 * initial contents): calls that may run at the same time on one GPU (other
 * streams, other threads) race and must be ordered by the caller.
 * Errors: as sparda_topk_block_sparse_attn, and SPARDA_ERR_UNSUPPORTED when
 * the sizes need more than the array's 16 MiB (sparda_workspace_bytes(
 * SPARDA_OP_BLOCK_SPARSE_ATTN, ...) > 16 << 20; of the sizes the call
 * accepts, only groups of 8 query heads with 2017 to 2047 (sequence, KV
 * head) rows and k >= 2 do): nothing is then looked up or launched.
 */
int sparda_topk_block_sparse_attn_noalloc(const float* blk_scores, const void* q, const void* k, const void* v,
                                          int32_t* idx, void* out, int dtype, int B, int Hq, int Hkv, int q_start,
                                          const int* q_pos, int T, int d, int block, int k_sel, float scale,
                                          void* stream);

/*
 * The decode step in the order of the method's layers. Layer L's Forecast
 * selects layer L+1's blocks ([P1] paragraph on the Forecast predicting the
 * next layer's blocks; [P2] 二), so layer L+1's selection needs nothing from
 * layer L's attention output. These three calls let that selection share a
 * launch with the last part of layer L's attention, the merge of its block
 * ranges:
 *
 * sparda_topk_block_sparse_attn_partial: as sparda_topk_block_sparse_attn,
 *   but leaves the block ranges' results in ws; `out` is complete only after
 *   sparda_merge_partials or sparda_select_forecast_merge has merged them.
 *   (When a row is not split into ranges, which needs few blocks and a large
 *   batch, the call writes `out` itself and the merge does nothing.)
 * sparda_merge_partials: that merge on its own. ws, out, dtype, B, Hq, Hkv,
 *   T, d, k_sel: those of the partial call, whose results ws holds.
 * sparda_select_forecast_merge: sparda_select_forecast for one query per
 *   sequence, plus the merge of a partial attention call with the same B,
 *   Hkv and dtype (m_ws, m_out, m_Hq, m_T, m_k_sel: that call's ws, out, Hq,
 *   T, k_sel), in one launch.
 * Every call gives the same bits as sparda_topk_block_sparse_attn and
 * sparda_select_forecast. ws must not be reused until the merge has run (same
 * stream, or ordered by events).
 */
int sparda_topk_block_sparse_attn_partial(const float* blk_scores, const void* q, const void* k, const void* v,
                                          int32_t* idx, void* out, int dtype, int B, int Hq, int Hkv, int q_start,
                                          const int* q_pos, int T, int d, int block, int k_sel, float scale,
                                          void* ws, size_t ws_bytes, void* stream);
int sparda_merge_partials(void* ws, size_t ws_bytes, void* out, int dtype, int B, int Hq, int Hkv, int T, int d,
                          int k_sel, void* stream);
int sparda_select_forecast_merge(const void* f, const void* k_cmp, float* blk_scores, int dtype, int B, int Hkv,
                                 int q_start, const int* q_pos, int T, int d, int kernel, int stride, int block,
                                 float scale, void* m_ws, size_t m_ws_bytes, void* m_out, int m_Hq, int m_T,
                                 int m_k_sel, void* stream);

/*
 * One decode layer: this layer's top-k + attention and the next layer's
 * Forecast selection, in one launch. Layer L's Forecast picks layer L+1's
 * blocks ([P1] paragraph on the Forecast predicting the next layer's blocks;
 * [P2] 二), and in a model both it and layer L's queries come from layer L's
 * hidden state, so the two parts need the same inputs and nothing from each
 * other; the next layer's queries need this layer's finished output (through
 * the output projection and the MLP, outside this library), so `out` is
 * complete when the call's work ends.
 *   blk_scores, q, k, v, idx, out, q_pos, scale, k_sel: as
 *     sparda_topk_block_sparse_attn (this layer; T, Hq, q_start its sizes)
 *   f_next [B, Hkv, 1, d], k_cmp_next [B, Hkv, W_next, d], blk_scores_next
 *     [B, Hkv, 1, nB_next] out, q_start_next, q_pos_next, T_next, scale_next:
 *     as sparda_select_forecast with Tq = 1 for the next layer (f_next NULL:
 *     no selection)
 *   ws: sparda_workspace_bytes(SPARDA_OP_DECODE_LAYER, B, Hq, Hkv, 1, T, d,
 *     k_sel) bytes, 0 when B * Hkv >= 96: each (sequence, KV head) row then
 *     gets one workgroup that merges its block ranges itself. With fewer
 *     rows the ranges' results go to ws and a second, small launch merges them.
 * idx holds the bits sparda_topk_blocks gives and blk_scores_next those of
 * sparda_select_forecast; out agrees with sparda_topk_block_sparse_attn to
 * float32 rounding (the block ranges a row is split into differ). bf16 only;
 * B, Hkv, d, block, kernel and stride are shared by both parts.
 * Errors as the separate calls, and SPARDA_ERR_INVALID_ARG when
 * blk_scores_next overlaps blk_scores, idx, out or ws, or out, idx and
 * blk_scores overlap one another (both parts run in one grid).
 */
int sparda_decode_layer(const float* blk_scores, const void* q, const void* k, const void* v, int32_t* idx,
                        void* out, int Hq, int q_start, const int* q_pos, int T, int k_sel, float scale, void* ws,
                        size_t ws_bytes, const void* f_next, const void* k_cmp_next, float* blk_scores_next,
                        int q_start_next, const int* q_pos_next, int T_next, float scale_next, int dtype, int B,
                        int Hkv, int d, int block, int kernel, int stride, void* stream);

/*
 * Step 5 - lookahead prefetch of the selected blocks from host memory.
 * [P1] paragraph on prefetching on a separate stream; [P2] 二 and 三: the blocks
 * the Forecast picks for the next layer are pulled from CPU memory into GPU
 * memory by a persistent kernel with a small, batch-dependent number of
 * workgroups, overlapped with the current layer; the indices never leave the GPU.
 *   host_k, host_v  [B, Hkv, nB*block, d] pinned host memory (hipHostMalloc),
 *                   read by the kernel over the host link
 *   idx             [B, Hkv, k] int32 device memory, -1 = leave the slot untouched
 *   stage_k/stage_v [B, Hkv, k, block, d] device memory, out: a bit copy
 *   num_workgroups  0 = library default (128), else 1..4096
 * Enqueued on side_stream; order it against producers and consumers of idx
 * and the staging buffers with events.
 */
int sparda_prefetch_blocks(const void* host_k, const void* host_v, const int32_t* idx,
                           void* stage_k, void* stage_v, int dtype, int B, int Hkv, int nB,
                           int block, int d, int k_sel, int num_workgroups, void* side_stream);

/*
 * Step 5 with the staging buffer kept as a cache of host blocks across calls
 * (the pages fetch every selected block each step; successive selections
 * often share blocks, and the host link is the step's bound).
 *   slot_tags  [B, Hkv, n_slots] int32 device memory, in/out: the block each
 *              staging slot holds, -1 = empty. Fill with -1 once before the
 *              first call; the calls keep it up to date.
 *   slot_of    [B, Hkv, k] int32 device memory, out: the slot holding block
 *              idx[.., j] after the call, -1 where idx is -1 or out of range
 *   stage_k/stage_v [B, Hkv, n_slots, block, d] device memory
 * A selected block already held keeps its slot and is not fetched again; each
 * other selected block takes a slot that no selected block holds (lowest
 * slot first) and is fetched. Needs k <= n_slots <= 1024 and k <= 256. The
 * host blocks are assumed unchanged since they were fetched. Same stream and
 * ordering rules as sparda_prefetch_blocks; the attention then reads the
 * blocks with kv_mode SPARDA_KV_SLOTS.
 */
int sparda_prefetch_blocks_cached(const void* host_k, const void* host_v, const int32_t* idx,
                                  int32_t* slot_tags, int32_t* slot_of, void* stage_k, void* stage_v,
                                  int dtype, int B, int Hkv, int nB, int block, int d, int k_sel,
                                  int n_slots, int num_workgroups, void* side_stream);

/*
 * The projections upstream of the path at decode: Q, K, V and the Forecast
 * vector from one hidden state per sequence, as one GEMM over the
 * concatenated weights. [P1] paragraph on the four projections every layer
 * emits (Q, K, V and a Forecast); [P1] abstract: the Forecast is a fourth
 * projection per layer beside Query, Key and Value.
 *   x  [B, D]                       hidden states (one token per sequence)
 *   w  [(Hq + 2*Hkv + n_f*Hkv)*d, D] weight rows: Hq query heads, Hkv key
 *                                   heads, Hkv value heads, then n_f sets of
 *                                   Hkv Forecast heads, d rows per head
 *   q  [B, Hq, 1, d]   k, v [B, Hkv, 1, d]   f [n_f, B, Hkv, 1, d]   (out)
 * out[b, n] = sum over c of x[b, c] * w[n, c], accumulated in fp32 and
 * rounded to nearest-even bf16. n_f = 1 for a layer whose Forecast looks one
 * layer ahead; the first layer, which also scores its own blocks, has n_f = 2
 * (set 0: its same-layer Forecast, set 1: the next layer's). n_f = 0 skips the
 * Forecast (f may be NULL). Supported: bf16, d = 128, D a positive multiple of
 * 512 up to 2^24, 0 <= n_f <= 8 (else SPARDA_ERR_UNSUPPORTED / _INVALID_ARG). All pointers are device memory, 16-byte aligned; the
 * outputs must not overlap the inputs. B = 0 is a no-op. Async on stream.
 */
int sparda_project_qkvf(const void* x, const void* w, void* q, void* k, void* v, void* f, int dtype, int B,
                        int D, int Hq, int Hkv, int n_f, int d, void* stream);

/*
 * Token-level Forecast (a variant). [P2] 六 names, as future work for models
 * with token-level sparse attention, a forecaster that predicts an importance
 * score per key token instead of per block; [P1] paragraph on DSA: a small
 * indexer picks the important tokens in place of the queries. The pages fix
 * neither the keys nor the number of tokens kept; here the Forecast vector
 * scores every visible key token directly and the top k_tok tokens are kept
 * by the top-k rule (sparda_topk_blocks on the token scores).
 *
 * sparda_select_tokens: decode token scores
 *   f [B, Hkv, 1, d], k [B, Hkv, T, d] (the layer's keys)
 *   tok_scores [B, Hkv, 1, T] float32 out: scale * f . k[t] for t <= p, -inf
 *   for t > p, where p is the sequence's q_pos entry (clamped to -1..T-1) or
 *   q_start when q_pos is NULL.
 * Supported: fp32/bf16, d = 128, 1 <= T <= 2^26, -1 <= q_start < T,
 * B * Hkv <= 65535. f and k 16-byte aligned; B = 0 is a no-op. Async on stream.
 */
int sparda_select_tokens(const void* f, const void* k, float* tok_scores, int dtype, int B, int Hkv, int T,
                         int q_start, const int* q_pos, int d, float scale, void* stream);

/*
 * sparda_token_sparse_attn: GQA attention at decode over the kept tokens only
 *   q [B, Hq, 1, d], k, v [B, Hkv, T, d], tok_idx [B, Hkv, 1, k_tok] int32
 *   (token positions, any order; entries < 0 or > p are padding; a position
 *   may appear at most once in a row, as sparda_topk_blocks leaves it: a
 *   repeated position would be attended once per copy), out [B, Hq, 1, d]
 *   written: softmax(scale q . k[j]) over the kept j, times v[j]; a query
 *   with no kept token gets zeros.
 * The kept rows are read where they sit in k and v, the list taken as k_tok / 64
 * ranges of 64 entries split over workgroups whose results ws holds until a
 * second launch merges them. ws: sparda_workspace_bytes(SPARDA_OP_TOKEN_ATTN,
 * B, Hq, Hkv, 1, T, d, k_tok) bytes (0: ws may be NULL), 256-byte aligned,
 * owned by the caller; it must not be shared by calls in flight at once.
 * Supported: fp32/bf16, d = 128, Hq / Hkv in {1, 2, 4, 8}, k_tok a multiple of
 * 64 in 64..2^20, 1 <= T <= 2^26, B * Hkv <= 65535. Async on stream.
 */
int sparda_token_sparse_attn(const void* q, const void* k, const void* v, const int32_t* tok_idx, void* out,
                             int dtype, int B, int Hq, int Hkv, int T, int q_start, const int* q_pos, int d,
                             int k_tok, float scale, void* ws, size_t ws_bytes, void* stream);

/* Workspace bytes the call `op` needs for these sizes (0 when none). */
size_t sparda_workspace_bytes(int op, int B, int Hq, int Hkv, int Tq, int T, int d, int k_sel);

/* Static text for a status code. */
const char* sparda_status_string(int status);

/* Message of the calling thread's last failed call ("" if none). */
const char* sparda_last_error(void);

/* Library version, major*10000 + minor*100 + patch. */
int sparda_version(void);

#ifdef __cplusplus
}
#endif

#endif /* SPARDA_H */
