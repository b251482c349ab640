// Step 2 at decode (one query per sequence): block scoring from compressed keys.
//
// Forecast selector (bittide.aicompass.dev summary post, paragraph on one
// Forecast head per GQA group; techwalker.com article, section 二): one vector
// per KV head scores every window, no softmax. Multi-head selector (same post,
// paragraph on the standard selector; 10100.com commentary, section 痛点): every
// query head of the group scores every window, softmax per head, group sum.
//
// Both are HBM-bound GEMVs over K_cmp [rows, W, 128]. A workgroup owns a run of
// whole blocks plus the one window before it (block b meets windows
// 4b-1 .. 4b+3), so it finishes its block scores with no exchange between
// workgroups. 16 lanes hold one 256-byte window row (8 bf16 each); a wave reads
// 4 rows (1 KiB contiguous) per load. The dot products use v_dot2_f32_bf16 and a
// DPP butterfly across the 16 lanes. The Forecast kernel can also merge a
// previous decode attention's split results (extra workgroups dispatched
// first), since the next layer's selection needs nothing from that output.
//
// The multi-head selector needs each head's softmax normaliser over all
// windows before it can sum heads, so it runs in two passes: (1) logits to the
// workspace plus per-chunk (max, sum of exp); (2) combine the chunk statistics,
// normalise, sum over the group, pool into blocks.
#include "common.h"
#include "launch.h"
#include "merge_row.h"
#include "reduce16.h"
#include "select_row.h"

namespace sparda {

#ifndef SPARDA_FSEL_BLOCKS
#define SPARDA_FSEL_BLOCKS 16
#endif
constexpr int kFselBlocks = SPARDA_FSEL_BLOCKS;  // blocks per workgroup, Forecast pass
#ifndef SPARDA_MH_CHUNK
#define SPARDA_MH_CHUNK 128
#endif
constexpr int kMhChunk = SPARDA_MH_CHUNK;  // windows per workgroup, multi-head pass 1
#ifndef SPARDA_MH_POOL
#define SPARDA_MH_POOL 256
#endif
constexpr int kMhPoolBlocks = SPARDA_MH_POOL;  // blocks per workgroup, multi-head pass 2


// ---------------------------------------------------------------- Forecast --
// MERGE: the grid has one more row of workgroups, dispatched first (y = 0),
// each merging one row of a previous decode attention's block-range results
// (merge_row_lean, the merge kernel's bits); the others score as usual.
template <typename Tag, bool MERGE>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(8))) void fsel_decode_kernel(const uint8_t* __restrict__ f,
                                                          const uint8_t* __restrict__ kc,
                                                          float* __restrict__ scores, int W, int nB,
                                                          int n_vis, const int* __restrict__ q_pos, int hkv,
                                                          int T, float scale, const float* __restrict__ m_part_o,
                                                          const float2* __restrict__ m_part_ml,
                                                          uint8_t* __restrict__ m_out, int m_G, int m_splits) {
  if constexpr (MERGE) {
    if (blockIdx.y == 0) {
      merge_row_lean<Tag>(blockIdx.x, threadIdx.x, m_part_o, m_part_ml, m_out, m_G, m_splits);
      return;
    }
  }
  const int chunk = blockIdx.y - (MERGE ? 1 : 0);
  __shared__ float s_win[fsel_lds_floats<Tag, kFselBlocks>()];
  // rows on the fast axis: a row's chunks share an XCD
  fsel_blocks<Tag, kFselBlocks>(f, kc, scores, W, nB, n_vis, q_pos, hkv, T, scale, blockIdx.x, chunk, s_win,
                                threadIdx.x);
}

hipError_t launch_select_forecast_decode(const void* f, const void* kc, float* scores, bool bf16,
                                         const SelectDims& d, hipStream_t s, const DecodePartials* merge,
                                         void* merge_out) {
  const int n_vis = min(d.W, (d.q_start - kKernel + 1) >= 0 ? (d.q_start - kKernel + 1) / kStride + 1 : 0);
  // a merge is only needed when the attention split its rows (it wrote the
  // output itself otherwise); its rows are this call's rows
  const bool m = merge != nullptr && merge->splits > 1;
  dim3 grid(d.B * d.Hkv, (d.nB + kFselBlocks - 1) / kFselBlocks + (m ? 1 : 0));
  const float* mo = m ? merge->part_o : nullptr;
  const float2* mml = m ? merge->part_ml : nullptr;
  const int mG = m ? merge->G : 0, ms = m ? merge->splits : 0;
#define SPARDA_FSEL(TAG, MM)                                                                                  \
  hipLaunchKernelGGL((fsel_decode_kernel<TAG, MM>), grid, dim3(256), 0, s, (const uint8_t*)f, (const uint8_t*)kc, \
                     scores, d.W, d.nB, n_vis, d.q_pos, d.Hkv, d.T, d.scale, mo, mml, (uint8_t*)merge_out, mG, ms)
  if (bf16) {
    if (m) SPARDA_FSEL(BF16Tag, true); else SPARDA_FSEL(BF16Tag, false);
  } else {
    if (m) SPARDA_FSEL(F32Tag, true); else SPARDA_FSEL(F32Tag, false);
  }
#undef SPARDA_FSEL
  return hipGetLastError();
}

// -------------------------------------------------------------- multi-head --
// Pass 1 leaves, per window, each head's exp(logit - chunk max) as fp16
// (between 0 and 1: at most 2^-11 relative rounding, well inside the scores'
// 1e-3 tolerance), and per (chunk, head) the max and the sum of those
// exponentials; pass 2 turns the chunk statistics into one normaliser per head
// and sums the group's probabilities e * exp(chunk max - max) / sum.
struct MhWs {
  uint16_t* e;    // [rows, chunks * kMhChunk, G] fp16: the G heads' exponentials of a window side by
                  // side; a row's records padded to whole chunks, so each chunk's are one aligned run
  float2* stats;  // [rows, chunks, G] (chunk max, sum of exp over the chunk)
};

static inline size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

static MhWs mh_ws(void* ws, const SelectDims& d) {
  const int G = d.Hq / d.Hkv;
  const size_t rows = (size_t)d.B * d.Hkv;
  MhWs r;
  r.e = (uint16_t*)ws;
  const size_t chunks = (d.W + kMhChunk - 1) / kMhChunk;
  r.stats = (float2*)((char*)ws + align256(rows * chunks * kMhChunk * G * sizeof(uint16_t)));
  return r;
}

size_t multihead_decode_ws_bytes(const SelectDims& d) {
  const int G = d.Hq / d.Hkv;
  const size_t rows = (size_t)d.B * d.Hkv;
  const size_t chunks = (d.W + kMhChunk - 1) / kMhChunk;
  return align256(rows * chunks * kMhChunk * G * sizeof(uint16_t)) + align256(rows * chunks * G * sizeof(float2));
}

__device__ __forceinline__ uint16_t to_f16_bits(float x) { return __builtin_bit_cast(uint16_t, (_Float16)x); }
__device__ __forceinline__ float from_f16_bits(uint16_t b) { return (float)__builtin_bit_cast(_Float16, b); }

// A record of G fp16 values, stored and loaded whole.
template <int G>
struct alignas(2 * G) MhRec {
  uint16_t v[G];
};

// Pass 1: a workgroup scores kMhChunk windows of one row for all G heads. After
// the reduce-scatter each lane holds the logits of GR heads (lanes that share a
// head hold the same bits) and keeps them in registers: the chunk's max per
// head (lane, then the wave's slots by lane-pair swaps, then the four waves),
// the exponentials and their sum (the same order). With four lanes per head
// each lane stores its exponentials straight to the records; the other
// layouts stage a chunk's records in LDS and store them whole.
template <typename Tag, int G>
__global__ __launch_bounds__(256) void mhsel_logits_kernel(const uint8_t* __restrict__ q,
                                                           const uint8_t* __restrict__ kc, MhWs ws,
                                                           int W, int n_vis, const int* __restrict__ q_pos,
                                                           int hkv, int T, int chunks, float scale) {
  using R = RowGeom<Tag>;
  constexpr int ITER = kMhChunk / R::SLOTS;
  constexpr int GR = G < 4 ? 1 : G / 4;              // heads a lane holds after the reduce-scatter
  constexpr int HL = G >= 4 ? 4 : (G == 2 ? 8 : 16);  // lanes that share a head
  static_assert(kMhChunk % R::SLOTS == 0, "whole passes of the 256 threads");
  constexpr bool kQuad = G >= 4 && ITER % 4 == 0;  // exponentials split over the four lanes of a head
  __shared__ float red_m[4][G], red_z[4][G];
  __shared__ MhRec<G> s_e[kQuad ? 1 : kMhChunk];  // record staging of the other layouts

  // rows on the fast axis: a row's chunks run on one XCD, so its records
  // meet in that XCD's L2 (and pass 2 of the row reads them there)
  const long row = blockIdx.x;  // (b, kv head)
  if (q_pos != nullptr) n_vis = visible_windows(row_position(q_pos, row, hkv, 0, T), W);
  const int chunk = blockIdx.y;
  const int w0 = chunk * kMhChunk;
  const int lane = threadIdx.x % R::LPR;
  const int slot = threadIdx.x / R::LPR;
  const int c = lane & 15;
  const int hsub = (c / HL) & 3;  // this lane's head within each group of four
  const int wid = threadIdx.x / kWave;
  // one lane per (slot, head) records exponentials; one per (wave, head) the
  // wave's statistics (after the swaps every slot of the wave holds them)
  const bool rec_writer = lane < 16 && (c & (HL - 1)) == 0;
  const bool writer = (threadIdx.x % kWave) < 16 && (c & (HL - 1)) == 0;

  // query heads in the reduce-scatter's slot order for this lane
  u32x4 qv[G];
#pragma unroll
  for (int s = 0; s < G; ++s) qv[s] = load16(q + (row * G + slot_head<G>(s, c)) * R::RB + lane * 16);
  const uint8_t* base = kc + row * (long)W * R::RB + lane * 16;
  MhRec<G>* rec_row = reinterpret_cast<MhRec<G>*>(ws.e) + row * (long)chunks * kMhChunk;

  u32x4 kv[ITER];
#pragma unroll
  for (int it = 0; it < ITER; ++it) {
    const int w = w0 + it * R::SLOTS + slot;
    kv[it] = (w < n_vis) ? load16_nt(base + (long)w * R::RB) : u32x4{0, 0, 0, 0};
  }
  float lg[ITER][GR];
  float m[GR];
#pragma unroll
  for (int gr = 0; gr < GR; ++gr) m[gr] = -INFINITY;
#pragma unroll
  for (int it = 0; it < ITER; ++it) {
    const int w = w0 + it * R::SLOTS + slot;
    float part[G];
#pragma unroll
    for (int s = 0; s < G; ++s) part[s] = dot16<Tag>(qv[s], kv[it], 0.f);
    if constexpr (R::LPR == 32) {  // fp32: 32 lanes per row; fold the upper 16 first
#pragma unroll
      for (int s = 0; s < G; ++s) part[s] = sum16(part[s]);
    }
    float sc[GR];
    reduce_scatter16<G>(part, sc);
#pragma unroll
    for (int gr = 0; gr < GR; ++gr) {
      lg[it][gr] = w < n_vis ? sc[gr] * scale : -INFINITY;
      m[gr] = fmaxf(m[gr], lg[it][gr]);
    }
  }
  // the chunk's max per head: across the wave's slots (bf16 rows are 16 lanes,
  // four slots per wave; fp32 rows 32 lanes, two slots, lanes 16..31 repeating
  // lanes 0..15), then across the waves
#pragma unroll
  for (int gr = 0; gr < GR; ++gr) {
    if constexpr (R::LPR == 16) m[gr] = max16(m[gr]);
    m[gr] = max32(m[gr]);
    if (writer) red_m[wid][4 * gr + hsub] = m[gr];
  }
  lds_sync();
  float z[GR];
#pragma unroll
  for (int gr = 0; gr < GR; ++gr) {
    const int h = 4 * gr + hsub;
    m[gr] = fmaxf(fmaxf(red_m[0][h], red_m[1][h]), fmaxf(red_m[2][h], red_m[3][h]));
    z[gr] = 0.f;
  }
  if constexpr (kQuad) {
    // the four lanes that share a head split its windows: lane j of the quad
    // takes iterations j, j + 4, ..., so each exponential is computed once;
    // the quad's sums then meet by a butterfly (the same bits in all four)
    const int j = c & 3;
#pragma unroll
    for (int k = 0; k < ITER / 4; ++k) {
      const int lw = (4 * k + j) * R::SLOTS + slot;
#pragma unroll
      for (int gr = 0; gr < GR; ++gr) {
        const float x = j == 0 ? lg[4 * k][gr] : j == 1 ? lg[4 * k + 1][gr] : j == 2 ? lg[4 * k + 2][gr]
                                                                                   : lg[4 * k + 3][gr];
        const float e = x == -INFINITY ? 0.f : fast_exp(x - m[gr]);
        z[gr] += e;
        // straight to the row's records, 2 bytes a lane (an LDS staging for
        // whole-record stores measured 0.6 us slower at 128K)
        if (lane < 16 && w0 + lw < W) rec_row[w0 + lw].v[4 * gr + hsub] = to_f16_bits(e);
      }
    }
#pragma unroll
    for (int gr = 0; gr < GR; ++gr) {
      z[gr] += dpp<0xB1>(z[gr]);  // quad_perm [1,0,3,2]
      z[gr] += dpp<0x4E>(z[gr]);  // quad_perm [2,3,0,1]
    }
  } else {
#pragma unroll
    for (int it = 0; it < ITER; ++it) {
      const int lw = it * R::SLOTS + slot;
#pragma unroll
      for (int gr = 0; gr < GR; ++gr) {
        const float e = lg[it][gr] == -INFINITY ? 0.f : fast_exp(lg[it][gr] - m[gr]);
        z[gr] += e;
        if (rec_writer) s_e[lw].v[4 * gr + hsub] = to_f16_bits(e);
      }
    }
  }
#pragma unroll
  for (int gr = 0; gr < GR; ++gr) {
    if constexpr (R::LPR == 16) z[gr] = sum16(z[gr]);
    z[gr] = sum32(z[gr]);
    if (writer) red_z[wid][4 * gr + hsub] = z[gr];
  }
  lds_sync();
  const int t = threadIdx.x;
  if (t < G) {
    const float mc = fmaxf(fmaxf(red_m[0][t], red_m[1][t]), fmaxf(red_m[2][t], red_m[3][t]));
    const float zc = ((red_z[0][t] + red_z[1][t]) + red_z[2][t]) + red_z[3][t];
    ws.stats[(row * chunks + chunk) * G + t] = make_float2(mc, zc);
  }
  if constexpr (!kQuad) {
    const int nw = min(kMhChunk, W - w0);
    for (int i = t; i < nw; i += 256) rec_row[w0 + i] = s_e[i];
  }
}

// Pass 2: a workgroup combines the row's chunk statistics into each head's max
// M and sum Z (one wave per head), the weight exp(chunk max - M) / Z of each
// chunk its windows fall in, then for each window sums the G heads'
// probabilities e * weight and pools them into block scores.
template <typename Tag, int G>
__global__ __launch_bounds__(256) void mhsel_pool_kernel(MhWs ws, float* __restrict__ scores,
                                                         int W, int nB, int n_vis,
                                                         const int* __restrict__ q_pos, int hkv, int T,
                                                         int chunks) {
  constexpr int NWIN = 4 * kMhPoolBlocks + 1;
  constexpr int PER = (NWIN + 255) / 256;                    // windows per thread
  constexpr int NCH = (NWIN + kMhChunk - 2) / kMhChunk + 1;  // chunks a run of NWIN windows can meet
  static_assert(NCH <= kWave, "one lane per chunk weight");
  __shared__ float s_sum[NWIN];
  __shared__ float s_wt[NCH][G];
  const long row = blockIdx.x;  // rows on the fast axis, as in pass 1
  if (q_pos != nullptr) n_vis = visible_windows(row_position(q_pos, row, hkv, 0, T), W);
  const int beta0 = blockIdx.y * kMhPoolBlocks;
  const int nblk = min(kMhPoolBlocks, nB - beta0);
  const int nwin = 4 * nblk + 1;
  const int wstart = 4 * beta0 - 1;
  const int c0 = max(wstart, 0) / kMhChunk;
  const int t = threadIdx.x;

  // the records of this thread's windows go out first, beside the statistics
  const MhRec<G>* src = reinterpret_cast<const MhRec<G>*>(ws.e) + row * (long)chunks * kMhChunk;
  MhRec<G> rec[PER];
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    const int w = wstart + t + 256 * i;
    if (t + 256 * i < nwin && w >= 0 && w < n_vis) rec[i] = src[w];
  }
  // each head's max M and sum Z over the row's chunks (one wave per head),
  // then the weight exp(chunk max - M) / Z of the chunks these windows meet.
  // A lane's statistics (kHeld chunks, rows of up to 64 kHeld chunks) and the
  // chunk max its weight needs are all loaded at once, so the max, the sum and
  // the weights cost one memory round trip; longer rows read the rest twice.
  {
    constexpr int kHeld = 4;
    const int lane = t % kWave;
    const float2* st_row = ws.stats + row * chunks * G;
    for (int g = t / kWave; g < G; g += 256 / kWave) {
      const float mc = lane < NCH && c0 + lane < chunks ? st_row[(c0 + lane) * G + g].x : -INFINITY;
      float2 st[kHeld];
#pragma unroll
      for (int j = 0; j < kHeld; ++j) {
        const int cc = lane + kWave * j;
        st[j] = cc < chunks ? st_row[cc * G + g] : make_float2(-INFINITY, 0.f);
      }
      float mx = -INFINITY;
#pragma unroll
      for (int j = 0; j < kHeld; ++j) mx = fmaxf(mx, st[j].x);
      for (int cc = lane + kWave * kHeld; cc < chunks; cc += kWave) mx = fmaxf(mx, st_row[cc * G + g].x);
      mx = wave_max(mx);
      float z = 0.f;
#pragma unroll
      for (int j = 0; j < kHeld; ++j)
        if (st[j].x != -INFINITY) z += st[j].y * fast_exp(st[j].x - mx);
      for (int cc = lane + kWave * kHeld; cc < chunks; cc += kWave) {
        const float2 sc = st_row[cc * G + g];
        if (sc.x != -INFINITY) z += sc.y * fast_exp(sc.x - mx);
      }
      z = wave_sum(z);
      const float iz = 1.f / z;
      if (lane < NCH) s_wt[lane][g] = mc != -INFINITY ? fast_exp(mc - mx) * iz : 0.f;
    }
  }
  __syncthreads();
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    const int lw = t + 256 * i;
    const int w = wstart + lw;
    if (lw < nwin) {
      float S = -INFINITY;
      if (w >= 0 && w < n_vis) {
        const float* wt = s_wt[w / kMhChunk - c0];
        S = 0.f;
#pragma unroll
        for (int g = 0; g < G; ++g) S = fmaf(from_f16_bits(rec[i].v[g]), wt[g], S);
      }
      s_sum[lw] = S;
    }
  }
  __syncthreads();
  if (t < nblk) {
    float mx = s_sum[4 * t];
#pragma unroll
    for (int j = 1; j < 5; ++j) mx = fmaxf(mx, s_sum[4 * t + j]);
    scores[row * nB + beta0 + t] = mx;
  }
}

template <typename Tag, int G>
static void launch_mh(const void* q, const void* kc, float* scores, const SelectDims& d, MhWs w,
                      int n_vis, hipStream_t s) {
  const int chunks = (d.W + kMhChunk - 1) / kMhChunk;
  const int rows = d.B * d.Hkv;
  hipLaunchKernelGGL((mhsel_logits_kernel<Tag, G>), dim3(rows, chunks), dim3(256), 0, s,
                     (const uint8_t*)q, (const uint8_t*)kc, w, d.W, n_vis, d.q_pos, d.Hkv, d.T, chunks, d.scale);
  hipLaunchKernelGGL((mhsel_pool_kernel<Tag, G>),
                     dim3(rows, (d.nB + kMhPoolBlocks - 1) / kMhPoolBlocks), dim3(256), 0, s, w,
                     scores, d.W, d.nB, n_vis, d.q_pos, d.Hkv, d.T, chunks);
}

hipError_t launch_select_multihead_decode(const void* q, const void* kc, float* scores, bool bf16,
                                          const SelectDims& d, void* ws, hipStream_t s) {
  const int n_vis = min(d.W, (d.q_start - kKernel + 1) >= 0 ? (d.q_start - kKernel + 1) / kStride + 1 : 0);
  const MhWs w = mh_ws(ws, d);
  const int G = d.Hq / d.Hkv;
#define SPARDA_MH(TAG, GG) launch_mh<TAG, GG>(q, kc, scores, d, w, n_vis, s)
#define SPARDA_MH_G(TAG)                  \
  switch (G) {                            \
    case 1: SPARDA_MH(TAG, 1); break;     \
    case 2: SPARDA_MH(TAG, 2); break;     \
    case 4: SPARDA_MH(TAG, 4); break;     \
    case 8: SPARDA_MH(TAG, 8); break;     \
    default: return hipErrorInvalidValue; \
  }
  if (bf16) {
    SPARDA_MH_G(BF16Tag)
  } else {
    SPARDA_MH_G(F32Tag)
  }
#undef SPARDA_MH_G
#undef SPARDA_MH
  return hipGetLastError();
}

}  // namespace sparda
