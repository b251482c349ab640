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
constexpr int kMhChunk = 256;     // windows per workgroup, multi-head pass 1
constexpr int kMhPoolBlocks = 64; // blocks per workgroup, multi-head pass 2


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
struct MhWs {
  float* logits;  // [rows, G, W]
  float2* stats;  // [rows, chunks, G] (max, sum of exp)
};

static inline size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

static MhWs mh_ws(void* ws, const SelectDims& d) {
  const int G = d.Hq / d.Hkv;
  const size_t rows = (size_t)d.B * d.Hkv;
  MhWs r;
  r.logits = (float*)ws;
  r.stats = (float2*)((char*)ws + align256(rows * G * d.W * sizeof(float)));
  return r;
}

size_t multihead_decode_ws_bytes(const SelectDims& d) {
  const int G = d.Hq / d.Hkv;
  const size_t rows = (size_t)d.B * d.Hkv;
  const size_t chunks = (d.W + kMhChunk - 1) / kMhChunk;
  return align256(rows * G * d.W * sizeof(float)) + align256(rows * chunks * G * sizeof(float2));
}

template <typename Tag, int G>
__global__ __launch_bounds__(256) void mhsel_logits_kernel(const uint8_t* __restrict__ q,
                                                           const uint8_t* __restrict__ kc, MhWs ws,
                                                           int W, int n_vis, const int* __restrict__ q_pos,
                                                           int hkv, int T, int chunks, float scale) {
  using R = RowGeom<Tag>;
  constexpr int ITER = kMhChunk / R::SLOTS;
  static_assert(kMhChunk == 4 * kWave, "one window per thread, four waves");
  __shared__ float s_log[G][kMhChunk];
  __shared__ float red_m[4][G], red_z[4][G];

  const long row = blockIdx.y;  // (b, kv head)
  if (q_pos != nullptr) n_vis = visible_windows(row_position(q_pos, row, hkv, 0, T), W);
  const int chunk = blockIdx.x;
  const int w0 = chunk * kMhChunk;
  const int lane = threadIdx.x % R::LPR;
  const int slot = threadIdx.x / R::LPR;

  // query heads in the reduce-scatter's slot order for this lane
  u32x4 qv[G];
#pragma unroll
  for (int s = 0; s < G; ++s) qv[s] = load16(q + (row * G + slot_head<G>(s, lane & 15)) * R::RB + lane * 16);
  const uint8_t* base = kc + row * (long)W * R::RB + lane * 16;

  u32x4 kv[ITER];
#pragma unroll
  for (int it = 0; it < ITER; ++it) {
    const int w = w0 + it * R::SLOTS + slot;
    kv[it] = (w < n_vis) ? load16_nt(base + (long)w * R::RB) : u32x4{0, 0, 0, 0};
  }
  // All G logits of a window in one reduce-scatter: afterwards lanes 4 apart
  // (8 for G = 2, 16 for G = 1) hold different heads; the first lane of each
  // such group writes its head(s).
  constexpr int GR = G < 4 ? 1 : G / 4;
  constexpr int HL = G >= 4 ? 4 : (G == 2 ? 8 : 16);
#pragma unroll
  for (int it = 0; it < ITER; ++it) {
    const int lw = it * R::SLOTS + slot;
    const bool ok = w0 + lw < n_vis;
    float part[G];
#pragma unroll
    for (int s = 0; s < G; ++s) part[s] = dot16<Tag>(qv[s], kv[it], 0.f);
    if constexpr (R::LPR == 32) {  // fp32: 32 lanes per row; fold the upper 16 first
#pragma unroll
      for (int s = 0; s < G; ++s) part[s] = sum16(part[s]);
    }
    float sc[GR];
    reduce_scatter16<G>(part, sc);
    if ((lane & (HL - 1)) == 0 && lane < 16) {
      const int h = lane / HL;
#pragma unroll
      for (int gr = 0; gr < GR; ++gr) s_log[4 * gr + h][lw] = ok ? sc[gr] * scale : -INFINITY;
    }
  }
  __syncthreads();
  // Chunk statistics of all G heads at once: wave max and sum per head, one
  // LDS exchange of the four waves' partials each (the waves' partial sums
  // are added in wave order).
  const int t = threadIdx.x;
  const int wid = t / kWave;
  const int w = w0 + t;
  float x[G], m[G];
#pragma unroll
  for (int g = 0; g < G; ++g) {
    x[g] = s_log[g][t];
    m[g] = wave_max(x[g]);
    if (w < W) ws.logits[(row * G + g) * W + w] = x[g];
  }
  if (t % kWave == 0) {
#pragma unroll
    for (int g = 0; g < G; ++g) red_m[wid][g] = m[g];
  }
  __syncthreads();
#pragma unroll
  for (int g = 0; g < G; ++g) {
    m[g] = fmaxf(fmaxf(red_m[0][g], red_m[1][g]), fmaxf(red_m[2][g], red_m[3][g]));
    const float e = (m[g] == -INFINITY || x[g] == -INFINITY) ? 0.f : fast_exp(x[g] - m[g]);
    const float z = wave_sum(e);
    if (t % kWave == 0) red_z[wid][g] = z;
  }
  __syncthreads();
  if (t < G) {
    const float mt = fmaxf(fmaxf(red_m[0][t], red_m[1][t]), fmaxf(red_m[2][t], red_m[3][t]));
    const float z = ((red_z[0][t] + red_z[1][t]) + red_z[2][t]) + red_z[3][t];
    ws.stats[(row * chunks + chunk) * G + t] = make_float2(mt, z);
  }
}

template <typename Tag, int G>
__global__ __launch_bounds__(256) void mhsel_pool_kernel(MhWs ws, float* __restrict__ scores,
                                                         int W, int nB, int n_vis,
                                                         const int* __restrict__ q_pos, int hkv, int T,
                                                         int chunks) {
  constexpr int NWIN = 4 * kMhPoolBlocks + 1;
  __shared__ float s_sum[NWIN];
  __shared__ float s_m[G], s_iz[G];
  const long row = blockIdx.y;
  if (q_pos != nullptr) n_vis = visible_windows(row_position(q_pos, row, hkv, 0, T), W);
  const int beta0 = blockIdx.x * kMhPoolBlocks;
  const int nblk = min(kMhPoolBlocks, nB - beta0);
  const int nwin = 4 * nblk + 1;
  const int wstart = 4 * beta0 - 1;

  // Combine the per-chunk (max, sum of exp) of each head: one wave per head,
  // lanes read chunks in parallel.
  {
    const int lane = threadIdx.x % kWave;
    for (int g = threadIdx.x / kWave; g < G; g += (int)blockDim.x / kWave) {
      float m = -INFINITY;
      for (int c = lane; c < chunks; c += kWave) m = fmaxf(m, ws.stats[(row * chunks + c) * G + g].x);
      m = wave_max(m);
      float z = 0.f;
      for (int c = lane; c < chunks; c += kWave) {
        const float2 st = ws.stats[(row * chunks + c) * G + g];
        if (st.x != -INFINITY) z += st.y * fast_exp(st.x - m);
      }
      z = wave_sum(z);
      if (lane == 0) {
        s_m[g] = m;
        s_iz[g] = 1.f / z;
      }
    }
  }
  __syncthreads();
  for (int lw = threadIdx.x; lw < nwin; lw += blockDim.x) {
    const int w = wstart + lw;
    float S = -INFINITY;
    if (w >= 0 && w < n_vis) {
      S = 0.f;
#pragma unroll
      for (int g = 0; g < G; ++g)
        S += fast_exp(ws.logits[(row * G + g) * W + w] - s_m[g]) * s_iz[g];
    }
    s_sum[lw] = S;
  }
  __syncthreads();
  const int t = threadIdx.x;
  if (t < nblk) {
    float m = s_sum[4 * t];
#pragma unroll
    for (int j = 1; j < 5; ++j) m = fmaxf(m, s_sum[4 * t + j]);
    scores[row * nB + beta0 + t] = m;
  }
}

template <typename Tag, int G>
static void launch_mh(const void* q, const void* kc, float* scores, const SelectDims& d, MhWs w,
                      int n_vis, hipStream_t s) {
  const int chunks = (d.W + kMhChunk - 1) / kMhChunk;
  const int rows = d.B * d.Hkv;
  hipLaunchKernelGGL((mhsel_logits_kernel<Tag, G>), dim3(chunks, rows), dim3(256), 0, s,
                     (const uint8_t*)q, (const uint8_t*)kc, w, d.W, n_vis, d.q_pos, d.Hkv, d.T, chunks, d.scale);
  hipLaunchKernelGGL((mhsel_pool_kernel<Tag, G>),
                     dim3((d.nB + kMhPoolBlocks - 1) / kMhPoolBlocks, rows), dim3(256), 0, s, w,
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
