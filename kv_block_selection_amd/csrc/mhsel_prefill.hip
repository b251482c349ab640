// Step 2' for a chunk of queries (prefill): the multi-head selector, the
// comparison path that the Forecast replaces (bittide.aicompass.dev summary
// post, paragraph on the standard selector: every query head scores the
// compressed keys, softmax per head, then a sum over the GQA group;
// 10100.com commentary, section 痛点). Per query i of a 64-query tile and
// window w:  S_i[w] = sum_g softmax_w(scale * q_{g,i} . k~_w) over the windows
// visible to i; a block scores the max of S over its overlapping windows and
// the tile's queries.
//
// Every head's softmax normaliser must be known before the group sum, so the
// windows are swept twice, both times on the matrix cores
// (v_mfma_f32_32x32x16_bf16) with 128-window chunks of K~ staged in LDS:
//   pass 1  S^T = K~ Q^T. A lane owns one (query, head) column, so the running
//           max and sum of exp2 over the windows are lane-local.
//   pass 2  S = Q K~^T with rows ordered (query, head): for G <= 4 the G heads
//           of a query sit in one lane's accumulator registers, so the
//           normalised group sum is lane-local too (G = 8 adds one swap of the
//           lane halves); then the max over the tile's queries per window and
//           the block max-pool with a one-window carry between chunks.
// The same Q fragments in registers are the B operand of pass 1 and the A
// operand of pass 2. Pass 1 walks the chunks backwards so that pass 2 starts
// with chunks 0 and 1 already in LDS.
//
// A wave owns 64 rows = (64 / G queries) x G heads of one tile; a workgroup
// is G waves per tile, with 4 / G tiles per workgroup when G < 4.
#include <type_traits>

#include "prefill_lds.h"

namespace sparda {

namespace {

constexpr float kLog2e = 1.4426950408889634f;

template <int G>
struct MhLayout {
  static constexpr int kWavesPerTile = G;  // 64 queries x G heads / 64 rows per wave
  static constexpr int kTilesPerWg = G >= 4 ? 1 : 4 / G;
  static constexpr int kWaves = kWavesPerTile * kTilesPerWg;  // 4, or 8 for G = 8
  static constexpr int kThreads = kWaves * kWave;
  static constexpr int kQPerWave = 64 / G;
};

template <int G>
__global__ __launch_bounds__(MhLayout<G>::kThreads) void mhsel_prefill_kernel(
    const uint8_t* __restrict__ q, const uint8_t* __restrict__ kc, float* __restrict__ scores, int Tq, int q_start,
    int W, int nB, int n_tiles, float scale) {
  using L = MhLayout<G>;
  __shared__ __attribute__((aligned(16))) uint8_t s_kc[2][kChunkBytes];
  __shared__ float s_off[L::kWaves][64];                // per row: log2 of its softmax normaliser
  __shared__ float s_cm[L::kWaves][kChunkW];            // per wave: window max over its queries
  __shared__ float s_tc[L::kTilesPerWg][kChunkW + 1];  // per tile: window max; [0] = carry

  const long row = blockIdx.x;  // (b, h); query heads h*G .. h*G+G-1 of sequence b are rows row*G + g
  const int wave = threadIdx.x / kWave;
  const int lane = threadIdx.x % kWave;
  const int half = lane >> 5;
  const int l32 = lane & 31;
  const int tl = wave / L::kWavesPerTile;
  const int tile = blockIdx.y * L::kTilesPerWg + tl;
  const int qbase = min(tile, n_tiles - 1) * kTile + (wave % L::kWavesPerTile) * L::kQPerWave;
  const uint8_t* kc_row = kc + row * (long)W * kRowBytes;
  const float sl2 = scale * kLog2e;

  // Q fragments: row c = 32 n + l32 is head c % G, query qbase + c / G.
  u32x4 qa[2][8];
  int nv_col[2];
#pragma unroll
  for (int n = 0; n < 2; ++n) {
    const int c = 32 * n + l32;
    const int qi = qbase + c / G;
    const uint8_t* src = q + ((row * G + c % G) * (long)Tq + qi) * kRowBytes + half * 16;
#pragma unroll
    for (int s = 0; s < 8; ++s) qa[n][s] = load16(src + s * 32);
    nv_col[n] = visible_windows(q_start + qi, W);
  }
  // Windows visible to the workgroup's first query need no mask; none beyond
  // those visible to its last query is read at all.
  const int wg_q0 = blockIdx.y * L::kTilesPerWg * kTile;
  const int wg_q1 = min((blockIdx.y + 1) * L::kTilesPerWg, n_tiles) * kTile - 1;
  const int nv_lo = visible_windows(q_start + wg_q0, W);
  const int nv_hi = visible_windows(q_start + wg_q1, W);
  const int n_chunks = (nv_hi + kChunkW - 1) / kChunkW;

  if (threadIdx.x < L::kTilesPerWg) s_tc[threadIdx.x][0] = -INFINITY;
  int cur = 0;
  if (n_chunks > 0) {
    load_chunk_lds<L::kWaves>(kc_row, W, (n_chunks - 1) * kChunkW, s_kc[0]);
    __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
  }
  __syncthreads();

  // ---- pass 1: running max and sum of exp2 per (query, head), chunks backwards
  float m_run[2] = {-INFINITY, -INFINITY}, z_run[2] = {0.f, 0.f};
  for (int i = 0; i < n_chunks; ++i) {
    const int c = n_chunks - 1 - i;
    const bool more = i + 1 < n_chunks;
    if (more) load_chunk_lds<L::kWaves>(kc_row, W, (c - 1) * kChunkW, s_kc[cur ^ 1]);
    const uint8_t* ch = s_kc[cur];
    const int c0 = c * kChunkW;
    const bool masked = c0 + kChunkW > nv_lo;
    // two halves of 64 windows: half the accumulators, every fragment read once
#pragma unroll
    for (int mh = 0; mh < 2; ++mh) {
      f32x16 acc[2][2];
#pragma unroll
      for (int m = 0; m < 2; ++m)
#pragma unroll
        for (int n = 0; n < 2; ++n) acc[m][n] = f32x16{};
#pragma unroll
      for (int s = 0; s < 8; ++s)
#pragma unroll
        for (int m = 0; m < 2; ++m) {
          const bf16x8 a = as_bf16x8(chunk_frag(ch, 64 * mh + 32 * m + l32, s, half));
#pragma unroll
          for (int n = 0; n < 2; ++n)
            acc[m][n] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, as_bf16x8(qa[n][s]), acc[m][n], 0, 0, 0);
        }
      // Per column: the chunk half's max, then the sum of exp2 relative to
      // the new running max. Off the diagonal (every window visible to every
      // query) and with a positive scale the max is taken on the raw products
      // (the scaled max is the max of the scaled values) and the scale folds
      // into the exponent's fma; the masked form is a separate body so that
      // the common one carries no per-element selects.
      auto column = [&](auto kMask, int n) {
        float cmax = -INFINITY;
        if constexpr (decltype(kMask)::value) {
#pragma unroll
          for (int m = 0; m < 2; ++m)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
              const int w = c0 + 64 * mh + 32 * m + 8 * (r >> 2) + 4 * half + (r & 3);
              const float v = w < nv_col[n] ? acc[m][n][r] * sl2 : -INFINITY;
              acc[m][n][r] = v;
              cmax = fmaxf(cmax, v);
            }
        } else {
#pragma unroll
          for (int r = 0; r < 16; ++r) cmax = fmaxf(cmax, fmaxf(acc[0][n][r], acc[1][n][r]));
          cmax *= sl2;
        }
        const float mn = fmaxf(m_run[n], cmax);
        const float ms = mn == -INFINITY ? 0.f : mn;
        float z = z_run[n] * __builtin_amdgcn_exp2f(m_run[n] - ms);
#pragma unroll
        for (int m = 0; m < 2; ++m)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            if constexpr (decltype(kMask)::value) {
              z += __builtin_amdgcn_exp2f(acc[m][n][r] - ms);
            } else {
              z += __builtin_amdgcn_exp2f(fmaf(acc[m][n][r], sl2, -ms));
            }
          }
        z_run[n] = z;
        m_run[n] = mn;
      };
      if (masked || !(sl2 > 0.f)) {
        column(std::true_type{}, 0);
        column(std::true_type{}, 1);
      } else {
        column(std::false_type{}, 0);
        column(std::false_type{}, 1);
      }
    }
    if (more) {
      __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
      __syncthreads();  // the previous chunk is consumed and the next one has landed
      cur ^= 1;
    }
  }
  // The two lane halves hold different windows of the same column.
#pragma unroll
  for (int n = 0; n < 2; ++n) {
    const float mo = partner32(m_run[n]), zo = partner32(z_run[n]);
    const float mn = fmaxf(m_run[n], mo);
    const float ms = mn == -INFINITY ? 0.f : mn;
    const float z = z_run[n] * __builtin_amdgcn_exp2f(m_run[n] - ms) + zo * __builtin_amdgcn_exp2f(mo - ms);
    if (half == 0) s_off[wave][32 * n + l32] = mn == -INFINITY ? INFINITY : ms + __builtin_amdgcn_logf(z);
  }
  __syncthreads();
  float offr[2][16];  // normaliser of each accumulator row of pass 2
#pragma unroll
  for (int m = 0; m < 2; ++m)
#pragma unroll
    for (int r = 0; r < 16; ++r) offr[m][r] = s_off[wave][32 * m + 8 * (r >> 2) + 4 * half + (r & 3)];

  // ---- pass 2: normalised group sums, window max over the tile's queries, block pool
  for (int j = 0; j < n_chunks; ++j) {
    const bool more = j + 1 < n_chunks;
    // chunk 1 is still in LDS from the end of pass 1
    if (more && j > 0) load_chunk_lds<L::kWaves>(kc_row, W, (j + 1) * kChunkW, s_kc[cur ^ 1]);
    const uint8_t* ch = s_kc[cur];
    const int c0 = j * kChunkW;
    const bool masked = c0 + kChunkW > nv_lo;
#pragma unroll
    for (int nh = 0; nh < 2; ++nh) {
      f32x16 acc[2][2];
#pragma unroll
      for (int m = 0; m < 2; ++m)
#pragma unroll
        for (int n = 0; n < 2; ++n) acc[m][n] = f32x16{};
#pragma unroll
      for (int s = 0; s < 8; ++s)
#pragma unroll
        for (int n = 0; n < 2; ++n) {
          const bf16x8 bfr = as_bf16x8(chunk_frag(ch, 64 * nh + 32 * n + l32, s, half));
#pragma unroll
          for (int m = 0; m < 2; ++m)
            acc[m][n] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(qa[m][s]), bfr, acc[m][n], 0, 0, 0);
        }
      // Per column (window): the normalised group sum of each of the lane's
      // queries, max over them; the visibility mask only near the diagonal,
      // as a separate body.
      auto column = [&](auto kMask, int n) {
        const int wl = 64 * nh + 32 * n + l32;  // window within the chunk
        const int w = c0 + wl;
        float best = -INFINITY;
#pragma unroll
        for (int m = 0; m < 2; ++m) {
          // rows 32 m + 8 (r / 4) + 4 half + r % 4 = G * query + head
          constexpr int kRegsPerQ = G >= 4 ? 4 : G;  // registers holding one query's heads
#pragma unroll
          for (int r0 = 0; r0 < 16; r0 += kRegsPerQ) {
            float sum = __builtin_amdgcn_exp2f(fmaf(acc[m][n][r0], sl2, -offr[m][r0]));
#pragma unroll
            for (int u = 1; u < kRegsPerQ; ++u)
              sum += __builtin_amdgcn_exp2f(fmaf(acc[m][n][r0 + u], sl2, -offr[m][r0 + u]));
            if constexpr (G == 8) sum = sum32(sum);  // heads 4..7 sit in the other lane half
            if constexpr (decltype(kMask)::value) {
              const int rowc = 32 * m + 8 * (r0 >> 2) + 4 * half + (r0 & 3);
              sum = w < visible_windows(q_start + qbase + rowc / G, W) ? sum : -INFINITY;
            }
            best = fmaxf(best, sum);
          }
        }
        if constexpr (G != 8) best = max32(best);  // the other half holds other queries
        if (half == 0) s_cm[wave][wl] = best;
      };
      if (masked) {
        column(std::true_type{}, 0);
        column(std::true_type{}, 1);
      } else {
        column(std::false_type{}, 0);
        column(std::false_type{}, 1);
      }
    }
    __syncthreads();
    for (int e = threadIdx.x; e < L::kTilesPerWg * kChunkW; e += L::kThreads) {
      const int t = e / kChunkW, wi = e % kChunkW;
      float v = s_cm[t * L::kWavesPerTile][wi];
#pragma unroll
      for (int u = 1; u < L::kWavesPerTile; ++u) v = fmaxf(v, s_cm[t * L::kWavesPerTile + u][wi]);
      s_tc[t][1 + wi] = v;
    }
    __syncthreads();
    for (int e = threadIdx.x; e < L::kTilesPerWg * (kChunkW / 4); e += L::kThreads) {
      const int t = e / (kChunkW / 4), bt = e % (kChunkW / 4);
      const int blk = j * (kChunkW / 4) + bt;
      const int tile_e = blockIdx.y * L::kTilesPerWg + t;
      if (tile_e < n_tiles && blk < nB) {
        float v = s_tc[t][4 * bt];
#pragma unroll
        for (int u = 1; u < 5; ++u) v = fmaxf(v, s_tc[t][4 * bt + u]);
        scores[(row * n_tiles + tile_e) * (long)nB + blk] = v;
      }
    }
    if (more) __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));  // the next chunk has landed
    __syncthreads();
    if (threadIdx.x < L::kTilesPerWg) s_tc[threadIdx.x][0] = s_tc[threadIdx.x][kChunkW];
    if (more) cur ^= 1;
  }
  __syncthreads();
  // Blocks past the last chunk: the first may still see the carried window.
  for (int e = threadIdx.x; e < L::kTilesPerWg * nB; e += L::kThreads) {
    const int t = e / nB, blk = e % nB;
    const int tile_e = blockIdx.y * L::kTilesPerWg + t;
    if (tile_e < n_tiles && blk >= n_chunks * (kChunkW / 4))
      scores[(row * n_tiles + tile_e) * (long)nB + blk] =
          blk == n_chunks * (kChunkW / 4) ? s_tc[t][0] : -INFINITY;
  }
}

template <int G>
hipError_t launch_g(const void* q, const void* kc, float* scores, const SelectDims& d, hipStream_t s) {
  using L = MhLayout<G>;
  const dim3 grid(d.B * d.Hkv, (d.n_tiles + L::kTilesPerWg - 1) / L::kTilesPerWg);
  hipLaunchKernelGGL(mhsel_prefill_kernel<G>, grid, dim3(L::kThreads), 0, s, (const uint8_t*)q,
                     (const uint8_t*)kc, scores, d.Tq, d.q_start, d.W, d.nB, d.n_tiles, d.scale);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_select_multihead_prefill(const void* q, const void* kc, float* scores, const SelectDims& d,
                                           hipStream_t s) {
  switch (d.Hq / d.Hkv) {
    case 1: return launch_g<1>(q, kc, scores, d, s);
    case 2: return launch_g<2>(q, kc, scores, d, s);
    case 4: return launch_g<4>(q, kc, scores, d, s);
    case 8: return launch_g<8>(q, kc, scores, d, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace sparda
