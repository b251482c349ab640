// Token-level Forecast, the variant the pages name as future work
// (techwalker.com article, section 六: for models whose sparse attention is
// token-level, the forecaster would predict an importance score per key token
// instead of per block; bittide.aicompass.dev summary post, paragraph on DSA:
// a small indexer picks the important tokens in place of the queries). The
// pages define neither the keys such a forecaster reads nor how many tokens it
// keeps. Here the layer's Forecast vector scores every visible key token (no
// compression, no pooling), the same top-k rule as for blocks keeps the best
// k_tok tokens, and attention runs over exactly those tokens.
//
// token_scores_kernel: scores [rows, T] = scale * f . K[t] for t <= p and -inf
//   after p; an HBM-bound GEMV over every key row (16 lanes per 256-byte row,
//   all of a workgroup's loads in flight before the first is used; the
//   workgroup's scores leave through LDS as 16-byte pieces).
// topk_long_kernel: the top-k rule for rows too long for the LDS-resident
//   top-k (any length): one 1024-thread workgroup per row. A sample of 2048
//   scores spread evenly over the row gives a threshold t whose count in the
//   row is expected a little above k; one streaming pass keeps every score
//   at or above t, in index order, in LDS; when they are at least k (so t is
//   at or below the k-th largest score, and every kept score is among them)
//   and fit, the rule runs on them alone. Otherwise (heavy ties, a k near the
//   row length, few candidates) four 8-bit radix passes run over the order
//   keys streamed from memory. Either way the kept indices are written in ascending order
//   by a scan in index order (ties to the lower index), so the two paths give
//   the same result.
// The attention over the kept tokens reads their K and V rows where they sit
//   in the cache (the decode attention's token mode, attn_decode.hip).
#include "common.h"
#include "launch.h"
#include "select_row.h"
#include "topk_row.h"

namespace sparda {

constexpr int kTokIter = 32;       // key rows per thread group in flight
constexpr int kLongThreads = 1024;  // threads of a long-row top-k workgroup
constexpr int kLongEPT = 8;         // consecutive elements per thread in the output scan
constexpr int kLongSample = 2048;   // sampled scores for the threshold
constexpr int kLongCand = 8192;     // candidates the sampled path keeps in LDS (8 per thread)
constexpr int kLongSeg = 32;        // segments of kLongThreads scores per batch of the candidate pass

template <typename Tag>
__global__ __launch_bounds__(256) void token_scores_kernel(const uint8_t* __restrict__ f,
                                                           const uint8_t* __restrict__ kbuf,
                                                           float* __restrict__ scores, int T, int p_all,
                                                           const int* __restrict__ q_pos, int hkv, float scale) {
  using R = RowGeom<Tag>;
  const long row = blockIdx.y;
  const int p = row_position(q_pos, row, hkv, p_all, T);  // -1 .. T - 1
  const int lane = threadIdx.x % R::LPR;
  const int slot = threadIdx.x / R::LPR;
  const long t0 = (long)blockIdx.x * (kTokIter * R::SLOTS);
  const u32x4 fv = load16(f + row * R::RB + lane * 16);
  const uint8_t* base = kbuf + row * (long)T * R::RB + lane * 16;
  u32x4 kv[kTokIter];
#pragma unroll
  for (int it = 0; it < kTokIter; ++it) {
    const long t = t0 + it * R::SLOTS + slot;
    kv[it] = t <= p ? load16_nt(base + t * R::RB) : u32x4{0, 0, 0, 0};
  }
  // The workgroup's scores are gathered in LDS and leave as 16-byte pieces
  // through buffer stores with the sc1 cache-policy bit (device scope): at
  // 128K this takes the kernel from 0.70 to 0.66 ms against one 4-byte store
  // per key row (0.72 ms with plain 16-byte stores). A row whose scores do not
  // start 16-byte aligned takes plain 4-byte stores.
  constexpr int kRun = kTokIter * R::SLOTS;  // scores of one workgroup
  __shared__ float s_sc[kRun];
#pragma unroll
  for (int it = 0; it < kTokIter; ++it) {
    const long t = t0 + it * R::SLOTS + slot;
    const float s = group_sum<R::LPR>(dot16<Tag>(fv, kv[it], 0.f));
    if (lane == 0) s_sc[it * R::SLOTS + slot] = t <= p ? s * scale : -INFINITY;
  }
  __syncthreads();
  static_assert(kRun / 4 <= 256, "one 16-byte piece per thread");
  const int i = threadIdx.x;
  if (i < kRun / 4) {
    float* run = scores + row * (long)T + t0;
    const long t = t0 + 4 * i;
    const float4 v = *reinterpret_cast<const float4*>(&s_sc[4 * i]);
    if (((uintptr_t)run & 15) == 0 && t + 3 < T) {
      const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(run, (short)0, kRun * 4, 0x00020000);
      __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, v), rs, 16 * i, 0, 16);
    } else {
      const float e[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
      for (int j = 0; j < 4; ++j)
        if (t + j < T) run[4 * i + j] = e[j];
    }
  }
}

// Exclusive prefix over the workgroup of one int per thread, and the total;
// s_tot holds a slot per wave and is free again when this returns.
__device__ __forceinline__ int block_excl_scan(int v, int* s_tot, int& total) {
  const int lane = threadIdx.x % kWave;
  const int wid = threadIdx.x / kWave;
  const int incl = wave_incl_scan(v);
  if (lane == kWave - 1) s_tot[wid] = incl;
  __syncthreads();
  int before = incl - v;
  total = 0;
#pragma unroll
  for (int w = 0; w < kLongThreads / kWave; ++w) {
    const int x = s_tot[w];
    before += w < wid ? x : 0;
    total += x;
  }
  __syncthreads();
  return before;
}

// The want-th largest of the order keys keys[0 .. m) in LDS (0 = not a
// candidate; 1 <= want <= the number of nonzero keys), by 8-bit radix passes
// from the top: with all four passes tau is that key and take_eq the number
// of keys equal to it among the want largest; with fewer, tau is its top
// 8 PASSES bits (the rest zero), a key at or below it. Every thread of the
// workgroup calls it.
template <int PASSES>
__device__ void lds_radix_select(const uint32_t* keys, int m, int want, int* hist16, int* hist, int* s_digit,
                                 int* s_above, uint32_t& tau, int& take_eq) {
  const int t = threadIdx.x;
  const int lane = t % kWave;
  const int wid = t / kWave;
  uint32_t prefix = 0;
  int remaining = want;
  for (int pass = 0; pass < PASSES; ++pass) {
    const int shift = 24 - 8 * pass;
    const uint32_t hi_mask = pass == 0 ? 0u : (0xFFFFFFFFu << (shift + 8));
    for (int i = t; i < 256 * 16; i += kLongThreads) hist16[i] = 0;
    __syncthreads();
    for (int i = t; i < m; i += kLongThreads) {
      const uint32_t key = keys[i];
      if (key != 0u && (key & hi_mask) == prefix) atomicAdd(&hist16[((key >> shift) & 255u) * 16 + (lane & 15)], 1);
    }
    __syncthreads();
    if (t < 256) {
      int h = 0;
#pragma unroll
      for (int j = 0; j < 16; ++j) h += hist16[t * 16 + ((j + t) & 15)];
      hist[t] = h;
    }
    __syncthreads();
    if (wid == 0) {
      int h[4], sum = 0;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        h[i] = hist[255 - 4 * lane - i];
        sum += h[i];
      }
      int above = wave_incl_scan(sum) - sum;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        if (above < remaining && remaining <= above + h[i]) {
          *s_digit = 255 - 4 * lane - i;
          *s_above = above;
        }
        above += h[i];
      }
    }
    __syncthreads();
    prefix |= (uint32_t)*s_digit << shift;
    remaining -= *s_above;
  }
  tau = prefix;
  take_eq = remaining;
}

__global__ __launch_bounds__(kLongThreads) void topk_long_kernel(const float* __restrict__ scores,
                                                                 int32_t* __restrict__ idx, int n, int k) {
  // 16 copies of each digit's counter, lane l of a wave counting into copy
  // l % 16: the lanes of one atomic instruction that meet the same digit
  // (the top byte of similar scores is often shared) then spread over 16
  // addresses instead of queueing on one
  __shared__ int hist16[256 * 16];
  __shared__ int hist[256];
  __shared__ int s_tot[kLongThreads / kWave];
  __shared__ int s_digit, s_above, s_ncand;
  __shared__ uint32_t s_key[kLongCand];
  __shared__ int32_t s_pos[kLongCand];
  __shared__ int s_cnt[kLongSeg * (kLongThreads / kWave)];
  const int t = threadIdx.x;
  const int lane = t % kWave;
  const int wid = t / kWave;
  const float* src = scores + (long)blockIdx.x * n;
  int32_t* dst = idx + (long)blockIdx.x * k;

  // Sampled path, taken when the expected candidate count (1.2 k plus the
  // sample's slack of 16 positions) fits well inside the LDS store.
  const int r_sample = (int)(((long)6 * k * kLongSample + 5L * n - 1) / (5L * n)) + 16;
  if ((long)r_sample * n <= (long)kLongSample * (kLongCand * 4 / 5)) {
    // the threshold: the r-th largest of kLongSample scores spread evenly over
    // the row (one per 64 at 128K: every 64-key block of a token row is
    // represented, since neighbouring scores can be correlated, and only half
    // of the row's 128-byte lines are touched)
    int ns = 0;
    for (int j = t; j < kLongSample; j += kLongThreads) {
      const uint32_t key = order_key(src[((long)j * n) / kLongSample]);
      s_key[j] = key;
      ns += key != 0u;
    }
    int n_sampled;
    block_excl_scan(ns, s_tot, n_sampled);
    if (n_sampled > 0) {
      uint32_t t0;
      int unused;
      // the top 16 bits of the sample's r-th largest key are enough: a lower
      // threshold only admits a few more candidates
      lds_radix_select<2>(s_key, kLongSample, min(r_sample, n_sampled), hist16, hist, &s_digit, &s_above, t0,
                          unused);
      // One pass over the row: every key >= t0 into LDS in index order (t0 >
      // 0: the r-th key is not -inf, so its top 16 bits are not all zero). A
      // batch is kLongSeg segments of kLongThreads consecutive scores, one per
      // thread (coalesced loads, all in flight); a candidate's place is its
      // lane's rank in its wave (ballot) plus an exclusive prefix over the
      // batch's (segment, wave) counts.
      constexpr int kWaves = kLongThreads / kWave;
      int count = 0;
      for (long c0 = 0; c0 < n && count <= kLongCand; c0 += (long)kLongThreads * kLongSeg) {
        float x[kLongSeg];
#pragma unroll
        for (int j = 0; j < kLongSeg; ++j) {
          const long i = c0 + (long)j * kLongThreads + t;
          x[j] = i < n ? src[i] : -INFINITY;
        }
        int rank[kLongSeg];
#pragma unroll
        for (int j = 0; j < kLongSeg; ++j) {
          const uint64_t m = __ballot(order_key(x[j]) >= t0);
          rank[j] = __builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0));
          if (lane == 0) s_cnt[j * kWaves + wid] = __popcll(m);
        }
        __syncthreads();
        // exclusive prefix over the kLongSeg x kWaves counts, in index order
        // (one count per thread of the first kLongSeg * kWaves)
        const int v = t < kLongSeg * kWaves ? s_cnt[t] : 0;
        const int incl = wave_incl_scan(v);
        if (lane == kWave - 1 && wid < kLongSeg * kWaves / kWave) s_tot[wid] = incl;
        __syncthreads();
        int batch = 0, prior = 0;
#pragma unroll
        for (int w = 0; w < kLongSeg * kWaves / kWave; ++w) {
          batch += s_tot[w];
          prior += w < wid ? s_tot[w] : 0;
        }
        if (t < kLongSeg * kWaves) s_cnt[t] = incl - v + prior;
        __syncthreads();
#pragma unroll
        for (int j = 0; j < kLongSeg; ++j) {
          const uint32_t key = order_key(x[j]);
          const int pos = count + s_cnt[j * kWaves + wid] + rank[j];
          if (key >= t0 && pos < kLongCand) {
            s_key[pos] = key;
            s_pos[pos] = (int32_t)(c0 + (long)j * kLongThreads + t);
          }
        }
        count += batch;
        __syncthreads();  // s_cnt and s_tot are rewritten by the next batch
      }
      if (count >= k && count <= kLongCand) {  // the last batch's barrier published them
        uint32_t tau;
        int take_eq;
        lds_radix_select<4>(s_key, count, k, hist16, hist, &s_digit, &s_above, tau, take_eq);
        // kept: every candidate above tau and the first take_eq equal to it,
        // in index order (the candidates' order)
        const int c0 = t * (kLongCand / kLongThreads);
        uint32_t key[kLongCand / kLongThreads];
        int gt = 0, eq = 0;
#pragma unroll
        for (int j = 0; j < kLongCand / kLongThreads; ++j) {
          key[j] = c0 + j < count ? s_key[c0 + j] : 0u;
          gt += key[j] > tau;
          eq += key[j] == tau;  // tau > 0: a padding 0 never matches
        }
        int total;
        const int before = block_excl_scan(gt | (eq << 16), s_tot, total);
        int g_before = before & 0xFFFF, e_before = before >> 16;
#pragma unroll
        for (int j = 0; j < kLongCand / kLongThreads; ++j) {
          if (key[j] > tau) {
            const int pos = g_before + min(e_before, take_eq);
            if (pos < k) dst[pos] = s_pos[c0 + j];
            ++g_before;
          } else if (key[j] == tau) {
            if (e_before < take_eq && g_before + e_before < k) dst[g_before + e_before] = s_pos[c0 + j];
            ++e_before;
          }
        }
        return;
      }
    }
  }

  // Radix select of the k-th largest order key, 8 bits per pass from the top:
  // after the passes, `prefix` is that key and `remaining` the number of keys
  // equal to it still to take (the lowest indices first).
  uint32_t prefix = 0;
  int remaining = 0, n_cand = 0;
  bool take_all = false;
  for (int pass = 0; pass < 4; ++pass) {
    const int shift = 24 - 8 * pass;
    const uint32_t hi_mask = pass == 0 ? 0u : (0xFFFFFFFFu << (shift + 8));
    for (int i = t; i < 256 * 16; i += kLongThreads) hist16[i] = 0;
    __syncthreads();
    // kLongEPT independent loads per thread go out before their atomics (16
    // or 64 measured the same: the atomics, not the loads, set the pace)
    for (long c0 = 0; c0 < n; c0 += (long)kLongThreads * kLongEPT) {
      float x[kLongEPT];
#pragma unroll
      for (int j = 0; j < kLongEPT; ++j) {
        const long i = c0 + (long)j * kLongThreads + t;
        x[j] = i < n ? src[i] : -INFINITY;
      }
#pragma unroll
      for (int j = 0; j < kLongEPT; ++j) {
        const uint32_t key = order_key(x[j]);
        if (key != 0u && (key & hi_mask) == prefix) atomicAdd(&hist16[((key >> shift) & 255u) * 16 + (lane & 15)], 1);
      }
    }
    __syncthreads();
    if (t < 256) {
      int h = 0;
#pragma unroll
      for (int j = 0; j < 16; ++j) h += hist16[t * 16 + ((j + t) & 15)];  // rotated: distinct banks per lane
      hist[t] = h;
    }
    __syncthreads();
    if (wid == 0) {
      // lane handles digits 255 - 4 lane .. 252 - 4 lane, descending
      int h[4], sum = 0;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        h[i] = hist[255 - 4 * lane - i];
        sum += h[i];
      }
      const int incl = wave_incl_scan(sum);
      const int total = __builtin_amdgcn_readlane(incl, kWave - 1);
      const int want = pass == 0 ? min(k, total) : remaining;
      int above = incl - sum;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        if (above < want && want <= above + h[i]) {  // one lane, one digit (want >= 1)
          s_digit = 255 - 4 * lane - i;
          s_above = above;
        }
        above += h[i];
      }
      if (pass == 0 && lane == 0) s_ncand = total;
    }
    __syncthreads();
    if (pass == 0) {
      n_cand = s_ncand;
      remaining = min(k, n_cand);
      take_all = remaining == n_cand;  // includes a row with no candidate
      if (take_all) break;
    }
    prefix |= (uint32_t)s_digit << shift;
    remaining -= s_above;
  }

  // Kept: every key above `prefix` and the first `remaining` keys equal to it
  // (all candidates when take_all), written in index order.
  const uint32_t tau = prefix;
  const int take_eq = take_all ? 0 : remaining;
  const int kk = min(k, n_cand);
  int gt_base = 0, eq_base = 0;
  for (long c0 = 0; c0 < n; c0 += (long)kLongThreads * kLongEPT) {
    const long i0 = c0 + (long)t * kLongEPT;
    uint32_t key[kLongEPT];
    int gt = 0, eq = 0;
#pragma unroll
    for (int j = 0; j < kLongEPT; ++j) {
      key[j] = i0 + j < n ? order_key(src[i0 + j]) : 0u;
      gt += take_all ? key[j] != 0u : key[j] > tau;
      eq += !take_all && key[j] == tau;
    }
    const int packed = gt | (eq << 16);  // at most 8192 each
    const int incl = wave_incl_scan(packed);
    if (lane == kWave - 1) s_tot[wid] = incl;
    __syncthreads();
    int before = incl - packed, chunk = 0;
#pragma unroll
    for (int w = 0; w < kLongThreads / kWave; ++w) {
      const int v = s_tot[w];
      before += w < wid ? v : 0;
      chunk += v;
    }
    int g_before = gt_base + (before & 0xFFFF);
    int e_before = eq_base + (before >> 16);
#pragma unroll
    for (int j = 0; j < kLongEPT; ++j) {
      const bool is_gt = take_all ? key[j] != 0u : key[j] > tau;
      const bool is_eq = !take_all && key[j] == tau;
      if (is_gt) {
        const int pos = g_before + min(e_before, take_eq);
        if (pos < kk) dst[pos] = (int32_t)(i0 + j);
        ++g_before;
      } else if (is_eq) {
        if (e_before < take_eq && g_before + e_before < kk) dst[g_before + e_before] = (int32_t)(i0 + j);
        ++e_before;
      }
    }
    gt_base += chunk & 0xFFFF;
    eq_base += chunk >> 16;
    __syncthreads();  // s_tot is rewritten by the next chunk
  }
  for (int q = kk + t; q < k; q += kLongThreads) dst[q] = -1;
}

hipError_t launch_token_scores(const void* f, const void* k, float* scores, bool bf16, int rows, int T, int p,
                               const int* q_pos, int hkv, float scale, hipStream_t s) {
  if (bf16) {
    using R = RowGeom<BF16Tag>;
    const dim3 grid((unsigned)((T + kTokIter * R::SLOTS - 1) / (kTokIter * R::SLOTS)), rows);
    hipLaunchKernelGGL(token_scores_kernel<BF16Tag>, grid, dim3(256), 0, s, (const uint8_t*)f, (const uint8_t*)k,
                       scores, T, p, q_pos, hkv, scale);
  } else {
    using R = RowGeom<F32Tag>;
    const dim3 grid((unsigned)((T + kTokIter * R::SLOTS - 1) / (kTokIter * R::SLOTS)), rows);
    hipLaunchKernelGGL(token_scores_kernel<F32Tag>, grid, dim3(256), 0, s, (const uint8_t*)f, (const uint8_t*)k,
                       scores, T, p, q_pos, hkv, scale);
  }
  return hipGetLastError();
}

hipError_t launch_topk_long(const float* scores, int32_t* idx, int rows, int n, int k, hipStream_t s) {
  hipLaunchKernelGGL(topk_long_kernel, dim3(rows), dim3(kLongThreads), 0, s, scores, idx, n, k);
  return hipGetLastError();
}

}  // namespace sparda
