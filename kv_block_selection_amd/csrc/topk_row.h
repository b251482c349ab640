// The top-k of one score row by a 256-thread workgroup, shared by the top-k
// kernel and the fused top-k + attention kernel. The method is described at
// the top of topk.hip.
#pragma once

#include "common.h"

namespace sparda {

__device__ __forceinline__ uint32_t order_key(float x) {
  if (!(x > -INFINITY)) return 0u;  // -inf: not a candidate
  const uint32_t u = x == 0.f ? 0u : __float_as_uint(x);  // -0 ranks as +0
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

template <int CTRL>
__device__ __forceinline__ uint32_t dppu(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, CTRL, 0xF, 0xF, false);
}
// Value of lane `l` (read as a scalar), kept unsigned: readlane itself is
// typed int, and the keys compare as unsigned.
__device__ __forceinline__ uint32_t lane_u(uint32_t v, int l) {
  return (uint32_t)__builtin_amdgcn_readlane((int)v, l);
}
// Wave reductions: a butterfly inside each 16-lane DPP row, then the four row
// results read as scalars.
__device__ __forceinline__ uint32_t wave_umin(uint32_t v) {
  v = min(v, dppu<0xB1>(v));
  v = min(v, dppu<0x4E>(v));
  v = min(v, dppu<0x141>(v));
  v = min(v, dppu<0x140>(v));
  return min(min(lane_u(v, 0), lane_u(v, 16)), min(lane_u(v, 32), lane_u(v, 48)));
}
__device__ __forceinline__ uint32_t wave_umax(uint32_t v) {
  v = max(v, dppu<0xB1>(v));
  v = max(v, dppu<0x4E>(v));
  v = max(v, dppu<0x141>(v));
  v = max(v, dppu<0x140>(v));
  return max(max(lane_u(v, 0), lane_u(v, 16)), max(lane_u(v, 32), lane_u(v, 48)));
}
__device__ __forceinline__ int wave_isum(int v) {
  uint32_t u = (uint32_t)v;
  u += dppu<0xB1>(u);
  u += dppu<0x4E>(u);
  u += dppu<0x141>(u);
  u += dppu<0x140>(u);
  return (int)(lane_u(u, 0) + lane_u(u, 16) + lane_u(u, 32) + lane_u(u, 48));
}

// A value v with at least r lanes of the wave holding x >= v, and v no larger
// than the r-th largest x: a bitwise search from the highest bit where the
// lanes' x differ, stopped after `bits` bits (the bits below stay 0).
__device__ __forceinline__ uint32_t wave_rank_bound(uint32_t x, int r, int bits) {
  const uint32_t hi = wave_umax(x), lo = wave_umin(x);
  if (hi == lo) return hi;
  const int top = 31 - __clz(hi ^ lo);
  uint32_t v = top == 31 ? 0u : (hi >> (top + 1)) << (top + 1);  // the bits all lanes share
  for (int b = top; b >= 0 && b > top - bits; --b) {
    const uint32_t cand = v | (1u << b);
    if (__popcll(__ballot(x >= cand)) >= r) v = cand;
  }
  return v;
}

template <int NW = 4>
struct TopkShared {
  int hist[3][NW][256];  // [rotation][wave][digit]
  int wave_tot[NW];
  uint32_t wave_max[NW], wave_bound[NW];
  int wave_cnt[NW];
};

// Clears histogram buffer `b` (NW x 256 counters) with the workgroup's NW x 64 threads.
template <int NW>
__device__ __forceinline__ void clear_hist(TopkShared<NW>& sh, int b, int t) {
#pragma unroll
  for (int j = 0; j < 4; ++j) (&sh.hist[b][0][0])[t + j * NW * kWave] = 0;
}

// The k best blocks of one row of nB scores, by the NW x 64 threads of a
// workgroup (t = thread index; NPT scores per thread, NW x 64 x NPT >= nB).
// Its barriers order LDS only, so global loads the caller issued before it
// stay in flight.
// The indices go to dst_g (global memory) and/or dst_s (LDS), either of which
// may be NULL, ascending with -1 padding.
template <int NPT, int NW = 4>
__device__ __forceinline__ void topk_row(const float* __restrict__ src, int32_t* __restrict__ dst_g,
                                         int32_t* dst_s, int nB, int k, TopkShared<NW>& sh, int t) {
  constexpr int NT = NW * kWave;
  const int lane = t % kWave;
  const int wid = t / kWave;

  // All NPT loads go out before any is used: the index is clamped into the
  // row (nB >= 1) and the padding masked afterwards, since a guarded load
  // would wait for each value in turn.
  float x[NPT];
#pragma unroll
  for (int j = 0; j < NPT; ++j) x[j] = src[min(t * NPT + j, nB - 1)];
  uint32_t key[NPT];
  int cnt = 0;
  uint32_t kmax = 0u;
#pragma unroll
  for (int j = 0; j < NPT; ++j) {
    key[j] = t * NPT + j < nB ? order_key(x[j]) : 0u;
    cnt += key[j] != 0u;
    kmax = max(kmax, key[j]);
  }
  clear_hist(sh, 0, t);
  // every wave holds at least rnk keys >= its bound, so NW x rnk >= k keys are
  // >= the smallest bound: the k-th largest key is not below it
  const int rnk = (k + NW - 1) / NW;
  const uint32_t wbound = rnk <= kWave ? wave_rank_bound(kmax, rnk, 8) : 0u;  // kmax: this thread's largest
  cnt = wave_isum(cnt);
  const uint32_t wmax = wave_umax(kmax);
  if (lane == 0) {
    sh.wave_cnt[wid] = cnt;
    sh.wave_max[wid] = wmax;
    sh.wave_bound[wid] = wbound;
  }
  lds_sync();
  int n_cand = 0;
  kmax = 0u;
  uint32_t lb = 0xFFFFFFFFu;
#pragma unroll
  for (int w = 0; w < NW; ++w) {
    n_cand += sh.wave_cnt[w];
    kmax = max(kmax, sh.wave_max[w]);
    lb = min(lb, sh.wave_bound[w]);
  }
  const int kk = min(k, n_cand);
  const bool take_all = kk == n_cand;  // includes the empty row
  // keys below the bound cannot be among the k largest (the bound is 0 when a
  // wave had too few candidates, and then nothing is dropped)
  lb = max(lb, 1u);
#pragma unroll
  for (int j = 0; j < NPT; ++j) key[j] = key[j] >= lb ? key[j] : 0u;

  // radix select on x = key - lb over the bits below `lo`
  uint32_t prefix = 0;
  int remaining = kk;
  int lo = take_all ? 0 : 32 - __clz(kmax - lb);
  int cur = 0;
  while (lo > 0) {
    const int sft = max(lo - 8, 0);
    const uint32_t dmask = (1u << (lo - sft)) - 1u;
    const uint32_t phi = lo >= 32 ? 0u : prefix >> lo;
    const int nxt = cur == 2 ? 0 : cur + 1;
#pragma unroll
    for (int j = 0; j < NPT; ++j) {
      if (key[j] != 0u) {
        const uint32_t x = key[j] - lb;
        if ((lo >= 32 ? 0u : x >> lo) == phi) atomicAdd(&sh.hist[cur][wid][(x >> sft) & dmask], 1);
      }
    }
    // the buffer for the next pass was last read two passes ago, before the
    // previous pass's barrier
    clear_hist(sh, nxt, t);
    lds_sync();
    // every wave: lane handles digits 255-4*lane .. 252-4*lane (descending)
    int h[4], sum = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int d = 255 - 4 * lane - i;
      h[i] = 0;
#pragma unroll
      for (int w = 0; w < NW; ++w) h[i] += sh.hist[cur][w][d];
      sum += h[i];
    }
    int above = wave_incl_scan(sum) - sum;
    bool hit = false;
    uint32_t my_digit = 0;
    int my_above = 0, my_done = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      if (above < remaining && remaining <= above + h[i]) {
        hit = true;
        my_digit = (uint32_t)(255 - 4 * lane - i);
        my_above = above;
        my_done = remaining == above + h[i];  // the whole digit is taken
      }
      above += h[i];
    }
    const int src_lane = __ffsll(__ballot(hit)) - 1;  // exactly one lane holds the digit
    prefix |= lane_u(my_digit, src_lane) << sft;
    remaining -= __builtin_amdgcn_readlane(my_above, src_lane);
    lo = sft;
    cur = nxt;
    if (__builtin_amdgcn_readlane(my_done, src_lane)) break;
  }

  // Packed scan: low 16 bits = keys above the prefix, high 16 = keys equal to it.
  const uint32_t plo = lo >= 32 ? 0u : prefix >> lo;
  int gt = 0, eq = 0;
#pragma unroll
  for (int j = 0; j < NPT; ++j) {
    if (key[j] != 0u) {
      const uint32_t top = lo >= 32 ? 0u : (key[j] - lb) >> lo;
      gt += top > plo;
      eq += top == plo;
    }
  }
  const int packed = gt | (eq << 16);
  const int incl = wave_incl_scan(packed);
  if (lane == kWave - 1) sh.wave_tot[wid] = incl;
  lds_sync();
  int before = incl - packed;
#pragma unroll
  for (int w = 0; w < NW; ++w) before += w < wid ? sh.wave_tot[w] : 0;
  int eq_rank = before >> 16;
  int pos = (before & 0xFFFF) + min(eq_rank, remaining);
  auto put = [&](int at, int32_t v) {
    if (dst_g) dst_g[at] = v;
    if (dst_s) dst_s[at] = v;
  };
#pragma unroll
  for (int j = 0; j < NPT; ++j) {
    if (key[j] != 0u) {
      const uint32_t top = lo >= 32 ? 0u : (key[j] - lb) >> lo;
      // pos < kk holds by construction; the test keeps a row inside its k slots
      if (top > plo) {
        if (pos < kk) put(pos, t * NPT + j);
        ++pos;
      } else if (top == plo) {
        if (eq_rank < remaining && pos < kk) put(pos++, t * NPT + j);
        ++eq_rank;
      }
    }
  }
  for (int q = kk + t; q < k; q += NT) put(q, -1);
}


}  // namespace sparda
