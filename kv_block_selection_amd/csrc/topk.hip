// Step 3: keep the top-k blocks of each score row (bittide.aicompass.dev
// summary post, paragraph on block-sparse attention: score the cache by block,
// keep the top-k).
//
// One 256-thread workgroup per row. Scores become order-preserving 32-bit keys
// (larger key <=> larger score; -0 ranks as +0; -inf and padding become key 0).
// A 4-pass MSB-first radix select (8-bit digits, LDS histograms) finds the k-th
// largest key K* and how many keys equal to K* must be taken. Thread t owns the
// contiguous index range [t*NPT, (t+1)*NPT), so exclusive scans in thread order
// are scans in block-index order: they rank the ties (lower index first) and
// give every selected block its output slot, which makes the output ascending
// without a sort. Scans are DPP wave scans plus one LDS exchange of the four
// wave totals. Exact: the result depends only on the input bits.
#include "common.h"
#include "launch.h"

namespace sparda {

__device__ __forceinline__ uint32_t order_key(float x) {
  if (!(x > -INFINITY)) return 0u;  // -inf: not a candidate
  const uint32_t u = x == 0.f ? 0u : __float_as_uint(x);  // -0 ranks as +0
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// Exclusive scan over the 256 threads in thread order; also returns the total.
__device__ __forceinline__ int block_exclusive_scan(int v, int* wave_tot, int& total) {
  const int lane = threadIdx.x % kWave;
  const int wid = threadIdx.x / kWave;
  const int incl = wave_incl_scan(v);
  if (lane == kWave - 1) wave_tot[wid] = incl;
  __syncthreads();
  int before = 0;
  total = 0;
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    const int t = wave_tot[w];
    before += w < wid ? t : 0;
    total += t;
  }
  __syncthreads();
  return before + incl - v;
}

template <int NPT>
__global__ __launch_bounds__(256) void topk_kernel(const float* __restrict__ scores,
                                                   int32_t* __restrict__ idx, int nB, int k) {
  __shared__ int hist[256];
  __shared__ int wave_tot[4];
  __shared__ uint32_t s_digit;
  __shared__ int s_above;

  const long row = blockIdx.x;
  const int t = threadIdx.x;
  const float* src = scores + row * nB;

  uint32_t key[NPT];
  int n_cand_local = 0;
#pragma unroll
  for (int j = 0; j < NPT; ++j) {
    const int b = t * NPT + j;
    key[j] = b < nB ? order_key(src[b]) : 0u;
    n_cand_local += key[j] != 0u;
  }
  int n_cand;
  block_exclusive_scan(n_cand_local, wave_tot, n_cand);
  const int kk = min(k, n_cand);

  uint32_t prefix = 0, pmask = 0;
  int remaining = kk;  // how many keys that match the prefix must still be taken
  if (kk > 0 && kk < n_cand) {
    for (int pass = 0; pass < 4; ++pass) {
      const int shift = 24 - 8 * pass;
      hist[t] = 0;
      __syncthreads();
#pragma unroll
      for (int j = 0; j < NPT; ++j)
        if (key[j] != 0u && (key[j] & pmask) == prefix) atomicAdd(&hist[(key[j] >> shift) & 255u], 1);
      __syncthreads();
      // thread t handles digit 255 - t: above = #matching keys in larger digits
      const int h = hist[255 - t];
      int tot;
      const int above = block_exclusive_scan(h, wave_tot, tot);
      if (above < remaining && remaining <= above + h) {
        s_digit = 255u - (uint32_t)t;
        s_above = above;
      }
      __syncthreads();
      prefix |= s_digit << shift;
      pmask |= 255u << shift;
      remaining -= s_above;
      // the next pass rewrites hist only after its own barrier; s_digit and
      // s_above are rewritten only after the barriers inside the next scan
    }
  }
  // kk == n_cand: every candidate is taken (K* = smallest candidate key is not
  // needed: take all keys != 0).
  const bool take_all = kk == n_cand;
  const uint32_t kstar = prefix;

  // Rank the keys equal to K* in index order; take the first `remaining`.
  int eq_local = 0;
#pragma unroll
  for (int j = 0; j < NPT; ++j) eq_local += (!take_all && key[j] == kstar);
  int eq_total;
  int eq_rank = block_exclusive_scan(eq_local, wave_tot, eq_total);
  bool sel[NPT];
  int sel_local = 0;
#pragma unroll
  for (int j = 0; j < NPT; ++j) {
    bool s = false;
    if (key[j] != 0u) {
      if (take_all || key[j] > kstar) {
        s = true;
      } else if (key[j] == kstar) {
        s = eq_rank < remaining;
        ++eq_rank;
      }
    }
    sel[j] = s;
    sel_local += s;
  }
  int sel_total;
  int pos = block_exclusive_scan(sel_local, wave_tot, sel_total);
  int32_t* dst = idx + row * k;
#pragma unroll
  for (int j = 0; j < NPT; ++j)
    if (sel[j]) dst[pos++] = t * NPT + j;
  for (int p = kk + t; p < k; p += 256) dst[p] = -1;
}

hipError_t launch_topk(const float* scores, int32_t* idx, int rows, int nB, int k, hipStream_t s) {
  const int npt = (nB + 255) / 256;
  dim3 grid(rows);
#define SPARDA_TOPK(N) hipLaunchKernelGGL(topk_kernel<N>, grid, dim3(256), 0, s, scores, idx, nB, k)
  if (npt <= 1) SPARDA_TOPK(1);
  else if (npt <= 2) SPARDA_TOPK(2);
  else if (npt <= 4) SPARDA_TOPK(4);
  else if (npt <= 8) SPARDA_TOPK(8);
  else if (npt <= 16) SPARDA_TOPK(16);
  else if (npt <= 32) SPARDA_TOPK(32);
  else return hipErrorInvalidValue;
#undef SPARDA_TOPK
  return hipGetLastError();
}

}  // namespace sparda
