// Step 3: keep the top-k blocks of each score row (bittide.aicompass.dev
// summary post, paragraph on block-sparse attention: score the cache by block,
// keep the top-k).
//
// One 256-thread workgroup per row. Scores become order-preserving 32-bit keys
// (larger key <=> larger score; -0 ranks as +0; -inf and padding become key 0,
// never taken). A block reduction gives the candidate count and the smallest
// and largest candidate keys; the radix select then runs on x = key - kmin, so
// its first digit already splits the row's actual range (float keys of one
// row share their top bits, which would put every key in one or two bins).
// Each pass histograms the next <= 8 bits of x among the keys that match the
// prefix fixed so far (per-wave LDS histograms), one wave scans the bins and
// fixes the digit holding the k-th largest; it stops as soon as that digit is
// taken whole. Thread t owns the contiguous index range [t*NPT, (t+1)*NPT); one
// packed exclusive scan in thread order (above-prefix count in the low 16
// bits, equal-prefix count in the high 16) gives every selected block its
// output slot, ranks ties by lower index, and keeps the output ascending
// without a sort. Exact: the result depends only on the input bits.
#include "common.h"
#include "launch.h"

namespace sparda {

__device__ __forceinline__ uint32_t order_key(float x) {
  if (!(x > -INFINITY)) return 0u;  // -inf: not a candidate
  const uint32_t u = x == 0.f ? 0u : __float_as_uint(x);  // -0 ranks as +0
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ __forceinline__ uint32_t wave_umin(uint32_t v) {
  for (int m = 1; m < kWave; m <<= 1) v = min(v, (uint32_t)__shfl_xor((int)v, m, kWave));
  return v;
}
__device__ __forceinline__ uint32_t wave_umax(uint32_t v) {
  for (int m = 1; m < kWave; m <<= 1) v = max(v, (uint32_t)__shfl_xor((int)v, m, kWave));
  return v;
}
__device__ __forceinline__ int wave_isum(int v) {
  for (int m = 1; m < kWave; m <<= 1) v += __shfl_xor(v, m, kWave);
  return v;
}

struct TopkShared {
  int hist[2][4][256];  // [ping-pong][wave][digit]
  int wave_tot[4];
  uint32_t wave_min[4], wave_max[4];
  int wave_cnt[4];
  uint32_t digit;
  int above, done;
};

template <int NPT>
__global__ __launch_bounds__(256) void topk_kernel(const float* __restrict__ scores,
                                                   int32_t* __restrict__ idx, int nB, int k) {
  __shared__ TopkShared sh;
  const long row = blockIdx.x;
  const int t = threadIdx.x;
  const int lane = t % kWave;
  const int wid = t / kWave;
  const float* src = scores + row * nB;

  uint32_t key[NPT];
  int cnt = 0;
  uint32_t kmin = 0xFFFFFFFFu, kmax = 0u;
#pragma unroll
  for (int j = 0; j < NPT; ++j) {
    const int b = t * NPT + j;
    key[j] = b < nB ? order_key(src[b]) : 0u;
    if (key[j] != 0u) {
      ++cnt;
      kmin = min(kmin, key[j]);
      kmax = max(kmax, key[j]);
    }
  }
#pragma unroll
  for (int w = 0; w < 4; ++w) sh.hist[0][w][t] = 0;
  cnt = wave_isum(cnt);
  kmin = wave_umin(kmin);
  kmax = wave_umax(kmax);
  if (lane == 0) {
    sh.wave_cnt[wid] = cnt;
    sh.wave_min[wid] = kmin;
    sh.wave_max[wid] = kmax;
  }
  __syncthreads();
  int n_cand = 0;
  kmin = 0xFFFFFFFFu;
  kmax = 0u;
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    n_cand += sh.wave_cnt[w];
    kmin = min(kmin, sh.wave_min[w]);
    kmax = max(kmax, sh.wave_max[w]);
  }
  const int kk = min(k, n_cand);
  const bool take_all = kk == n_cand;  // includes the empty row

  // radix select on x = key - kmin over the bits below `lo`
  uint32_t prefix = 0;
  int remaining = kk;
  int lo = take_all ? 0 : 32 - __clz(kmax - kmin);
  int cur = 0;
  while (lo > 0) {
    const int sft = max(lo - 8, 0);
    const uint32_t dmask = (1u << (lo - sft)) - 1u;
    const uint32_t phi = lo >= 32 ? 0u : prefix >> lo;
#pragma unroll
    for (int j = 0; j < NPT; ++j) {
      if (key[j] != 0u) {
        const uint32_t x = key[j] - kmin;
        if ((lo >= 32 ? 0u : x >> lo) == phi) atomicAdd(&sh.hist[cur][wid][(x >> sft) & dmask], 1);
      }
    }
#pragma unroll
    for (int w = 0; w < 4; ++w) sh.hist[cur ^ 1][w][t] = 0;
    __syncthreads();
    if (wid == 0) {
      // lane handles digits 255-4*lane .. 252-4*lane (descending)
      int h[4], sum = 0;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int d = 255 - 4 * lane - i;
        h[i] = sh.hist[cur][0][d] + sh.hist[cur][1][d] + sh.hist[cur][2][d] + sh.hist[cur][3][d];
        sum += h[i];
      }
      int above = wave_incl_scan(sum) - sum;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        if (above < remaining && remaining <= above + h[i]) {
          sh.digit = (uint32_t)(255 - 4 * lane - i);
          sh.above = above;
          sh.done = remaining == above + h[i];  // the whole digit is taken
        }
        above += h[i];
      }
    }
    __syncthreads();
    prefix |= sh.digit << sft;
    remaining -= sh.above;
    lo = sft;
    cur ^= 1;
    if (sh.done) break;
    // sh.digit / above / done are rewritten only after the next pass's first barrier
  }

  // Packed scan: low 16 bits = keys above the prefix, high 16 = keys equal to it.
  const uint32_t plo = lo >= 32 ? 0u : prefix >> lo;
  int gt = 0, eq = 0;
#pragma unroll
  for (int j = 0; j < NPT; ++j) {
    if (key[j] != 0u) {
      const uint32_t top = lo >= 32 ? 0u : (key[j] - kmin) >> lo;
      gt += top > plo;
      eq += top == plo;
    }
  }
  const int packed = gt | (eq << 16);
  const int incl = wave_incl_scan(packed);
  if (lane == kWave - 1) sh.wave_tot[wid] = incl;
  __syncthreads();
  int before = incl - packed;
#pragma unroll
  for (int w = 0; w < 4; ++w) before += w < wid ? sh.wave_tot[w] : 0;
  int eq_rank = before >> 16;
  int pos = (before & 0xFFFF) + min(eq_rank, remaining);
  int32_t* dst = idx + row * k;
#pragma unroll
  for (int j = 0; j < NPT; ++j) {
    if (key[j] != 0u) {
      const uint32_t top = lo >= 32 ? 0u : (key[j] - kmin) >> lo;
      if (top > plo) {
        dst[pos++] = t * NPT + j;
      } else if (top == plo) {
        if (eq_rank < remaining) dst[pos++] = t * NPT + j;
        ++eq_rank;
      }
    }
  }
  for (int q = kk + t; q < k; q += 256) dst[q] = -1;
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
