// Decode-time state maintenance: append the new tokens' keys and values to
// the KV caches at each sequence's current length, and compress every window
// that the new tokens complete (the cache grows by one token per decode step;
// windows of 32 keys with stride 16 from the techwalker.com article on SparDA,
// section 四).
//
// One launch per call. Each (sequence, KV head) row gets ceil(items / 16)
// workgroups (bf16; 8 lane groups of 32 lanes for fp32), where the items are
// the n_new key rows, the n_new value rows and the windows the new tokens can
// complete; a lane group copies one 256-byte token row or pools one window.
// A window's keys before the old length come from the cache and the rest from
// the new tokens themselves, so the launch never reads a cache row it writes.
// The window arithmetic is that of the full compression (same bits).
#include "common.h"
#include "launch.h"
#include "window_mean.h"

namespace sparda {

// Windows that tokens at positions L .. L + n - 1 can complete: at most one
// per 16 positions, plus one.
__host__ __device__ inline int max_completed_windows(int n) { return n > 0 ? (n - 1) / kStride + 1 : 0; }

template <typename Tag>
__global__ __launch_bounds__(256) void append_kernel(const uint8_t* __restrict__ k_new,
                                                     const uint8_t* __restrict__ v_new,
                                                     uint8_t* __restrict__ k_cache, uint8_t* __restrict__ v_cache,
                                                     uint8_t* __restrict__ k_cmp, const int* __restrict__ seq_len,
                                                     int* __restrict__ status, int hkv, int n_new, int T_cap,
                                                     int W_cap) {
  constexpr int E = DT<Tag>::kElems;
  constexpr int LPR = kHeadDim / E;  // lanes per token row
  constexpr int GPB = 256 / LPR;     // lane groups per workgroup
  constexpr int RB = kHeadDim * DT<Tag>::kBytes;
  const long row = blockIdx.x;
  const int L = seq_len[row / hkv];
  if (L < 0 || L > T_cap - n_new) {  // the tokens would not fit: the row is left as it is
    if (status != nullptr && blockIdx.y == 0 && threadIdx.x == 0) atomicOr(status, 1);
    return;
  }
  const int lane = threadIdx.x % LPR;
  const int item = blockIdx.y * GPB + threadIdx.x / LPR;
  const long off = lane * 16;
  if (item < 2 * n_new) {
    const bool is_v = item >= n_new;
    const int i = is_v ? item - n_new : item;
    const uint8_t* src = (is_v ? v_new : k_new) + (row * n_new + i) * (long)RB + off;
    uint8_t* dst = (is_v ? v_cache : k_cache) + (row * (long)T_cap + L + i) * RB + off;
    store16(dst, load16_nt(src));
    return;
  }
  if (k_cmp == nullptr) return;
  // window w is complete once position 16 w + 31 is written
  const int last = L + n_new - 1;
  const int w_lo = L >= kKernel - 1 ? (L - kKernel + 1 + kStride - 1) / kStride : 0;
  const int w_hi = last >= kKernel - 1 ? min(W_cap - 1, (last - kKernel + 1) / kStride) : -1;
  const int w = w_lo + (item - 2 * n_new);
  if (w > w_hi) return;
  const uint8_t* cache_row = k_cache + row * (long)T_cap * RB + off;
  const uint8_t* new_row = k_new + row * (long)n_new * RB + off;
  auto half_sum = [&](int h, float* acc) {
    half_window_sum<Tag>(
        [&](int t) {
          const int pos = h * kStride + t;
          return pos < L ? cache_row + (long)pos * RB : new_row + (long)(pos - L) * RB;
        },
        acc);
  };
  float a[E], b[E];
  half_sum(w, a);
  half_sum(w + 1, b);
  store16(k_cmp + (row * (long)W_cap + w) * RB + off, window_from_halves<Tag>(a, b));
}

hipError_t launch_append_kv(const void* k_new, const void* v_new, void* k_cache, void* v_cache, void* k_cmp,
                            const int* seq_len, int* status, bool bf16, int B, int Hkv, int n_new, int T_cap,
                            int W_cap, hipStream_t s) {
  const int items = 2 * n_new + (k_cmp != nullptr ? max_completed_windows(n_new) : 0);
  const int gpb = bf16 ? 256 / (kHeadDim / DT<BF16Tag>::kElems) : 256 / (kHeadDim / DT<F32Tag>::kElems);
  const dim3 grid((unsigned)(B * Hkv), (unsigned)((items + gpb - 1) / gpb));
  if (bf16)
    hipLaunchKernelGGL(append_kernel<BF16Tag>, grid, dim3(256), 0, s, (const uint8_t*)k_new, (const uint8_t*)v_new,
                       (uint8_t*)k_cache, (uint8_t*)v_cache, (uint8_t*)k_cmp, seq_len, status, Hkv, n_new, T_cap,
                       W_cap);
  else
    hipLaunchKernelGGL(append_kernel<F32Tag>, grid, dim3(256), 0, s, (const uint8_t*)k_new, (const uint8_t*)v_new,
                       (uint8_t*)k_cache, (uint8_t*)v_cache, (uint8_t*)k_cmp, seq_len, status, Hkv, n_new, T_cap,
                       W_cap);
  return hipGetLastError();
}

int append_grid_y(bool bf16, int n_new, bool with_windows) {
  const int items = 2 * n_new + (with_windows ? max_completed_windows(n_new) : 0);
  const int gpb = bf16 ? 256 / (kHeadDim / DT<BF16Tag>::kElems) : 256 / (kHeadDim / DT<F32Tag>::kElems);
  return (items + gpb - 1) / gpb;
}

}  // namespace sparda
