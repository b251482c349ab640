// Step 1: mean-pooled key windows, kernel 32 and stride 16 (techwalker.com
// article on SparDA, section 四: compressed-key windows used at inference).
//
// HBM-bound stream: read K once, write K_cmp (1/16 of K). The same kernel
// serves a window range [w_begin, w_end) of a cache whose rows hold T_cap
// tokens and W_cap windows (incremental compression while decoding: a
// sequence that has grown past 16 w + 31 tokens completes window w). A 16-lane group
// (bf16; 32 lanes for fp32) owns one (row, window chunk) and walks its tokens
// in order; each lane keeps 8 (or 4) channels. Each 16-token half-window sum is
// formed once and shared by the two windows that contain it. Per load
// instruction a wave reads 4 (bf16) or 2 (fp32) whole 256-byte token rows:
// 1 KiB contiguous per row group, fully used.
#include "common.h"
#include "launch.h"
#include "window_mean.h"

namespace sparda {

constexpr int kCompressChunk = 64;  // windows per lane group (64: 4% faster than 32 at 128K, 8: 12% slower)

template <typename Tag>
__global__ __launch_bounds__(256) void compress_kernel(const uint8_t* __restrict__ k,
                                                       uint8_t* __restrict__ kc, int rows, int T,
                                                       int W, int w_begin, int w_end, int chunks_per_row) {
  constexpr int E = DT<Tag>::kElems;
  constexpr int LPR = kHeadDim / E;        // lanes per token row
  constexpr int GPB = 256 / LPR;           // lane groups per workgroup
  constexpr int RB = kHeadDim * DT<Tag>::kBytes;  // row bytes
  const int lane_in_row = threadIdx.x % LPR;
  const long group = (long)blockIdx.x * GPB + threadIdx.x / LPR;
  if (group >= (long)rows * chunks_per_row) return;
  const long row = group / chunks_per_row;
  const int w0 = w_begin + (int)(group % chunks_per_row) * kCompressChunk;
  const int w1 = min(w_end, w0 + kCompressChunk);

  const uint8_t* src = k + row * (long)T * RB + lane_in_row * 16;
  uint8_t* dst = kc + row * (long)W * RB + lane_in_row * 16;

  // half-window h covers tokens [16h, 16h+16)
  auto half_sum = [&](int h, float* acc) {
    half_window_sum<Tag>([&](int t) { return src + (long)(h * kStride + t) * RB; }, acc);
  };

  float prev[E], next[E];
  half_sum(w0, prev);
  for (int w = w0; w < w1; ++w) {
    half_sum(w + 1, next);
    store16(dst + (long)w * RB, window_from_halves<Tag>(prev, next));
#pragma unroll
    for (int e = 0; e < E; ++e) prev[e] = next[e];
  }
}

hipError_t launch_compress(const void* k, void* kc, bool bf16, int rows, int T, int W, int w_begin, int w_end,
                           hipStream_t s) {
  const int chunks = (w_end - w_begin + kCompressChunk - 1) / kCompressChunk;
  const long groups = (long)rows * chunks;
  if (bf16) {
    const int gpb = 256 / (kHeadDim / DT<BF16Tag>::kElems);
    dim3 grid((unsigned)((groups + gpb - 1) / gpb));
    hipLaunchKernelGGL(compress_kernel<BF16Tag>, grid, dim3(256), 0, s, (const uint8_t*)k,
                       (uint8_t*)kc, rows, T, W, w_begin, w_end, chunks);
  } else {
    const int gpb = 256 / (kHeadDim / DT<F32Tag>::kElems);
    dim3 grid((unsigned)((groups + gpb - 1) / gpb));
    hipLaunchKernelGGL(compress_kernel<F32Tag>, grid, dim3(256), 0, s, (const uint8_t*)k,
                       (uint8_t*)kc, rows, T, W, w_begin, w_end, chunks);
  }
  return hipGetLastError();
}

}  // namespace sparda
