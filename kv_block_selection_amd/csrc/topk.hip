// Step 3: keep the top-k blocks of each score row (bittide.aicompass.dev
// summary post, paragraph on block-sparse attention: score the cache by block,
// keep the top-k).
//
// One 256-thread workgroup per row. Scores become order-preserving 32-bit keys
// (larger key <=> larger score; -0 ranks as +0; -inf and padding become key 0,
// never taken). Every key at or above a lower bound L of the k-th largest key
// is kept, the rest dropped: each wave takes the ceil(k/4)-th largest of its
// lanes' maxima (a ballot search over the bits where those maxima differ, cut
// short after 8 bits, which only lowers it), so each wave holds at least
// ceil(k/4) keys at or above its value and L, the smallest of the four, has at
// least k keys at or above it. A block reduction gives the candidate count and
// the largest key; the radix select then runs on x = key - L over the few
// keys left. Each pass histograms the next <= 8 bits of x among the keys that
// match the prefix fixed so far (per-wave LDS histograms, three buffers in
// rotation), and every wave scans the bins itself to fix the digit holding the
// k-th largest, so a pass needs one barrier; it stops as soon as that digit is
// taken whole. Thread t owns the contiguous index range [t*NPT, (t+1)*NPT); one
// packed exclusive scan in thread order (above-prefix count in the low 16
// bits, equal-prefix count in the high 16) gives every selected block its
// output slot, ranks ties by lower index, and keeps the output ascending
// without a sort. Exact: the result depends only on the input bits.
#include "common.h"
#include "topk_row.h"
#include "launch.h"

namespace sparda {

template <int NPT>
__global__ __launch_bounds__(256) void topk_kernel(const float* __restrict__ scores,
                                                   int32_t* __restrict__ idx, int nB, int k) {
  __shared__ TopkShared<> sh;
  const long row = blockIdx.x;
  topk_row<NPT>(scores + row * nB, idx + row * k, nullptr, nB, k, sh, threadIdx.x);
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
