// Step 5: lookahead prefetch of the next layer's selected blocks from pinned
// host memory into a device staging buffer (bittide.aicompass.dev summary
// post, paragraph on prefetching over a separate stream; techwalker.com
// article, sections 二 and 三: a persistent kernel with a few workgroups pulls
// the blocks through host-mapped memory, the block indices never leave the GPU).
//
// A fixed set of workgroups walks the (sequence, head, slot, K|V) items. Each
// item is one 64-token block: 16 KiB contiguous in host memory for bf16. The
// kernel reads the index from device memory, loads the block straight from
// host memory over the host link (pinned memory is mapped into the GPU's
// address space) and stores it to HBM. Loads are 16 B per lane, four in flight
// per lane per block, so a 256-thread workgroup keeps 16 KiB of reads
// outstanding on the link.
#include "common.h"
#include "launch.h"

namespace sparda {

__global__ __launch_bounds__(256) void prefetch_kernel(const uint8_t* __restrict__ host_k,
                                                       const uint8_t* __restrict__ host_v,
                                                       const int32_t* __restrict__ idx,
                                                       uint8_t* __restrict__ stage_k,
                                                       uint8_t* __restrict__ stage_v, int rows, int nB,
                                                       int k, int block_bytes) {
  const long items = 2L * rows * k;
  const int vec_per_block = block_bytes / 16;
  for (long it = blockIdx.x; it < items; it += gridDim.x) {
    const bool is_v = it & 1;
    const long slot = it >> 1;  // row * k + j
    const long row = slot / k;
    const int beta = idx[slot];
    if (beta < 0 || beta >= nB) continue;
    const uint8_t* src = (is_v ? host_v : host_k) + (row * nB + beta) * (long)block_bytes;
    uint8_t* dst = (is_v ? stage_v : stage_k) + slot * (long)block_bytes;
    for (int base = 0; base < vec_per_block; base += 4 * 256) {
      u32x4 v[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int vi = base + u * 256 + threadIdx.x;
        if (vi < vec_per_block) v[u] = load16_nt(src + (long)vi * 16);
      }
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int vi = base + u * 256 + threadIdx.x;
        if (vi < vec_per_block) store16(dst + (long)vi * 16, v[u]);
      }
    }
  }
}

hipError_t launch_prefetch(const void* host_k, const void* host_v, const int32_t* idx, void* stage_k,
                           void* stage_v, int elem_bytes, int B, int Hkv, int nB, int k,
                           int num_workgroups, hipStream_t s) {
  const int rows = B * Hkv;
  const int block_bytes = kBlock * kHeadDim * elem_bytes;
  hipLaunchKernelGGL(prefetch_kernel, dim3(num_workgroups), dim3(256), 0, s, (const uint8_t*)host_k,
                     (const uint8_t*)host_v, idx, (uint8_t*)stage_k, (uint8_t*)stage_v, rows, nB, k,
                     block_bytes);
  return hipGetLastError();
}

}  // namespace sparda
