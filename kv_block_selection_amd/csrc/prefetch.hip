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

// ------------------------------------------------- staging as a block cache --
// The same gather with the staging buffer kept as a cache across calls: each
// (sequence, KV head) row owns n_slots staging slots whose tags name the block
// they hold. A persistent workgroup takes a row, matches the row's selected
// blocks against the tags in LDS (a hit keeps its slot), hands each missing
// block a slot that no selected block occupies (ascending slot order), writes
// slot_of and the new tags, then copies only the misses. n_slots >= k, so
// there are always enough free slots: a kept slot holds a hit, and hits plus
// misses are at most k.
__device__ __forceinline__ int wave_prefix(bool flag, int lane, int& total) {
  const unsigned long long m = __ballot(flag);
  total = __popcll(m);
  return __popcll(m & ((1ull << lane) - 1ull));
}

__global__ __launch_bounds__(256) void prefetch_cached_kernel(
    const uint8_t* __restrict__ host_k, const uint8_t* __restrict__ host_v, const int32_t* __restrict__ idx,
    int32_t* __restrict__ slot_tags, int32_t* __restrict__ slot_of, uint8_t* __restrict__ stage_k,
    uint8_t* __restrict__ stage_v, int rows, int nB, int k, int n_slots, int block_bytes) {
  __shared__ int s_idx[kCacheMaxK];     // selected block of slot j, -1 = none
  __shared__ int s_slot[kCacheMaxK];    // staging slot of slot j (hit, assigned, or -1)
  __shared__ int s_tag[kCacheMaxSlots];  // block held by each staging slot
  __shared__ int s_keep[kCacheMaxSlots]; // slot holds a block selected in this call
  __shared__ int s_free[kCacheMaxSlots]; // free slots, ascending
  __shared__ int s_miss[kCacheMaxK];    // slots j that miss, ascending
  __shared__ int s_nmiss;
  const int t = threadIdx.x;
  const int lane = t % kWave;
  const int vec_per_block = block_bytes / 16;
  for (long row = blockIdx.x; row < rows; row += gridDim.x) {
    for (int j = t; j < k; j += 256) {
      const int b = idx[row * k + j];
      s_idx[j] = b >= 0 && b < nB ? b : -1;
    }
    for (int sl = t; sl < n_slots; sl += 256) {
      s_tag[sl] = slot_tags[row * n_slots + sl];
      s_keep[sl] = 0;
    }
    __syncthreads();
    // hits: the first slot whose tag is the block
    for (int j = t; j < k; j += 256) {
      const int b = s_idx[j];
      int hit = -1;
      if (b >= 0)
        for (int sl = 0; sl < n_slots; ++sl)
          if (s_tag[sl] == b) {
            hit = sl;
            break;
          }
      s_slot[j] = hit;
      if (hit >= 0) s_keep[hit] = 1;  // several writers store the same value
    }
    __syncthreads();
    if (t < kWave) {  // one wave compacts the free slots and the misses
      int nfree = 0, nmiss = 0;
      for (int base = 0; base < n_slots; base += kWave) {
        const int sl = base + lane;
        const bool f = sl < n_slots && !s_keep[sl];
        int cnt;
        const int pos = wave_prefix(f, lane, cnt);
        if (f) s_free[nfree + pos] = sl;
        nfree += cnt;
      }
      for (int base = 0; base < k; base += kWave) {
        const int j = base + lane;
        const bool m = j < k && s_idx[j] >= 0 && s_slot[j] < 0;
        int cnt;
        const int pos = wave_prefix(m, lane, cnt);
        if (m) s_miss[nmiss + pos] = j;
        nmiss += cnt;
      }
      if (lane == 0) s_nmiss = nmiss;
    }
    __syncthreads();
    const int nmiss = s_nmiss;
    for (int m = t; m < nmiss; m += 256) {
      const int j = s_miss[m];
      const int sl = s_free[m];
      s_slot[j] = sl;
      s_tag[sl] = s_idx[j];
    }
    __syncthreads();
    for (int j = t; j < k; j += 256) slot_of[row * k + j] = s_slot[j];
    for (int sl = t; sl < n_slots; sl += 256) slot_tags[row * n_slots + sl] = s_tag[sl];
    // copy the misses, K then V, one 16 KiB (bf16) block at a time
    for (int it = 0; it < 2 * nmiss; ++it) {
      const bool is_v = it >= nmiss;
      const int j = s_miss[is_v ? it - nmiss : it];
      const int beta = s_idx[j];
      const int sl = s_slot[j];
      const uint8_t* src = (is_v ? host_v : host_k) + (row * nB + beta) * (long)block_bytes;
      uint8_t* dst = (is_v ? stage_v : stage_k) + (row * n_slots + sl) * (long)block_bytes;
      for (int base = 0; base < vec_per_block; base += 4 * 256) {
        u32x4 v[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const int vi = base + u * 256 + t;
          if (vi < vec_per_block) v[u] = load16_nt(src + (long)vi * 16);
        }
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const int vi = base + u * 256 + t;
          if (vi < vec_per_block) store16(dst + (long)vi * 16, v[u]);
        }
      }
    }
    __syncthreads();  // LDS is reused by the next row
  }
}

hipError_t launch_prefetch_cached(const void* host_k, const void* host_v, const int32_t* idx, int32_t* slot_tags,
                                  int32_t* slot_of, void* stage_k, void* stage_v, int elem_bytes, int B, int Hkv,
                                  int nB, int k, int n_slots, int num_workgroups, hipStream_t s) {
  const int rows = B * Hkv;
  const int block_bytes = kBlock * kHeadDim * elem_bytes;
  hipLaunchKernelGGL(prefetch_cached_kernel, dim3(num_workgroups), dim3(256), 0, s, (const uint8_t*)host_k,
                     (const uint8_t*)host_v, idx, slot_tags, slot_of, (uint8_t*)stage_k, (uint8_t*)stage_v, rows, nB,
                     k, n_slots, block_bytes);
  return hipGetLastError();
}

}  // namespace sparda
