// Step 2 for a chunk of queries (prefill): Forecast block scoring of every
// 64-query tile (bittide.aicompass.dev summary post, paragraph on one Forecast
// head per GQA group; techwalker.com article, sections 二 and 五: in prefill the
// gain comes from the cheaper selection itself).
//
// A dense contraction: per KV head, F [Tq x 128] times K_cmp^T [128 x W], so it
// runs on the matrix cores (v_mfma_f32_32x32x16_bf16). One 512-thread
// workgroup owns one (sequence, KV head) and two query tiles (128 queries) and
// sweeps the windows in chunks of 256, so each chunk staged in LDS serves both
// tiles:
//   * the workgroup's 128 rows of F are staged once through LDS, and every wave
//     keeps the fragments of all 128 queries in registers (4 x 32 queries);
//   * each chunk's compressed keys (256 x 256 B) land in LDS through direct
//     global->LDS loads into two buffers; each 16-byte granule of row r is
//     stored at position (granule ^ (r & 15)), so the fragment reads of 16
//     consecutive rows hit 16 different bank groups;
//   * wave v owns windows [32 v, 32 v + 32) of every chunk: one key fragment
//     per K step serves four products (the 4 x 32 queries);
//   * each window's score is masked where the window is not visible to the
//     query, and reduced to the max over each tile's queries (in-lane, then one
//     swap of the two lane halves);
//   * block b takes the max over windows 4b-1 .. 4b+3: chunk c finishes blocks
//     64c .. 64c+63, reusing the previous chunk's last window (a one-window
//     carry), so no window is computed twice and no workgroup waits on another.
//
// The two waves of a SIMD work out of phase. Waves 0-3 (group 0) and 4-7
// (group 1) share the SIMDs pairwise, and each chunk takes two phases, each
// ended by a barrier. In a phase one group runs its 32 products per wave from
// registers while the other reduces its previous chunk to window maxima, pools
// a finished chunk into block scores and reads its next chunk's key fragments
// into registers; so the matrix cores of a SIMD alternate between its two
// waves instead of idling while both reduce. The loads of chunk c + 1 go out
// in phase 2c: group 0's in its memory phase, group 1's between its products.
#include "prefill_lds.h"

namespace sparda {

// Barrier that publishes this wave's LDS writes but leaves its global->LDS
// loads in flight (a fence here would wait for those too).
__device__ __forceinline__ void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

// A phase boundary: nothing is scheduled across it, so the products stay in
// their phase.
__device__ __forceinline__ void phase_barrier() {
  __builtin_amdgcn_sched_barrier(0);
  lds_barrier();
  __builtin_amdgcn_sched_barrier(0);
}

__global__ __launch_bounds__(512) void fsel_prefill_kernel(const uint8_t* __restrict__ f,
                                                           const uint8_t* __restrict__ kc,
                                                           float* __restrict__ scores, int Tq, int q_start, int W,
                                                           int nB, int n_tiles, float scale) {
  constexpr int CW = 2 * kChunkW;  // windows per chunk: 32 per wave
  constexpr int CB = CW * kRowBytes;
  __shared__ __attribute__((aligned(16))) uint8_t s_kc[2][CB];
  __shared__ float s_cmax[2][2][CW + 1];  // [c % 2][tile][0] = carry: last window of chunk c - 1

  const long row = blockIdx.x;  // (b, h): rows on the fast axis share an XCD
  const int v = threadIdx.x / kWave;
  const int grp = v / 4;
  const int lane = threadIdx.x % kWave;
  const int half = lane >> 5;
  const int l32 = lane & 31;
  const uint8_t* kc_row = kc + row * (long)W * kRowBytes;
  const int tile0 = blockIdx.y * 2;  // tile0 + 1 may be n_tiles (an odd count's last workgroup): no output
  const int q0 = tile0 * kTile;      // first query of the workgroup (relative to the chunk)

  // visibility: window w is visible to query position p iff 16 w + 31 <= p;
  // a tile's first query sees the fewest windows
  int vis_min[2];
#pragma unroll
  for (int t = 0; t < 2; ++t) vis_min[t] = visible_windows(q_start + min(q0 + t * kTile, Tq - 1), W);
  const int n = (W + CW - 1) / CW;

  u32x4 fa[4][8];  // A operands: 4 M-tiles of 32 queries x 8 K steps
  u32x4 bf[8];     // B operands: this wave's 32 windows x 8 K steps
  f32x16 acc[4];   // [M-tile]: queries 32 m .. 32 m + 31 x this wave's windows

  const ChunkLoader<8, CW> ld;
  const uint32_t kc_lds = lds_addr(s_kc[0]);
  // this wave's eighth of chunk c (rows past W - 1 read row W - 1; masked)
  auto load_one = [&](int it, int c) { ld.one(it, kc_row, W, c * CW, kc_lds + (uint32_t)((c & 1) * CB)); };
  auto load = [&](int c) {
#pragma unroll
    for (int it = 0; it < ChunkLoader<8, CW>::kLoads; ++it) load_one(it, c);
  };
  auto read_frags = [&](int c) {
    const uint8_t* tileb = s_kc[c & 1];
#pragma unroll
    for (int s = 0; s < 8; ++s) bf[s] = chunk_frag(tileb, 32 * v + l32, s, half);
  };
  // the products of the chunk whose fragments are in bf
  auto products = [&]() {
#pragma unroll
    for (int m = 0; m < 4; ++m) acc[m] = f32x16{};
#pragma unroll
    for (int s = 0; s < 8; ++s)
#pragma unroll
      for (int m = 0; m < 4; ++m)
        acc[m] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(fa[m][s]), as_bf16x8(bf[s]), acc[m], 0, 0, 0);
  };
  // the same with this wave's loads of chunk load_c between the K steps
  auto products_load = [&](int load_c) {
#pragma unroll
    for (int m = 0; m < 4; ++m) acc[m] = f32x16{};
#pragma unroll
    for (int s = 0; s < 8; ++s) {
#pragma unroll
      for (int m = 0; m < 4; ++m)
        acc[m] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(fa[m][s]), as_bf16x8(bf[s]), acc[m], 0, 0, 0);
      __builtin_amdgcn_sched_barrier(0);
      load_one(s, load_c);
      __builtin_amdgcn_sched_barrier(0);
    }
  };
  // window maxima of chunk c over each tile's visible queries
  auto reduce = [&](int c) {
    const int wr = 32 * v + l32;  // this lane's window row in the chunk
    const int w = c * CW + wr;
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      float cm;
      if (scale > 0.f && c * CW + 32 * v + 31 < vis_min[t]) {
        // every window of this wave is visible to every query of the tile, and
        // with scale > 0 the max of the scaled scores is the scaled max (same
        // bits)
        float a = -INFINITY;
#pragma unroll
        for (int r = 0; r < 16; ++r) a = fmaxf(a, fmaxf(acc[2 * t][r], acc[2 * t + 1][r]));
        cm = max32(a) * scale;
      } else {
        // accumulator row r of M-tile m holds query 32 m + 8 (r / 4) + 4 half +
        // r % 4. Window w is visible to query q iff w < W and 16 w + 31 <=
        // q_start + min(q, Tq - 1); with q = q0 + 64 t + 4 half + k, k = 32 m' +
        // 8 (r / 4) + r % 4 a compile-time offset, that is k >= d for this
        // lane's bound d
        const int th = 16 * w + 31 - q_start;
        const int d = (w < W && Tq - 1 >= th) ? th - q0 - 64 * t - 4 * half : 64;
        cm = -INFINITY;
#pragma unroll
        for (int m = 0; m < 2; ++m)
#pragma unroll
          for (int r = 0; r < 16; ++r)
            if (32 * m + 8 * (r >> 2) + (r & 3) >= d) cm = fmaxf(cm, acc[2 * t + m][r] * scale);
        cm = max32(cm);
      }
      if (half == 0) s_cmax[c & 1][t][1 + wr] = cm;
    }
  };
  // blocks of chunk c for tile t (one wave), and the carry into chunk c + 1:
  // slot 0 of a chunk's maxima is read only by the lane of its block 0
  auto pool = [&](int c, int t) {
    const int tile = tile0 + t;
    const float* cm = s_cmax[c & 1][t];
    const int b = c * (CW / 4) + lane;
    if (b < nB && tile < n_tiles) {
      float m = cm[4 * lane];
#pragma unroll
      for (int j = 1; j < 5; ++j) m = fmaxf(m, cm[4 * lane + j]);
      scores[(row * n_tiles + tile) * (long)nB + b] = m;
    }
    if (lane == 0) s_cmax[(c + 1) & 1][t][0] = cm[CW];
  };

  // Prologue: the workgroup's 128 rows of F into the second buffer (the same
  // row layout as a chunk of K_cmp; rows past Tq - 1 read row Tq - 1) and
  // chunk 0 into the first; every wave takes its F fragments, and the second
  // buffer is free again after the barrier.
  if (threadIdx.x < 2) s_cmax[0][threadIdx.x][0] = -INFINITY;
  {
    const ChunkLoader<8, 2 * kTile> fld;
#pragma unroll
    for (int it = 0; it < ChunkLoader<8, 2 * kTile>::kLoads; ++it)
      fld.one(it, f + row * Tq * (long)kRowBytes, Tq, q0, kc_lds + (uint32_t)CB);
  }
  load(0);
  __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
  __syncthreads();
#pragma unroll
  for (int m = 0; m < 4; ++m)
#pragma unroll
    for (int s = 0; s < 8; ++s) fa[m][s] = chunk_frag(s_kc[1], 32 * m + l32, s, half);
  __syncthreads();

  // Phases 2c and 2c + 1 of chunk c. Chunk c sits in buffer c % 2 from the
  // end of phase 2c - 1 (its loads went out in phase 2c - 2, and each wave
  // waits for its own at the end of phase 2c - 1); group 0 reads its
  // fragments in phase 2c and group 1 in phase 2c + 1, so the buffer takes
  // chunk c + 2 from phase 2c + 2 on. The maxima of chunk c come from group 0
  // in phase 2c + 2 and from group 1 in phase 2c + 3; wave 0 (tile 0) and
  // wave 4 (tile 1) pool the chunk in phases 2c + 4 and 2c + 5, while the
  // maxima of chunk c + 1 go to the other half of s_cmax.
  if (grp == 0) {
    for (int c = 0; c <= n + 1; ++c) {
      // memory phase 2c: maxima of c - 1, blocks of c - 2, loads of c + 1,
      // fragments of c (after the maxima, so they reuse the accumulators'
      // registers)
      if (c >= 1 && c <= n) reduce(c - 1);
      if (c >= 2 && v == 0) pool(c - 2, 0);
      __builtin_amdgcn_sched_barrier(0);
      if (c + 1 < n) load(c + 1);
      if (c < n) read_frags(c);
      phase_barrier();
      // compute phase 2c + 1: products of chunk c
      if (c < n) products();
      __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
      phase_barrier();
    }
  } else {
    if (1 < n) load(1);  // phase 0 has no products for this group
    for (int c = 0; c <= n + 1; ++c) {
      // compute phase 2c: products of chunk c - 1 with the loads of c + 1
      if (c >= 1 && c <= n) {
        if (c + 1 < n) {
          products_load(c + 1);
        } else {
          products();
        }
      }
      phase_barrier();
      // memory phase 2c + 1: maxima of c - 1, blocks of c - 2, fragments of c
      if (c >= 1 && c <= n) reduce(c - 1);
      if (c >= 2 && v == 4) pool(c - 2, 1);
      __builtin_amdgcn_sched_barrier(0);
      if (c < n) read_frags(c);
      __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
      phase_barrier();
    }
  }
}

hipError_t launch_select_forecast_prefill(const void* f, const void* kc, float* scores, const SelectDims& d,
                                          hipStream_t s) {
  dim3 grid(d.B * d.Hkv, (d.n_tiles + 1) / 2);
  hipLaunchKernelGGL(fsel_prefill_kernel, grid, dim3(512), 0, s, (const uint8_t*)f, (const uint8_t*)kc, scores, d.Tq,
                     d.q_start, d.W, d.nB, d.n_tiles, d.scale);
  return hipGetLastError();
}

}  // namespace sparda
