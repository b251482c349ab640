// Step 2 for a chunk of queries (prefill): Forecast block scoring of every
// 64-query tile (bittide.aicompass.dev summary post, paragraph on one Forecast
// head per GQA group; techwalker.com article, sections 二 and 五: in prefill the
// gain comes from the cheaper selection itself).
//
// A dense contraction: per KV head, F [Tq x 128] times K_cmp^T [128 x W], so it
// runs on the matrix cores (v_mfma_f32_32x32x16_bf16). One workgroup owns one
// (sequence, KV head) and TPW query tiles (two when the chunk has two or more;
// 4 waves per tile), and sweeps the windows in chunks of 256, so each chunk
// staged in LDS serves every tile of the workgroup:
//   * the chunk's compressed keys (256 x 256 B) land in LDS through direct
//     global->LDS loads issued one chunk ahead into two buffers; each 16-byte
//     granule of row r is stored at position (granule ^ (r & 15)), so the
//     fragment reads of 16 consecutive rows hit 16 different bank groups. Each
//     wave waits for its own loads (vmcnt) and the barriers wait for LDS
//     writes only, so the next chunk's loads stay in flight across them;
//   * wave w computes the 64 x 64 score block of windows [64 (w % 4), +64) for
//     the 64 queries of tile w / 4 (four products per K step: each window
//     fragment serves both query halves and each F fragment both window
//     halves), with that tile's F fragments in registers;
//   * each window's score is masked where the window is not visible to the
//     query, and reduced to the max over the tile's queries (in-lane, then one
//     swap of the two lane halves);
//   * block b takes the max over windows 4b-1 .. 4b+3: chunk c finishes blocks
//     64c .. 64c+63, reusing the previous chunk's last window (a one-window
//     carry), so no window is computed twice and no workgroup waits on another.
#include "prefill_lds.h"

namespace sparda {

// Barrier that publishes this wave's LDS writes but leaves its global->LDS
// loads in flight (a fence here would wait for those too).
__device__ __forceinline__ void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

template <int TPW>
__global__ __launch_bounds__(256 * TPW) void fsel_prefill_kernel(const uint8_t* __restrict__ f,
                                                                 const uint8_t* __restrict__ kc,
                                                                 float* __restrict__ scores, int Tq,
                                                                 int q_start, int W, int nB, int n_tiles,
                                                                 float scale) {
  constexpr int NWAVES = 4 * TPW;
  constexpr int CW = 2 * kChunkW;                 // windows per chunk: 64 per wave
  constexpr int CB = CW * kRowBytes;              // bytes per chunk
  __shared__ __attribute__((aligned(16))) uint8_t s_kc[2][CB];
  __shared__ float s_cmax[2][TPW][CW + 1];  // [c % 2][t][0] = carry: last window of chunk c - 1

  const long row = blockIdx.x;  // (b, h): rows on the fast axis share an XCD
  const int tl = threadIdx.x / (4 * kWave);  // this wave's tile in the workgroup
  const int tile = blockIdx.y * TPW + tl;    // may be n_tiles (an odd count's last workgroup): no output
  const int wave = (threadIdx.x / kWave) % 4;
  const int lane = threadIdx.x % kWave;
  const int half = lane >> 5;
  const int l32 = lane & 31;
  const uint8_t* kc_row = kc + row * (long)W * kRowBytes;
  const int q0 = tile * kTile;  // first query of the tile (relative to the chunk)

  // F fragments: A operand of the 64 x 128 tile, 2 M-tiles x 8 k-steps
  u32x4 fa[2][8];
#pragma unroll
  for (int m = 0; m < 2; ++m) {
    const int q = min(q0 + 32 * m + l32, Tq - 1);
    const uint8_t* src = f + (row * Tq + q) * (long)kRowBytes + half * 16;
#pragma unroll
    for (int s = 0; s < 8; ++s) fa[m][s] = load16(src + s * 32);
  }
  // visibility: window w is visible to query position p iff 16 w + 31 <= p;
  // the tile's first query sees the fewest windows
  const int vis_min = visible_windows(q_start + min(q0, Tq - 1), W);

  const int nchunks = (W + CW - 1) / CW;
  const ChunkOffsets<NWAVES, CW> offs = chunk_lds_offsets<NWAVES, CW>();
  // whole chunks from a scalar base, the last partial one with clamped rows
  auto load = [&](int c, uint8_t* dst) {
    if ((c + 1) * CW <= W) {
      load_full_chunk_lds<NWAVES, CW>(kc_row, c * CW, offs, dst);
    } else {
      load_chunk_lds<NWAVES, CW>(kc_row, W, c * CW, dst);
    }
  };
  if (threadIdx.x < TPW) s_cmax[0][threadIdx.x][0] = -INFINITY;
  load(0, s_kc[0]);
  __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
  __syncthreads();
  // One barrier per chunk. Iteration c issues chunk c + 1 into the buffer
  // chunk c - 1 used, scores chunk c into window maxima s_cmax[c % 2], waits
  // for its own loads and meets the other waves: chunk c + 1 and the maxima
  // are then visible, and chunk c's buffer is read by none. The block pooling
  // of chunk c runs after that barrier, beside the next chunk's products; the
  // maxima are double-buffered so those writes go to the other half.
  for (int c = 0; c < nchunks; ++c) {
    const int bc = c & 1;
    if (c + 1 < nchunks) load(c + 1, s_kc[bc ^ 1]);
    const uint8_t* tileb = s_kc[bc];
    f32x16 acc[2][2] = {};  // [query half m][window half n]
#pragma unroll
    for (int s = 0; s < 8; ++s) {
      const u32x4 b0 = chunk_frag(tileb, 64 * wave + l32, s, half);
      const u32x4 b1 = chunk_frag(tileb, 64 * wave + 32 + l32, s, half);
#pragma unroll
      for (int m = 0; m < 2; ++m) {
        acc[m][0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(fa[m][s]), as_bf16x8(b0), acc[m][0], 0, 0, 0);
        acc[m][1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(fa[m][s]), as_bf16x8(b1), acc[m][1], 0, 0, 0);
      }
    }
    float* cmax = s_cmax[bc][tl];
    // column (window) max over the tile's visible queries
#pragma unroll
    for (int n = 0; n < 2; ++n) {
      const int wr = 64 * wave + 32 * n + l32;  // this lane's window row in the chunk
      const int w = c * CW + wr;
      float cm;
      if (scale > 0.f && c * CW + 64 * wave + 32 * n + 31 < vis_min) {
        // every window of this lane group is visible to every query of the
        // tile, and with scale > 0 the max of the scaled scores is the scaled
        // max (same bits)
        float a = -INFINITY;
#pragma unroll
        for (int r = 0; r < 16; ++r) a = fmaxf(a, fmaxf(acc[0][n][r], acc[1][n][r]));
        cm = max32(a) * scale;
      } else {
        cm = -INFINITY;
#pragma unroll
        for (int m = 0; m < 2; ++m)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            // accumulator row r of M-tile m holds query 32 m + 8 (r / 4) + 4 half + r % 4
            const int q = q0 + 32 * m + 8 * (r >> 2) + 4 * half + (r & 3);
            if (w < visible_windows(q_start + min(q, Tq - 1), W)) cm = fmaxf(cm, acc[m][n][r] * scale);
          }
        cm = max32(cm);
      }
      if (half == 0) cmax[1 + wr] = cm;
    }
    // chunk c + 1 has landed for this wave's loads; after the barrier for
    // every wave, with this chunk's maxima
    __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
    lds_barrier();
    const int t = threadIdx.x;
    if (t < TPW * (CW / 4)) {  // 64 blocks per tile
      const int ot = t / (CW / 4), bt = t % (CW / 4);
      const int b = c * (CW / 4) + bt;
      const int otile = blockIdx.y * TPW + ot;
      const float* cm = s_cmax[bc][ot];
      if (b < nB && otile < n_tiles) {
        float m = cm[4 * bt];
#pragma unroll
        for (int j = 1; j < 5; ++j) m = fmaxf(m, cm[4 * bt + j]);
        scores[(row * n_tiles + otile) * (long)nB + b] = m;
      }
      // The carry: this chunk's last window becomes window 0 of the next
      // chunk's half. Slot 0 of a half is read only by the thread of block 0,
      // this thread, after the barrier that follows this write.
      if (bt == 0) s_cmax[bc ^ 1][ot][0] = cm[CW];
    }
  }
}

hipError_t launch_select_forecast_prefill(const void* f, const void* kc, float* scores, const SelectDims& d,
                                          hipStream_t s) {
  if (d.n_tiles >= 2) {
    dim3 grid(d.B * d.Hkv, (d.n_tiles + 1) / 2);
    hipLaunchKernelGGL(fsel_prefill_kernel<2>, grid, dim3(512), 0, s, (const uint8_t*)f, (const uint8_t*)kc, scores,
                       d.Tq, d.q_start, d.W, d.nB, d.n_tiles, d.scale);
  } else {
    dim3 grid(d.B * d.Hkv, d.n_tiles);
    hipLaunchKernelGGL(fsel_prefill_kernel<1>, grid, dim3(256), 0, s, (const uint8_t*)f, (const uint8_t*)kc, scores,
                       d.Tq, d.q_start, d.W, d.nB, d.n_tiles, d.scale);
  }
  return hipGetLastError();
}

}  // namespace sparda
