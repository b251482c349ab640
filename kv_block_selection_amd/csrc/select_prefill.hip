// Step 2 for a chunk of queries (prefill): Forecast block scoring of every
// 64-query tile (bittide.aicompass.dev summary post, paragraph on one Forecast
// head per GQA group; techwalker.com article, sections 二 and 五: in prefill the
// gain comes from the cheaper selection itself).
//
// A dense contraction: per KV head, F [Tq x 128] times K_cmp^T [128 x W], so it
// runs on the matrix cores (v_mfma_f32_32x32x16_bf16). One workgroup owns one
// (sequence, KV head) and TPW query tiles (two when the chunk has two or more;
// 4 waves per tile), and sweeps the windows in chunks of 128, so each chunk
// staged in LDS serves every tile of the workgroup:
//   * the chunk's compressed keys (128 x 256 B) land in LDS through direct
//     global->LDS loads, issued two chunks ahead into three buffers (one ahead
//     into two for a one-tile workgroup); each 16-byte granule of row r is
//     stored at position (granule ^ (r & 15)), so the fragment reads of 16
//     consecutive rows hit 16 different bank groups. Each wave waits for its
//     own loads (vmcnt) and the barriers wait for LDS writes only, so the
//     loads of later chunks stay in flight across them;
//   * wave w computes the 64 x 32 score block of windows [32 (w % 4), +32) for
//     the 64 queries of tile w / 4, with that tile's F fragments in registers;
//   * each window's score is masked where the window is not visible to the
//     query, and reduced to the max over the tile's queries (in-lane, then one
//     swap of the two lane halves);
//   * block b takes the max over windows 4b-1 .. 4b+3: chunk c finishes blocks
//     32c .. 32c+31, reusing the previous chunk's last window (a one-window
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
  constexpr int NBUF = TPW == 2 ? 3 : 2;  // chunk buffers; loads go NBUF - 1 chunks ahead
  constexpr int LPC = kChunkBytes / (NWAVES * kWave * 16);  // direct loads per wave per chunk
  __shared__ __attribute__((aligned(16))) uint8_t s_kc[NBUF][kChunkBytes];
  __shared__ float s_cmax[TPW][kChunkW + 1];  // [t][0] = carry: last window of the previous chunk

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
  // visibility: window w is visible to query position p iff 16 w + 31 <= p
  // the tile's first query sees the fewest windows
  const int vis_min = visible_windows(q_start + min(q0, Tq - 1), W);
  int vis_lim[2][16];  // per accumulator row: number of visible windows
#pragma unroll
  for (int m = 0; m < 2; ++m)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int q = q0 + 32 * m + 8 * (r >> 2) + 4 * half + (r & 3);
      vis_lim[m][r] = visible_windows(q_start + min(q, Tq - 1), W);
    }

  const int nchunks = (W + kChunkW - 1) / kChunkW;
  if (threadIdx.x < TPW) s_cmax[threadIdx.x][0] = -INFINITY;
  for (int a = 0; a < NBUF - 1 && a < nchunks; ++a) load_chunk_lds<NWAVES>(kc_row, W, a * kChunkW, s_kc[a]);
  __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
  __syncthreads();
  // Chunk c + NBUF - 1 goes out at the top of iteration c, into the buffer
  // that chunk c - 1 used (every wave left it at the previous barrier).
  int bc = 0;  // buffer of chunk c
  for (int c = 0; c < nchunks; ++c) {
    const int bl = bc == 0 ? NBUF - 1 : bc - 1;  // buffer for chunk c + NBUF - 1
    if (c + NBUF - 1 < nchunks) load_chunk_lds<NWAVES>(kc_row, W, (c + NBUF - 1) * kChunkW, s_kc[bl]);
    const uint8_t* tileb = s_kc[bc];
    f32x16 acc0 = {}, acc1 = {};
    const int wr = 32 * wave + l32;  // this lane's window row in the chunk
#pragma unroll
    for (int s = 0; s < 8; ++s) {
      const u32x4 b = chunk_frag(tileb, wr, s, half);
      acc0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(fa[0][s]), as_bf16x8(b), acc0, 0, 0, 0);
      acc1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(fa[1][s]), as_bf16x8(b), acc1, 0, 0, 0);
    }
    // column (window) max over the tile's visible queries
    const int w = c * kChunkW + wr;
    float cm;
    if (scale > 0.f && c * kChunkW + 32 * wave + 31 < vis_min) {
      // every window of this wave is visible to every query of the tile, and
      // with scale > 0 the max of the scaled scores is the scaled max (same bits)
      float a = -INFINITY;
#pragma unroll
      for (int r = 0; r < 16; ++r) a = fmaxf(a, fmaxf(acc0[r], acc1[r]));
      cm = max32(a) * scale;
    } else {
      cm = -INFINITY;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        if (w < vis_lim[0][r]) cm = fmaxf(cm, acc0[r] * scale);
        if (w < vis_lim[1][r]) cm = fmaxf(cm, acc1[r] * scale);
      }
      cm = max32(cm);
    }
    if (half == 0) s_cmax[tl][1 + wr] = cm;
    lds_barrier();
    const int t = threadIdx.x;
    if (t < TPW * (kChunkW / 4)) {  // 32 blocks per tile
      const int ot = t / (kChunkW / 4), bt = t % (kChunkW / 4);
      const int b = c * (kChunkW / 4) + bt;
      const int otile = blockIdx.y * TPW + ot;
      if (b < nB && otile < n_tiles) {
        float m = s_cmax[ot][4 * bt];
#pragma unroll
        for (int j = 1; j < 5; ++j) m = fmaxf(m, s_cmax[ot][4 * bt + j]);
        scores[(row * n_tiles + otile) * (long)nB + b] = m;
      }
    }
    // The carry: this chunk's last window becomes the next chunk's window 0.
    // Its readers above are lanes of wave 0 too, earlier in program order (the
    // wait keeps the compiler from moving the copy above them), and the next
    // chunk's writes of s_cmax come after the barrier below.
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    if (t < TPW) s_cmax[t][0] = s_cmax[t][kChunkW];
    // chunk c + 1 has landed: loads complete in order, so at most LPC
    // outstanding (the score store above counts too) leaves only chunk c + 2's
    if (NBUF == 3 && c + 2 < nchunks) {
      __builtin_amdgcn_s_waitcnt(vmcnt_imm(LPC));
    } else {
      __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
    }
    lds_barrier();
    bc = bc == NBUF - 1 ? 0 : bc + 1;
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
