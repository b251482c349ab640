// Forecast scoring of a run of blocks of one (sequence, KV head) row at
// decode, shared by the selection kernel and the one-launch decode layer
// kernel. 16 lanes hold one 256-byte window row (8 bf16 each); a wave reads 4
// rows (1 KiB contiguous) per load; v_dot2_f32_bf16 and a DPP butterfly across
// the 16 lanes give each window's score.
#pragma once

#include "common.h"

namespace sparda {

template <typename Tag>
struct RowGeom {
  static constexpr int E = DT<Tag>::kElems;
  static constexpr int LPR = kHeadDim / E;   // lanes per 128-channel row
  static constexpr int SLOTS = 256 / LPR;    // rows per 256-thread pass
  static constexpr int RB = kHeadDim * DT<Tag>::kBytes;
};

// Forecast scores of blocks [NBLK * chunk, NBLK * chunk + NBLK) of one row by
// NT threads (t = thread index): the windows they meet, scored into s_win
// (LDS, at least fsel_lds_floats<Tag, NBLK, NT>() floats), max-pooled per block.
template <typename Tag, int NBLK, int NT = 256>
constexpr int fsel_lds_floats() {
  constexpr int slots = NT / RowGeom<Tag>::LPR;
  return ((4 * NBLK + 1 + slots - 1) / slots) * slots;
}
template <typename Tag, int NBLK, int NT = 256>
__device__ __forceinline__ void fsel_blocks(const uint8_t* __restrict__ f, const uint8_t* __restrict__ kc,
                                            float* __restrict__ scores, int W, int nB, int n_vis,
                                            const int* __restrict__ q_pos, int hkv, int T, float scale, long row,
                                            int chunk, float* s_win, int t) {
  using R = RowGeom<Tag>;
  constexpr int SLOTS = NT / R::LPR;  // window rows per pass of the NT threads
  constexpr int NWIN = 4 * NBLK + 1;
  constexpr int ITER = (NWIN + SLOTS - 1) / SLOTS;
  if (q_pos != nullptr) n_vis = visible_windows(row_position(q_pos, row, hkv, 0, T), W);
  const int beta0 = chunk * NBLK;
  const int nblk = min(NBLK, nB - beta0);
  const int nwin = 4 * nblk + 1;
  const int wstart = 4 * beta0 - 1;
  const int lane = t % R::LPR;
  const int slot = t / R::LPR;

  const u32x4 fv = load16(f + row * R::RB + lane * 16);
  const uint8_t* base = kc + row * (long)W * R::RB + lane * 16;

  u32x4 kv[ITER];
#pragma unroll
  for (int it = 0; it < ITER; ++it) {
    const int lw = it * SLOTS + slot;
    const int w = wstart + lw;
    const bool ok = lw < nwin && w >= 0 && w < n_vis;
    kv[it] = ok ? load16_nt(base + (long)w * R::RB) : u32x4{0, 0, 0, 0};
  }
#pragma unroll
  for (int it = 0; it < ITER; ++it) {
    const int lw = it * SLOTS + slot;
    const int w = wstart + lw;
    const bool ok = lw < nwin && w >= 0 && w < n_vis;
    const float s = group_sum<R::LPR>(dot16<Tag>(fv, kv[it], 0.f));
    if (lane == 0) s_win[lw] = ok ? s * scale : -INFINITY;
  }
  lds_sync();
  if (t < nblk) {
    float m = s_win[4 * t];
#pragma unroll
    for (int j = 1; j < 5; ++j) m = fmaxf(m, s_win[4 * t + j]);
    scores[row * nB + beta0 + t] = m;
  }
}

}  // namespace sparda

