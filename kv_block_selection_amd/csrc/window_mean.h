// Arithmetic of one compressed key window (techwalker.com article on SparDA,
// section 四: windows of 32 keys with stride 16 at inference), shared by the
// full and the incremental compression so that both give the same bits: a
// half window is the fp32 sum of its 16 keys in token order starting from 0,
// and a window is (first half + second half) / 32.
#pragma once

#include "common.h"

namespace sparda {

// acc = sum of the 16 rows tok(0) .. tok(15) (this lane's 16 bytes of each).
template <typename Tag, typename TokPtr>
__device__ __forceinline__ void half_window_sum(TokPtr tok, float* acc) {
  constexpr int E = DT<Tag>::kElems;
  u32x4 v[kStride];
#pragma unroll
  for (int t = 0; t < kStride; ++t) v[t] = load16_nt(tok(t));
#pragma unroll
  for (int e = 0; e < E; ++e) acc[e] = 0.f;
#pragma unroll
  for (int t = 0; t < kStride; ++t) {
    float x[E];
    unpack<Tag>(v[t], x);
#pragma unroll
    for (int e = 0; e < E; ++e) acc[e] += x[e];
  }
}

template <typename Tag>
__device__ __forceinline__ u32x4 window_from_halves(const float* a, const float* b) {
  constexpr int E = DT<Tag>::kElems;
  float m[E];
#pragma unroll
  for (int e = 0; e < E; ++e) m[e] = (a[e] + b[e]) * (1.0f / kKernel);
  return pack<Tag>(m);
}

}  // namespace sparda
