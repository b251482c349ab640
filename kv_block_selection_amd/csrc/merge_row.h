// Merge of one (sequence, KV head) row's block-range results at decode, shared
// by the merge kernel and the selection kernel that merges the previous
// layer's attention in the same launch.
#pragma once

#include "common.h"

namespace sparda {

// Each of the row's `splits` block ranges left, per head g, its running max
// and sum (part_ml) and its unnormalised output (part_o). Thread t (t < 32 G)
// takes head t / 32, channels 4 (t % 32) .. + 3: the largest max M over the
// ranges, then each range's sums weighted by exp(max - M), in range order;
// the output is their ratio, rounded to the storage dtype.
template <typename Tag, int MAXS>
__device__ __forceinline__ void merge_row(long row, int t, const float* __restrict__ part_o,
                                          const float2* __restrict__ part_ml, uint8_t* __restrict__ out, int G,
                                          int splits) {
  const int g = t / (kHeadDim / 4);
  const int ch = (t % (kHeadDim / 4)) * 4;
  if (g >= G) return;
  float2 ml[MAXS];
  float4 po[MAXS];
#pragma unroll
  for (int s = 0; s < MAXS; ++s) {
    if (s < splits) {
      ml[s] = part_ml[(row * splits + s) * G + g];
      po[s] = *reinterpret_cast<const float4*>(part_o + ((row * splits + s) * G + g) * kHeadDim + ch);
    }
  }
  float M = -INFINITY;
#pragma unroll
  for (int s = 0; s < MAXS; ++s)
    if (s < splits) M = fmaxf(M, ml[s].x);
  float L = 0.f, O[4] = {0.f, 0.f, 0.f, 0.f};
  if (M != -INFINITY) {
#pragma unroll
    for (int s = 0; s < MAXS; ++s) {
      if (s < splits && ml[s].x != -INFINITY) {
        const float w = fast_exp(ml[s].x - M);
        L = fmaf(ml[s].y, w, L);
        O[0] = fmaf(po[s].x, w, O[0]);
        O[1] = fmaf(po[s].y, w, O[1]);
        O[2] = fmaf(po[s].z, w, O[2]);
        O[3] = fmaf(po[s].w, w, O[3]);
      }
    }
  }
  float o[4];
#pragma unroll
  for (int e = 0; e < 4; ++e) o[e] = L > 0.f ? O[e] / L : 0.f;
  const long off = (row * G + g) * kHeadDim + ch;
  if constexpr (DT<Tag>::kBytes == 2) {
    uint2 v;
    v.x = pack_bf16(o[0], o[1]);
    v.y = pack_bf16(o[2], o[3]);
    *reinterpret_cast<uint2*>(out + off * 2) = v;
  } else {
    *reinterpret_cast<float4*>(out + off * 4) = make_float4(o[0], o[1], o[2], o[3]);
  }
}

// The same merge with the ranges loaded 4 at a time (under 64 registers
// instead of 6 per range), for a kernel whose own work needs few: the same
// operations in the same order, so the same bits.
template <typename Tag>
__device__ __forceinline__ void merge_row_lean(long row, int t, const float* __restrict__ part_o,
                                               const float2* __restrict__ part_ml, uint8_t* __restrict__ out, int G,
                                               int splits) {
  constexpr int SB = 4;
  const int g = t / (kHeadDim / 4);
  const int ch = (t % (kHeadDim / 4)) * 4;
  if (g >= G) return;
  float M = -INFINITY;
  for (int s0 = 0; s0 < splits; s0 += SB) {
    float mx[SB];
#pragma unroll
    for (int i = 0; i < SB; ++i) mx[i] = s0 + i < splits ? part_ml[(row * splits + s0 + i) * G + g].x : -INFINITY;
#pragma unroll
    for (int i = 0; i < SB; ++i) M = fmaxf(M, mx[i]);
  }
  float L = 0.f, O[4] = {0.f, 0.f, 0.f, 0.f};
  if (M != -INFINITY) {
    for (int s0 = 0; s0 < splits; s0 += SB) {
      float2 ml[SB];
      float4 po[SB];
#pragma unroll
      for (int i = 0; i < SB; ++i) {
        if (s0 + i < splits) {
          ml[i] = part_ml[(row * splits + s0 + i) * G + g];
          po[i] = *reinterpret_cast<const float4*>(part_o + ((row * splits + s0 + i) * G + g) * kHeadDim + ch);
        }
      }
#pragma unroll
      for (int i = 0; i < SB; ++i) {
        if (s0 + i < splits && ml[i].x != -INFINITY) {
          const float w = fast_exp(ml[i].x - M);
          L = fmaf(ml[i].y, w, L);
          O[0] = fmaf(po[i].x, w, O[0]);
          O[1] = fmaf(po[i].y, w, O[1]);
          O[2] = fmaf(po[i].z, w, O[2]);
          O[3] = fmaf(po[i].w, w, O[3]);
        }
      }
    }
  }
  float o[4];
#pragma unroll
  for (int e = 0; e < 4; ++e) o[e] = L > 0.f ? O[e] / L : 0.f;
  const long off = (row * G + g) * kHeadDim + ch;
  if constexpr (DT<Tag>::kBytes == 2) {
    uint2 v;
    v.x = pack_bf16(o[0], o[1]);
    v.y = pack_bf16(o[2], o[3]);
    *reinterpret_cast<uint2*>(out + off * 2) = v;
  } else {
    *reinterpret_cast<float4*>(out + off * 4) = make_float4(o[0], o[1], o[2], o[3]);
  }
}

}  // namespace sparda
