// Reduction of G dot products at once over the 16 lanes that hold one
// 128-channel row (8 bf16 channels per lane), shared by the decode attention's
// query-key scores and the multi-head selector's window logits.
#pragma once

#include "common.h"

namespace sparda {

// Reduce-scatter of G partial dot products over the 16 lanes of a key row.
// Lane c keeps its query slots in the order head = slot XOR mask(c), with
// mask(c) built from lane bits 3 and 2. Then a lane and its row_ror:8 partner
// (bit 3 flipped) exchange half of their slots, a lane and its half-mirror
// partner (bit 2 flipped) exchange half of the rest, and a quad butterfly
// finishes the sum: each lane ends with the full score of head mask(c), and the
// four lanes that share a head hold bitwise-identical values.
template <int G>
__device__ __forceinline__ int slot_head(int slot, int c) {
  if constexpr (G == 1) {
    return 0;
  } else if constexpr (G == 2) {
    return slot ^ ((c >> 3) & 1);
  } else {
    const int mask = (((c >> 3) & 1) << 1) | ((c >> 2) & 1);
    return (slot & ~3) | ((slot & 3) ^ mask);  // G = 8: two independent groups of 4
  }
}

template <int G>
__device__ __forceinline__ void reduce_scatter16(const float* part, float* out) {
  if constexpr (G == 1) {
    out[0] = row16_sum(part[0]);
  } else if constexpr (G == 2) {
    float a = part[0] + dpp<0x128>(part[1]);  // row_ror:8
    a += dpp<0x141>(a);                       // row_half_mirror
    a += dpp<0xB1>(a);
    a += dpp<0x4E>(a);
    out[0] = a;
  } else {
#pragma unroll
    for (int grp = 0; grp < G / 4; ++grp) {
      const float* pp = part + 4 * grp;
      const float a0 = pp[0] + dpp<0x128>(pp[2]);
      const float a1 = pp[1] + dpp<0x128>(pp[3]);
      float b = a0 + dpp<0x141>(a1);
      b += dpp<0xB1>(b);
      b += dpp<0x4E>(b);
      out[grp] = b;
    }
  }
}

}  // namespace sparda
