// Staging of compressed-key chunks in LDS for the prefill selectors: 128 (or
// 256) windows x 128 bf16 channels (32 or 64 KiB) per chunk, loaded straight from global
// memory into LDS, with a granule swizzle so the matrix-core fragment reads of
// 16 consecutive rows hit 16 different bank groups.
#pragma once

#include "common.h"
#include "launch.h"
#include "lds_dma.h"

namespace sparda {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kChunkW = 128;                 // windows per chunk
constexpr int kRowBytes = kHeadDim * 2;      // one bf16 row
constexpr int kChunkBytes = kChunkW * kRowBytes;

__device__ __forceinline__ bf16x8 as_bf16x8(const u32x4& v) { return __builtin_bit_cast(bf16x8, v); }

// Byte offset of logical 16-byte granule g of row r inside a swizzled chunk.
__device__ __forceinline__ int swz(int r, int g) { return r * kRowBytes + ((g ^ (r & 15)) << 4); }

// Direct global->LDS load of rows [w0, w0 + CW) of one (b, h) row of K_cmp
// into `dst` by a workgroup of NWAVES waves. Lane l of a wave instruction fills
// LDS bytes [base + 16 l, base + 16 l + 16) from the global granule the swizzle
// maps there. Rows at or beyond W read row W - 1 (callers mask them).
template <int NWAVES, int CW = kChunkW>
__device__ __forceinline__ void load_chunk_lds(const uint8_t* __restrict__ kc_row, int W, int w0, uint8_t* dst) {
  constexpr int kBytes = CW * kRowBytes;
  static_assert(kBytes % (NWAVES * kWave * 16) == 0, "chunk must split evenly over the waves");
  const int wave = threadIdx.x / kWave;
  const int lane = threadIdx.x % kWave;
#pragma unroll
  for (int it = 0; it < kBytes / (NWAVES * kWave * 16); ++it) {
    const int pos = (it * NWAVES + wave) * kWave + lane;  // 16-byte slot in the chunk
    const int r = pos >> 4;
    const int g = (pos & 15) ^ (r & 15);
    const int w = min(w0 + r, W - 1);
    const uint8_t* src = kc_row + (long)w * kRowBytes + g * 16;
    dma16(src, dst + (it * NWAVES + wave) * kWave * 16);
  }
}

// The same load of a whole chunk (rows w0 .. w0 + CW - 1 all below W) from a
// scalar base: off[it] holds this lane's offset within the chunk for load
// `it`, from chunk_lds_offsets.
template <int NWAVES, int CW>
struct ChunkOffsets {
  static constexpr int kLoads = CW * kRowBytes / (NWAVES * kWave * 16);
  uint32_t off[kLoads];
};
template <int NWAVES, int CW>
__device__ __forceinline__ ChunkOffsets<NWAVES, CW> chunk_lds_offsets() {
  ChunkOffsets<NWAVES, CW> o;
  const int wave = threadIdx.x / kWave;
  const int lane = threadIdx.x % kWave;
#pragma unroll
  for (int it = 0; it < ChunkOffsets<NWAVES, CW>::kLoads; ++it) {
    const int pos = (it * NWAVES + wave) * kWave + lane;
    const int r = pos >> 4;
    o.off[it] = (uint32_t)(r * kRowBytes + (((pos & 15) ^ (r & 15)) << 4));
  }
  return o;
}
template <int NWAVES, int CW>
__device__ __forceinline__ void load_full_chunk_lds(const uint8_t* __restrict__ kc_row, int w0,
                                                    const ChunkOffsets<NWAVES, CW>& o, uint8_t* dst) {
  const int wave = threadIdx.x / kWave;
  const uint8_t* base = kc_row + (long)w0 * kRowBytes;
#pragma unroll
  for (int it = 0; it < ChunkOffsets<NWAVES, CW>::kLoads; ++it)
    dma16_sv(base, o.off[it], dst + (it * NWAVES + wave) * kWave * 16);
}

// Fragment of a chunk row for a 32x32x16 MFMA operand whose rows (A) or columns
// (B) are windows: lane l reads window row `r` (= 32 * tile + l % 32), channels
// [16 s + 8 (l / 32), +8).
__device__ __forceinline__ u32x4 chunk_frag(const uint8_t* chunk, int r, int s, int half) {
  return *reinterpret_cast<const u32x4*>(chunk + swz(r, 2 * s + half));
}

}  // namespace sparda
