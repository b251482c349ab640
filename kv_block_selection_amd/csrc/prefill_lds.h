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

// Direct loads of a chunk by NWAVES waves (a multiple of 4): load `it` of
// wave v fills LDS bytes [(it NWAVES + v) KiB, +1 KiB), i.e. rows
// 4 (it NWAVES + v) .. +3 of the chunk. Those rows start at a multiple of 16
// plus 4 v, so the swizzle does not depend on `it`: a lane's source is row
// w0 + it * 4 NWAVES + r0 at a fixed granule offset, and the loader keeps two
// registers per lane (no 64-bit address per load). Each lane's row is clamped
// to W - 1, so the last, partial chunk takes the same code (callers mask the
// rows past W - 1). Offsets are 32-bit: a row of K_cmp (or F) is under 2 GiB.
template <int NWAVES, int CW>
struct ChunkLoader {
  static constexpr int kLoads = CW * kRowBytes / (NWAVES * kWave * 16);
  static constexpr int kRowsPerLoad = 4 * NWAVES;
  static_assert(NWAVES % 4 == 0 && kLoads * NWAVES * kWave * 16 == CW * kRowBytes, "chunk must split evenly");
  int r0;         // this lane's row within a load's rows
  uint32_t gran;  // this lane's byte offset within its row
  __device__ __forceinline__ ChunkLoader() {
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    const int lane = threadIdx.x % kWave;
    r0 = 4 * wave + (lane >> 4);
    gran = (uint32_t)(((lane & 15) ^ (r0 & 15)) << 4);
  }
  // load `it` of this wave: rows from w0 of the row block at `base`, into the
  // chunk buffer at LDS address m0
  __device__ __forceinline__ void one(int it, const uint8_t* __restrict__ base, int W, int w0, uint32_t m0) const {
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    const uint32_t r = min(w0 + it * kRowsPerLoad + r0, W - 1);
    dma16_sv_m0(base, r * kRowBytes + gran, m0 + (uint32_t)((it * NWAVES + wave) * kWave * 16));
  }
};

// Fragment of a chunk row for a 32x32x16 MFMA operand whose rows (A) or columns
// (B) are windows: lane l reads window row `r` (= 32 * tile + l % 32), channels
// [16 s + 8 (l / 32), +8).
__device__ __forceinline__ u32x4 chunk_frag(const uint8_t* chunk, int r, int s, int half) {
  return *reinterpret_cast<const u32x4*>(chunk + swz(r, 2 * s + half));
}

}  // namespace sparda
