// Internal helpers shared by the libsparda kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <cmath>

#include "launch.h"

namespace sparda {

constexpr int kWave = 64;

// 16 bytes of a row: 8 bf16 or 4 fp32 values.
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

// Number of compressed windows visible to the query at position p: window w
// is visible iff every token of it is at or before p, i.e. 16 w + 31 <= p.
__device__ __forceinline__ int visible_windows(int p, int W) {
  return p >= kKernel - 1 ? min(W, (p - kKernel + 1) / kStride + 1) : 0;
}

// Query position of the (sequence, KV head) row `row` of a decode call: the
// sequence's own entry of q_pos when given (clamped to [-1, T - 1]; -1 leaves
// nothing visible), else the shared position p.
__device__ __forceinline__ int row_position(const int* q_pos, long row, int hkv, int p, int T) {
  if (q_pos == nullptr) return p;
  return min(max(q_pos[row / hkv], -1), T - 1);
}

struct F32Tag {};
struct BF16Tag {};

template <typename Tag> struct DT;
template <> struct DT<F32Tag> {
  static constexpr int kElems = 4;  // per 16-byte vector
  static constexpr int kBytes = 4;
};
template <> struct DT<BF16Tag> {
  static constexpr int kElems = 8;
  static constexpr int kBytes = 2;
};

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// Round-to-nearest-even fp32 -> bf16 pair packed in a dword (lo = a, hi = b).
__device__ __forceinline__ uint32_t pack_bf16(float a, float b) {
  bf16x2 v = {(__bf16)a, (__bf16)b};
  return __builtin_bit_cast(uint32_t, v);
}

// Expand a 16-byte vector into fp32 values.
template <typename Tag>
__device__ __forceinline__ void unpack(const u32x4& v, float* out);
template <>
__device__ __forceinline__ void unpack<BF16Tag>(const u32x4& v, float* out) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    out[2 * i] = bf16_lo(v[i]);
    out[2 * i + 1] = bf16_hi(v[i]);
  }
}
template <>
__device__ __forceinline__ void unpack<F32Tag>(const u32x4& v, float* out) {
#pragma unroll
  for (int i = 0; i < 4; ++i) out[i] = __uint_as_float(v[i]);
}

// Pack fp32 values into a 16-byte vector in storage format.
template <typename Tag>
__device__ __forceinline__ u32x4 pack(const float* in);
template <>
__device__ __forceinline__ u32x4 pack<BF16Tag>(const float* in) {
  u32x4 r;
#pragma unroll
  for (int i = 0; i < 4; ++i) r[i] = pack_bf16(in[2 * i], in[2 * i + 1]);
  return r;
}
template <>
__device__ __forceinline__ u32x4 pack<F32Tag>(const float* in) {
  u32x4 r;
#pragma unroll
  for (int i = 0; i < 4; ++i) r[i] = __float_as_uint(in[i]);
  return r;
}

// Dot product of two 16-byte vectors, fp32 accumulation.
template <typename Tag>
__device__ __forceinline__ float dot16(const u32x4& a, const u32x4& b, float acc);
template <>
__device__ __forceinline__ float dot16<BF16Tag>(const u32x4& a, const u32x4& b, float acc) {
  // Each element goes through a scalar first: __builtin_bit_cast applied to a
  // vector-element lvalue reads element 0 (the whole vector's storage).
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint32_t x = a[i], y = b[i];
    acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, x), __builtin_bit_cast(bf16x2, y),
                                          acc, false);
  }
  return acc;
}
template <>
__device__ __forceinline__ float dot16<F32Tag>(const u32x4& a, const u32x4& b, float acc) {
#pragma unroll
  for (int i = 0; i < 4; ++i) acc = fmaf(__uint_as_float(a[i]), __uint_as_float(b[i]), acc);
  return acc;
}

__device__ __forceinline__ u32x4 load16(const void* p) {
  return *reinterpret_cast<const u32x4*>(p);
}
__device__ __forceinline__ u32x4 load16_nt(const void* p) {
  return __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
}
__device__ __forceinline__ void store16(void* p, const u32x4& v) {
  *reinterpret_cast<u32x4*>(p) = v;
}

// ---- cross-lane reductions (DPP within a 16-lane row) ----
template <int CTRL>
__device__ __forceinline__ float dpp(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, false));
}
// Butterfly over the 16 lanes of a DPP row: xor 1, xor 2, then half-mirror and
// mirror. Every step pairs lanes symmetrically, so all 16 lanes end with the
// bitwise-identical sum.
__device__ __forceinline__ float row16_sum(float x) {
  x += dpp<0xB1>(x);   // quad_perm [1,0,3,2]
  x += dpp<0x4E>(x);   // quad_perm [2,3,0,1]
  x += dpp<0x141>(x);  // row_half_mirror
  x += dpp<0x140>(x);  // row_mirror
  return x;
}
__device__ __forceinline__ float row16_max(float x) {
  x = fmaxf(x, dpp<0xB1>(x));
  x = fmaxf(x, dpp<0x4E>(x));
  x = fmaxf(x, dpp<0x141>(x));
  x = fmaxf(x, dpp<0x140>(x));
  return x;
}
// Lanes l and l ^ 16 (l ^ 32) exchange values with one VALU instruction,
// v_permlane16_swap (v_permlane32_swap), instead of a round trip through the
// LDS crossbar. `lo` is always the lower lane's value, so a pair reduction
// (lo + hi, max(lo, hi)) is bitwise the same in both lanes.
struct LanePair {
  float lo, hi;
};
__device__ __forceinline__ LanePair pair16(float x) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return {__uint_as_float(r[0]), __uint_as_float(r[1])};
}
__device__ __forceinline__ LanePair pair32(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return {__uint_as_float(r[0]), __uint_as_float(r[1])};
}
__device__ __forceinline__ float sum16(float x) {
  const LanePair p = pair16(x);
  return p.lo + p.hi;
}
__device__ __forceinline__ float sum32(float x) {
  const LanePair p = pair32(x);
  return p.lo + p.hi;
}
__device__ __forceinline__ float max16(float x) {
  const LanePair p = pair16(x);
  return fmaxf(p.lo, p.hi);
}
__device__ __forceinline__ float max32(float x) {
  const LanePair p = pair32(x);
  return fmaxf(p.lo, p.hi);
}
// The value held by lane l ^ 32 (waves start at multiples of 64 threads).
__device__ __forceinline__ float partner32(float x) {
  const LanePair p = pair32(x);
  return (threadIdx.x & 32) ? p.lo : p.hi;
}
// Sum over a group of LANES (16 or 32) consecutive lanes; every lane gets it.
template <int LANES>
__device__ __forceinline__ float group_sum(float x) {
  x = row16_sum(x);
  if constexpr (LANES == 32) x = sum16(x);
  return x;
}
__device__ __forceinline__ float wave_sum(float x) { return sum32(sum16(row16_sum(x))); }
__device__ __forceinline__ float wave_max(float x) { return max32(max16(row16_max(x))); }

// Inclusive prefix sum over the 64 lanes of a wave (DPP: row shifts, then
// row broadcasts 15 and 31).
__device__ __forceinline__ int wave_incl_scan(int x) {
  x += __builtin_amdgcn_update_dpp(0, x, 0x111, 0xF, 0xF, false);  // row_shr:1
  x += __builtin_amdgcn_update_dpp(0, x, 0x112, 0xF, 0xF, false);  // row_shr:2
  x += __builtin_amdgcn_update_dpp(0, x, 0x114, 0xF, 0xF, false);  // row_shr:4
  x += __builtin_amdgcn_update_dpp(0, x, 0x118, 0xF, 0xF, false);  // row_shr:8
  x += __builtin_amdgcn_update_dpp(0, x, 0x142, 0xA, 0xF, false);  // row_bcast:15 -> rows 1, 3
  x += __builtin_amdgcn_update_dpp(0, x, 0x143, 0xC, 0xF, false);  // row_bcast:31 -> rows 2, 3
  return x;
}

// s_waitcnt immediate that waits until at most n vector-memory loads are
// outstanding and leaves the other counters alone (gfx9 encoding: vmcnt bits
// 3:0 and 15:14, expcnt 6:4, lgkmcnt 11:8).
// One direct global->LDS load of 16 bytes per lane: lane i's bytes land at
// lds_wave_dst + 16 i. Written as an asm statement so that the compiler, which
// cannot tell which LDS buffer such a load fills, does not make every later
// LDS read (and every workgroup barrier) wait for it: a kernel that uses it
// waits for its own loads (vmcnt) before the barrier that publishes them.
__device__ __forceinline__ void dma16(const uint8_t* gsrc, const uint8_t* lds_wave_dst) {
  const uint32_t base = __builtin_amdgcn_readfirstlane(
      (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) uint8_t*)lds_wave_dst);
  asm volatile("global_load_lds_dwordx4 %0, off" ::"v"(gsrc), "{m0}"(base) : "memory");
}

// Workgroup barrier for LDS hand-offs only: waits for this wave's LDS
// operations, not for its global loads (a __syncthreads fence would wait for
// every load in flight, including ones issued ahead on purpose).
__device__ __forceinline__ void lds_sync() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

constexpr int vmcnt_imm(int n) { return 0x0F70 | (n & 15) | ((n >> 4) << 14); }

__device__ __forceinline__ float fast_exp(float x) {
  return __builtin_amdgcn_exp2f(x * 1.4426950408889634f);
}

}  // namespace sparda
