// Device fill for the seeded synthetic inputs: the same definition as the numpy
// code in synth/__init__.py (SplitMix64 stream per (seed, tag), 65537-knot
// inverse-CDF table, separately rounded fp32 operations, round-to-nearest-even
// bf16), so both produce identical bits. Inputs only: no step of the
// block-selection method is computed here.
#include <hip/hip_runtime.h>
#include <stdint.h>

#pragma clang fp contract(off)

namespace {

constexpr uint64_t kGamma = 0x9E3779B97F4A7C15ull;

__device__ __forceinline__ uint64_t mix64(uint64_t z) {
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return z ^ (z >> 31);
}

__device__ __forceinline__ float std_normal(uint64_t base, uint64_t i, const float* __restrict__ table) {
  const uint64_t r = mix64(base + (i + 1) * kGamma);
  const uint32_t j = (uint32_t)(r >> 48);
  const float u = __fmul_rn((float)(uint32_t)((r >> 32) & 0xFFFFu), 1.0f / 65536.0f);
  const float t0 = table[j];
  const float t1 = table[j + 1];
  return __fadd_rn(t0, __fmul_rn(u, __fsub_rn(t1, t0)));
}

__device__ __forceinline__ uint16_t to_bf16_rne(float x) {
  const uint32_t b = __float_as_uint(x);
  return (uint16_t)((b + 0x7FFFu + ((b >> 16) & 1u)) >> 16);
}

struct FillArgs {
  uint64_t base;      // stream state of (seed, tag)
  uint64_t off_base;  // stream state of (seed, offset_tag)
  int has_scale;
  float scale;
  int has_offset;
  float offset_std;
  long T, d, block;   // trailing [T, d] geometry for the per-block offset
  long start, n;      // fill flat indices [start, start + n)
  int bf16;
};

__global__ void fill_kernel(FillArgs a, const float* __restrict__ table, void* __restrict__ out) {
  const long stride = (long)gridDim.x * blockDim.x;
  const long nblk = a.T / a.block;
  for (long t = (long)blockIdx.x * blockDim.x + threadIdx.x; t < a.n; t += stride) {
    const long i = a.start + t;
    float z = std_normal(a.base, (uint64_t)i, table);
    if (a.has_scale) z = __fmul_rn(z, a.scale);
    if (a.has_offset) {
      const long c = i % a.d;
      const long tok = (i / a.d) % a.T;
      const long lead = i / (a.d * a.T);
      const long oi = (lead * nblk + tok / a.block) * a.d + c;
      const float zo = std_normal(a.off_base, (uint64_t)oi, table);
      z = __fadd_rn(z, __fmul_rn(a.offset_std, zo));
    }
    if (a.bf16)
      reinterpret_cast<uint16_t*>(out)[t] = to_bf16_rne(z);
    else
      reinterpret_cast<float*>(out)[t] = z;
  }
}

}  // namespace

extern "C" __attribute__((visibility("default"))) int synth_fill(
    void* out, const float* table, uint64_t base, uint64_t off_base, int has_scale, float scale,
    int has_offset, float offset_std, long T, long d, long block, long start, long n, int bf16,
    void* stream) {
  if (n <= 0) return 0;
  if (out == nullptr || table == nullptr || T <= 0 || d <= 0 || block <= 0) return 1;
  FillArgs a{base, off_base, has_scale, scale, has_offset, offset_std, T, d, block, start, n, bf16};
  long blocks = (n + 255) / 256;
  if (blocks > 65536) blocks = 65536;
  hipLaunchKernelGGL(fill_kernel, dim3((unsigned)blocks), dim3(256), 0, (hipStream_t)stream, a, table, out);
  return hipGetLastError() == hipSuccess ? 0 : 2;
}
