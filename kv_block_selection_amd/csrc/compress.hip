// Step 1: mean-pooled key windows, kernel 32 and stride 16 (techwalker.com
// article on SparDA, section 四: compressed-key windows used at inference).
//
// HBM-bound stream: read K once, write K_cmp (1/16 of K). The same kernels
// serve a window range [w_begin, w_end) of a cache whose rows hold T_cap
// tokens and W_cap windows (incremental compression while decoding: a
// sequence that has grown past 16 w + 31 tokens completes window w). Each
// 16-token half-window sum is formed once, in token order (the bits of
// half_window_sum, which the append path uses too), and shared by the two
// windows that contain it. bf16: one wave per (row, run of windows), four
// consecutive halves per step, 16 KiB contiguous; fp32: a 32-lane group per
// (row, run of windows), 4 channels a lane, walking its tokens in order.
#include "common.h"
#include "launch.h"
#include "window_mean.h"

namespace sparda {

// windows per wave (bf16) or lane group (fp32); bf16 at 128K: 32 853 µs, 64
// 829, 128 815, 256 816
constexpr int kCompressChunk = 128;

// Stores of K_cmp beside the stream of K reads. The writes, 1/16 of the reads,
// cost more than their bytes at any address pattern (a plain kernel that reads
// 4 GiB takes 0.62 ms, 0.80 ms when it also writes 256 MiB); a buffer store
// with the sc1 cache-policy bit (device scope) takes 3% off this kernel against
// a plain store. The buffer covers one wave's run of windows (at most
// kCompressChunk rows of K_cmp, so offsets stay small), and stores past its
// end would be dropped.
struct RunStore {
  __amdgpu_buffer_rsrc_t rs;
  __device__ __forceinline__ RunStore(uint8_t* run_base, int bytes)
      : rs(__builtin_amdgcn_make_buffer_rsrc(run_base, (short)0, bytes, 0x00020000)) {}
  __device__ __forceinline__ void put(int off, const u32x4& v) const {
    __builtin_amdgcn_raw_buffer_store_b128(v, rs, off, 0, 16);
  }
};

// bf16, one wave per (row, run of kCompressChunk windows): a step takes four
// consecutive half windows, lane group g (16 lanes, 8 channels each) summing
// half 4 s + g over its 16 tokens in token order, so the wave's 16 load
// instructions of a step cover 16 KiB contiguous and each half's sum has the
// bits of half_window_sum. Window 4 s + g then adds the half of lane group
// g + 1 (the next step's group 0 for g = 3), fetched across lanes.
__global__ __launch_bounds__(256) void compress_wave_kernel(const uint8_t* __restrict__ k, uint8_t* __restrict__ kc,
                                                            int rows, int T, int W, int w_begin, int w_end,
                                                            int chunks_per_row) {
  constexpr int RB = kHeadDim * 2;  // bf16 row bytes
  const int lane = threadIdx.x % kWave;
  const int c16 = lane & 15;  // 16-byte slice of a row: channels 8 c16 .. + 7
  const int g = lane >> 4;    // lane group: half 4 s + g of step s
  const long item = (long)blockIdx.x * (256 / kWave) + threadIdx.x / kWave;
  if (item >= (long)rows * chunks_per_row) return;
  const long row = item / chunks_per_row;
  const int w0 = w_begin + (int)(item % chunks_per_row) * kCompressChunk;
  const int w1 = min(w_end, w0 + kCompressChunk);  // windows [w0, w1); halves w0 .. w1
  const uint8_t* src = k + row * (long)T * RB + c16 * 16;
  const RunStore dst(kc + (row * (long)W + w0) * RB, (w1 - w0) * RB);

  // the 16 token rows of half h; halves past w1 (never summed into a stored
  // window) read half w1 instead, so every load is unconditional
  auto load_half = [&](int h, u32x4 (&v)[kStride]) {
    const long t0 = (long)min(h, w1) * kStride;
#pragma unroll
    for (int t = 0; t < kStride; ++t) v[t] = load16_nt(src + (t0 + t) * RB);
  };
  auto half_sum = [&](const u32x4 (&v)[kStride], float* acc) {
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[e] = 0.f;
#pragma unroll
    for (int t = 0; t < kStride; ++t) {
      float x[8];
      unpack<BF16Tag>(v[t], x);
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[e] += x[e];
    }
  };
  // the value of lane (lane + 16) % 64: group g + 1's half, group 0's for g = 3
  auto from_next_group = [&](float x) {
    return __int_as_float(__builtin_amdgcn_ds_bpermute(((lane + 16) & 63) << 2, __float_as_int(x)));
  };

  // Step s covers windows w0 + 4 s + g. Its halves' sums (a) come from the
  // step before; the halves of step s + 1 were loaded during step s - 1, and
  // step s issues the loads of step s + 2 into the buffer its own halves left
  // (summed during step s - 1). The two buffers alternate, so no register that
  // a load in flight fills is copied, and the loads of step s + 2 stay in
  // flight while step s sums.
  const int nsteps = (w1 - w0 + 3) / 4;
  u32x4 vA[kStride], vB[kStride];
  float a[8], n[8];
  load_half(w0 + g, vA);
  load_half(w0 + 4 + g, vB);
  half_sum(vA, a);
  auto step = [&](int st, const u32x4 (&cur)[kStride], u32x4 (&fre)[kStride]) {
    const int hb = w0 + 4 * st;  // this step's first half
    load_half(hb + 8 + g, fre);
    half_sum(cur, n);  // halves hb + 4 .. hb + 7
    // window hb + g = half hb + g + half hb + g + 1: group g + 1's sum of this
    // step, or for g = 3 group 0's of the next
    float b[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float pa = from_next_group(a[e]), pn = from_next_group(n[e]);
      b[e] = g < 3 ? pa : pn;
    }
    const int w = hb + g;
    if (w < w1) dst.put((w - w0) * RB + c16 * 16, window_from_halves<BF16Tag>(a, b));
#pragma unroll
    for (int e = 0; e < 8; ++e) a[e] = n[e];
  };
  int st = 0;
  for (; st + 1 < nsteps; st += 2) {
    step(st, vB, vA);
    step(st + 1, vA, vB);
  }
  if (st < nsteps) step(st, vB, vA);
}

// fp32 (a 32-lane group per run of windows; the bf16 form above)
template <typename Tag>
__global__ __launch_bounds__(256) void compress_kernel(const uint8_t* __restrict__ k,
                                                       uint8_t* __restrict__ kc, int rows, int T,
                                                       int W, int w_begin, int w_end, int chunks_per_row) {
  constexpr int E = DT<Tag>::kElems;
  constexpr int LPR = kHeadDim / E;        // lanes per token row
  constexpr int GPB = 256 / LPR;           // lane groups per workgroup
  constexpr int RB = kHeadDim * DT<Tag>::kBytes;  // row bytes
  const int lane_in_row = threadIdx.x % LPR;
  const long group = (long)blockIdx.x * GPB + threadIdx.x / LPR;
  if (group >= (long)rows * chunks_per_row) return;
  const long row = group / chunks_per_row;
  const int w0 = w_begin + (int)(group % chunks_per_row) * kCompressChunk;
  const int w1 = min(w_end, w0 + kCompressChunk);

  const uint8_t* src = k + row * (long)T * RB + lane_in_row * 16;
  uint8_t* dst = kc + row * (long)W * RB + lane_in_row * 16;

  // half-window h covers tokens [16h, 16h+16)
  auto half_sum = [&](int h, float* acc) {
    half_window_sum<Tag>([&](int t) { return src + (long)(h * kStride + t) * RB; }, acc);
  };

  float prev[E], next[E];
  half_sum(w0, prev);
  for (int w = w0; w < w1; ++w) {
    half_sum(w + 1, next);
    store16(dst + (long)w * RB, window_from_halves<Tag>(prev, next));
#pragma unroll
    for (int e = 0; e < E; ++e) prev[e] = next[e];
  }
}

hipError_t launch_compress(const void* k, void* kc, bool bf16, int rows, int T, int W, int w_begin, int w_end,
                           hipStream_t s) {
  const int chunks = (w_end - w_begin + kCompressChunk - 1) / kCompressChunk;
  const long groups = (long)rows * chunks;
  if (bf16) {
    const int wpb = 256 / kWave;  // one wave per (row, run of windows)
    dim3 grid((unsigned)((groups + wpb - 1) / wpb));
    hipLaunchKernelGGL(compress_wave_kernel, grid, dim3(256), 0, s, (const uint8_t*)k, (uint8_t*)kc, rows, T, W,
                       w_begin, w_end, chunks);
  } else {
    const int gpb = 256 / (kHeadDim / DT<F32Tag>::kElems);
    dim3 grid((unsigned)((groups + gpb - 1) / gpb));
    hipLaunchKernelGGL(compress_kernel<F32Tag>, grid, dim3(256), 0, s, (const uint8_t*)k,
                       (uint8_t*)kc, rows, T, W, w_begin, w_end, chunks);
  }
  return hipGetLastError();
}

}  // namespace sparda
