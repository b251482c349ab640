// The four projections of a layer's hidden state at decode: Q, K, V and the
// Forecast vector, as one GEMM over the concatenated weights
// (bittide.aicompass.dev summary post, paragraph on the four projections each
// layer emits; arXiv abstract on the same post: the Forecast is a fourth
// projection beside Query, Key and Value).
//
//   out[b, n] = sum_c x[b, c] * W[n, c]
//
// for the N = (Hq + 2 Hkv + n_f Hkv) * 128 rows of W, ordered [Q heads | K heads
// | V heads | n_f Forecast sets of Hkv heads]; bf16 inputs, fp32 accumulation,
// rounded to nearest-even bf16 and written to q [B, Hq, 1, 128],
// k and v [B, Hkv, 1, 128] and f [n_f, B, Hkv, 1, 128].
//
// At decode the batch is small (16 to 64 sequences), so the GEMM streams W once
// from HBM (N x D x 2 bytes) and is HBM-bound; the products run on the matrix
// cores (v_mfma_f32_16x16x32_bf16) with rows of W as the A operand and rows of x
// as the B operand. A workgroup owns ROWS rows of W (16-row tiles; 32 in use)
// and up to 64 sequences, and walks D in chunks of 128 columns. Each chunk's 32 weight
// rows and the sequences' hidden-state rows (256 bytes each) come straight
// from global memory into an LDS ring by direct loads, DEPTH - 1 chunks ahead
// of the one being multiplied, so a wave never waits on a load it has just
// issued and no register holds data in flight. Within a chunk, wave v takes
// the 32-column slice v: MFMA fragments of the two row tiles and of every
// sequence tile come from LDS (lane group g holds columns 8 g .. 8 g + 7 of the
// slice, in W and in x alike: the sum over c may run in any order as long as
// both operands follow the same one), and the four waves' partial tiles are
// summed in LDS at the end. x is read once per workgroup, so its bytes are
// B/ROWS of W's.
#include "common.h"
#include "launch.h"
#include "prefill_lds.h"

namespace sparda {

typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kProjChunk = 128;   // columns per chunk: 256 bytes of a row
constexpr int kProjMaxTiles = 4;  // 16-sequence tiles per workgroup, at most

// MT sequence tiles; DEPTH chunk buffers in LDS. A chunk buffer holds ROWS + 16 MT
// rows of 256 bytes (W's rows, then the sequences'), granule q of row r at
// slot q ^ (r % 16) (the swizzle of prefill_lds.h), so that the 16 rows of a
// fragment read hit 16 different bank groups.
template <int ROWS, int MT, int DEPTH>
__global__ __launch_bounds__(256) void qkvf_kernel(const uint8_t* __restrict__ x, const uint8_t* __restrict__ w,
                                                   uint8_t* __restrict__ q, uint8_t* __restrict__ k,
                                                   uint8_t* __restrict__ v, uint8_t* __restrict__ f, int B, int D,
                                                   int Hq, int Hkv) {
  constexpr int NT = ROWS / 16;
  constexpr int kRows = ROWS + 16 * MT;  // rows of a chunk buffer
  constexpr int kBufBytes = kRows * kRowBytes;
  constexpr int kPerWave = kRows / 16;        // direct loads (4 rows each) per wave per chunk
  constexpr int kWLoads = ROWS / 16;     // of them, loads of W's rows
  static_assert(ROWS % 16 == 0 && kRows % 16 == 0, "rows split evenly over four waves");
  static_assert(DEPTH >= 2 && (DEPTH - 2) * kPerWave <= 63, "vmcnt range");
  __shared__ __attribute__((aligned(16))) uint8_t s_ring[DEPTH][kBufBytes];
  const int lane = threadIdx.x % kWave;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const int r16 = lane & 15;  // row of W (A) and sequence of the tile (B)
  const int g = lane >> 4;    // column group
  const long n0 = (long)blockIdx.x * ROWS;
  const int b0 = blockIdx.y * (16 * MT);
  const uint8_t* wbase = w + n0 * D * 2;
  const uint8_t* xbase = x + (long)b0 * D * 2;

  // Load u of this wave fills LDS bytes [(4 u + wave) KiB, + 1 KiB) of a buffer:
  // buffer rows 4 (4 u + wave) .. + 3, W's for the first ROWS / 16 loads, the
  // sequences' after (sequences past B read row B - 1; their outputs are not
  // stored). Offsets are 32-bit: with D <= 2^24, 64 rows stay under 2 GiB.
  uint32_t roff[kPerWave];
#pragma unroll
  for (int u = 0; u < kPerWave; ++u) {
    const int rr = 4 * (4 * u + wave) + (lane >> 4);
    const uint32_t gran = (uint32_t)(((lane & 15) ^ (rr & 15)) << 4);
    const int src_row = u < kWLoads ? rr : min(b0 + rr - ROWS, B - 1) - b0;
    roff[u] = (uint32_t)src_row * (uint32_t)D * 2u + gran;
  }
  auto issue = [&](int c, int buf) {
    const uint32_t m0 = lds_addr(s_ring[buf]);
#pragma unroll
    for (int u = 0; u < kPerWave; ++u)
      dma16_sv_m0(u < kWLoads ? wbase : xbase, roff[u] + (uint32_t)c * (kProjChunk * 2),
                  m0 + (uint32_t)((4 * u + wave) * kWave * 16));
  };
  // wait until at most n of this wave's direct loads are in flight
  auto wait_loads = [&](int chunks_after) {
    switch (chunks_after) {
#define SPARDA_WAIT(N) \
  case N:              \
    __builtin_amdgcn_s_waitcnt(vmcnt_imm(N * kPerWave)); break;
      SPARDA_WAIT(0) SPARDA_WAIT(1) SPARDA_WAIT(2) SPARDA_WAIT(3) SPARDA_WAIT(4) SPARDA_WAIT(5) SPARDA_WAIT(6)
      SPARDA_WAIT(7) SPARDA_WAIT(8)
#undef SPARDA_WAIT
      default: __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
    }
  };
  static_assert(DEPTH - 2 <= 8, "wait_loads covers up to 8 chunks in flight behind the awaited one");

  f32x4 acc[NT][MT];
#pragma unroll
  for (int nt = 0; nt < NT; ++nt)
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) acc[nt][mt] = f32x4{0.f, 0.f, 0.f, 0.f};
  const int nch = D / kProjChunk;
#pragma unroll
  for (int c = 0; c < DEPTH - 1; ++c)
    if (c < nch) issue(c, c);
  const int q_slice = 4 * wave + g;  // this lane's logical granule in every row
  for (int c = 0, buf = 0; c < nch; ++c, buf = buf + 1 == DEPTH ? 0 : buf + 1) {
    // chunk c's loads (each wave waits for its own) are in; the barrier makes
    // them visible to every wave and tells that chunk c - 1's buffer is free
    wait_loads(min(DEPTH - 2, nch - 1 - c));
    lds_sync();
    if (c + DEPTH - 1 < nch) issue(c + DEPTH - 1, buf == 0 ? DEPTH - 1 : buf - 1);
    const uint8_t* cb = s_ring[buf];
    u32x4 af[NT], bf[MT];
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) af[nt] = *reinterpret_cast<const u32x4*>(cb + swz(16 * nt + r16, q_slice));
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) bf[mt] = *reinterpret_cast<const u32x4*>(cb + swz(ROWS + 16 * mt + r16, q_slice));
#pragma unroll
    for (int nt = 0; nt < NT; ++nt)
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
        acc[nt][mt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(af[nt]), as_bf16x8(bf[mt]), acc[nt][mt], 0, 0, 0);
  }

  // sum the four waves' partial tiles (the ring is free once every wave is past
  // its last chunk)
  lds_sync();
  f32x4* s_acc = reinterpret_cast<f32x4*>(&s_ring[0][0]);  // [3][NT][MT][kWave]
  static_assert(3 * NT * MT * kWave * 16 <= DEPTH * kBufBytes, "partial tiles fit the ring");
  if (wave > 0) {
#pragma unroll
    for (int nt = 0; nt < NT; ++nt)
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) s_acc[((wave - 1) * NT + nt) * MT * kWave + mt * kWave + lane] = acc[nt][mt];
  }
  lds_sync();
  if (wave != 0) return;
#pragma unroll
  for (int nt = 0; nt < NT; ++nt)
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int r = 0; r < 3; ++r) acc[nt][mt] += s_acc[(r * NT + nt) * MT * kWave + mt * kWave + lane];

  // The workgroup's 16 * NT rows sit inside one head of one output (they divide 128).
  const int head = (int)(n0 / kHeadDim);
  const int ch = (int)(n0 % kHeadDim) + 4 * g;  // this lane's 4 consecutive rows of tile 0
  uint8_t* dst;
  long bstride;  // bytes between sequences
  if (head < Hq) {
    dst = q + ((long)head * kHeadDim + ch) * 2;
    bstride = (long)Hq * kHeadDim * 2;
  } else if (head < Hq + Hkv) {
    dst = k + ((long)(head - Hq) * kHeadDim + ch) * 2;
    bstride = (long)Hkv * kHeadDim * 2;
  } else if (head < Hq + 2 * Hkv) {
    dst = v + ((long)(head - Hq - Hkv) * kHeadDim + ch) * 2;
    bstride = (long)Hkv * kHeadDim * 2;
  } else {
    const int fh = head - Hq - 2 * Hkv;
    const int set = fh / Hkv;
    dst = f + (((long)set * B * Hkv + fh % Hkv) * kHeadDim + ch) * 2;
    bstride = (long)Hkv * kHeadDim * 2;
  }
#pragma unroll
  for (int nt = 0; nt < NT; ++nt)
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      const int b = b0 + 16 * mt + r16;
      if (b < B) {
        uint2 o;
        o.x = pack_bf16(acc[nt][mt][0], acc[nt][mt][1]);
        o.y = pack_bf16(acc[nt][mt][2], acc[nt][mt][3]);
        *reinterpret_cast<uint2*>(dst + b * bstride + 16 * nt * 2) = o;
      }
    }
}

hipError_t launch_project_qkvf(const void* x, const void* w, void* q, void* k, void* v, void* f, int B, int D, int Hq,
                               int Hkv, int n_f, hipStream_t s) {
  const long rows = (long)(Hq + 2 * Hkv + n_f * Hkv) * kHeadDim;
  const int tiles = (B + 15) / 16;
  // 32 rows of W per workgroup and 5 or 4 chunk buffers (60 to 96 KiB of LDS):
  // at B = 16 and 64, 13.0 and 18.1 us against 13.8 and 18.7 with 10 to 6
  // buffers, 13.1 and 18.8 with 4 and 3, 14.0 and 22.1 with 16 rows and 15.7
  // and 22.2 with 64 rows per workgroup
#define SPARDA_PROJ(R, MT, DEPTH)                                                                                \
  hipLaunchKernelGGL((qkvf_kernel<R, MT, DEPTH>), dim3((unsigned)(rows / R), (B + 16 * MT - 1) / (16 * MT)),   \
                     dim3(256), 0, s,                                                                            \
                     (const uint8_t*)x, (const uint8_t*)w, (uint8_t*)q, (uint8_t*)k, (uint8_t*)v, (uint8_t*)f, B, \
                     D, Hq, Hkv)
  if (tiles <= 1) SPARDA_PROJ(32, 1, 5);
  else if (tiles <= 2) SPARDA_PROJ(32, 2, 5);
  else if (tiles <= 3) SPARDA_PROJ(32, 3, 4);
  else SPARDA_PROJ(32, 4, 4);
#undef SPARDA_PROJ
  return hipGetLastError();
}

}  // namespace sparda
