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
// as the B operand. A workgroup owns 32 rows of W (two 16-row tiles) and up
// to 64 sequences; its four waves take a quarter of D each and add their
// partial tiles in LDS. Each x fragment a wave loads feeds both row tiles:
// x is re-read once per workgroup, so its bytes are B/32 of W's. A 128-column step is four MFMAs; MFMA j of a step consumes columns
// 32 j + 8 g .. 32 j + 8 g + 7 in lane group g (lanes 16 g .. 16 g + 15), in W
// and in x alike (the sum over c may run in any order as long as both
// operands follow the same one), so each load instruction reads 64 contiguous
// bytes from each of 16 rows. W streams a chunk of steps ahead of use.
#include "common.h"
#include "launch.h"
#include "prefill_lds.h"

namespace sparda {

typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kProjRows = 16;   // rows of W per tile
constexpr int kProjStep = 128;  // columns per step
constexpr int kProjMaxTiles = 4;  // 16-sequence tiles per workgroup

template <int MT, int NT, int CS>
__global__ __launch_bounds__(256) void qkvf_kernel(const uint8_t* __restrict__ x, const uint8_t* __restrict__ w,
                                                   uint8_t* __restrict__ q, uint8_t* __restrict__ k,
                                                   uint8_t* __restrict__ v, uint8_t* __restrict__ f, int B, int D,
                                                   int Hq, int Hkv) {
  __shared__ f32x4 s_acc[3][NT][MT][kWave];
  const int lane = threadIdx.x % kWave;
  const int wave = threadIdx.x / kWave;
  const int r16 = lane & 15;  // row of W (A) and sequence of the tile (B)
  const int g = lane >> 4;    // column group
  const long n0 = (long)blockIdx.x * (kProjRows * NT);
  const int b0 = blockIdx.y * (16 * kProjMaxTiles);
  const int kq = D / 4;
  const int c0 = wave * kq, c1 = c0 + kq;

  const uint8_t* wrow[NT];
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) wrow[nt] = w + ((n0 + 16 * nt + r16) * (long)D) * 2;
  const uint8_t* xrow[MT];
  bool xok[MT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
    const int b = b0 + 16 * mt + r16;
    xok[mt] = b < B;
    xrow[mt] = x + ((long)min(b, B - 1) * D) * 2;
  }

  // Steps come in chunks of CS (CS * 128 columns). A chunk's x fragments are
  // loaded first, then the next chunk's W fragments, then the chunk is
  // computed: loads complete in issue order, so waiting for this chunk's x
  // never waits for the W loads in flight behind it. Each x fragment serves
  // the NT row tiles of the wave.
  f32x4 acc[NT][MT];
#pragma unroll
  for (int nt = 0; nt < NT; ++nt)
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) acc[nt][mt] = f32x4{0.f, 0.f, 0.f, 0.f};
  // lane group g takes 8 columns of each 32-column slice j: one load
  // instruction reads 64 contiguous bytes of each of 16 rows
  auto wload_chunk = [&](u32x4 (&wf)[NT][CS][4], int c) {
#pragma unroll
    for (int nt = 0; nt < NT; ++nt)
#pragma unroll
      for (int s = 0; s < CS; ++s)
#pragma unroll
        for (int j = 0; j < 4; ++j) wf[nt][s][j] = load16(wrow[nt] + (c + s * kProjStep + 32 * j + 8 * g) * 2);
  };
  const int nchunks = kq / (CS * kProjStep);
  // workgroups start at different chunks, so at any moment they read
  // different parts of x (every wave of a quarter reads the same x columns)
  const int rot = (int)(blockIdx.x % (unsigned)max(nchunks, 1));
  auto chunk_col = [&](int i) { const int r = i + rot; return c0 + (r >= nchunks ? r - nchunks : r) * CS * kProjStep; };
  u32x4 wa[NT][CS][4], wb[NT][CS][4];
  if (nchunks > 0) wload_chunk(wa, chunk_col(0));
  for (int i = 0; i < nchunks; ++i) {
    const int c = chunk_col(i);
    u32x4 xf[CS][MT][4];
#pragma unroll
    for (int s = 0; s < CS; ++s)
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          xf[s][mt][j] = load16(xrow[mt] + (c + s * kProjStep + 32 * j + 8 * g) * 2);
          if (!xok[mt]) xf[s][mt][j] = u32x4{0, 0, 0, 0};
        }
    if (i + 1 < nchunks) wload_chunk(wb, chunk_col(i + 1));
#pragma unroll
    for (int s = 0; s < CS; ++s)
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
          for (int nt = 0; nt < NT; ++nt)
            acc[nt][mt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(wa[nt][s][j]), as_bf16x8(xf[s][mt][j]),
                                                                  acc[nt][mt], 0, 0, 0);
#pragma unroll
    for (int nt = 0; nt < NT; ++nt)
#pragma unroll
      for (int s = 0; s < CS; ++s)
#pragma unroll
        for (int j = 0; j < 4; ++j) wa[nt][s][j] = wb[nt][s][j];
  }
  // steps left over when a quarter of D is not a whole number of chunks
  for (int c = c0 + nchunks * CS * kProjStep; c < c1; c += kProjStep) {
    u32x4 wf[NT][4];
#pragma unroll
    for (int nt = 0; nt < NT; ++nt)
#pragma unroll
      for (int j = 0; j < 4; ++j) wf[nt][j] = load16(wrow[nt] + (c + 32 * j + 8 * g) * 2);
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        u32x4 xf = load16(xrow[mt] + (c + 32 * j + 8 * g) * 2);
        if (!xok[mt]) xf = u32x4{0, 0, 0, 0};
#pragma unroll
        for (int nt = 0; nt < NT; ++nt)
          acc[nt][mt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(wf[nt][j]), as_bf16x8(xf), acc[nt][mt], 0,
                                                                0, 0);
      }
  }

  // sum the four quarters of D
  if (wave > 0) {
#pragma unroll
    for (int nt = 0; nt < NT; ++nt)
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) s_acc[wave - 1][nt][mt][lane] = acc[nt][mt];
  }
  __syncthreads();
  if (wave != 0) return;
#pragma unroll
  for (int nt = 0; nt < NT; ++nt)
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int r = 0; r < 3; ++r) acc[nt][mt] += s_acc[r][nt][mt][lane];

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
  const int by = (B + 16 * kProjMaxTiles - 1) / (16 * kProjMaxTiles);
  // a wave takes two row tiles, so each x fragment it loads feeds two
  // products; from 48 sequences on, chunks are one step (register budget)
#define SPARDA_PROJ(MT, NT, CS)                                                                                \
  hipLaunchKernelGGL((qkvf_kernel<MT, NT, CS>), dim3((unsigned)(rows / (kProjRows * NT)), by), dim3(256), 0, s, \
                     (const uint8_t*)x, (const uint8_t*)w, (uint8_t*)q, (uint8_t*)k, (uint8_t*)v, (uint8_t*)f, B, \
                     D, Hq, Hkv)
  if (tiles <= 1) SPARDA_PROJ(1, 2, 2);
  else if (tiles <= 2) SPARDA_PROJ(2, 2, 2);
  else if (tiles <= 3) SPARDA_PROJ(3, 2, 1);
  else SPARDA_PROJ(4, 2, 1);
#undef SPARDA_PROJ
  return hipGetLastError();
}

}  // namespace sparda
