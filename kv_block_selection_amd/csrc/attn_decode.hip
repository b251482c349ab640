// Step 4 at decode: GQA block-sparse attention over the selected blocks
// (bittide.aicompass.dev summary post, paragraphs on block-sparse attention and
// on the next layer attending with its own queries; 10100.com commentary,
// section 解法).
//
// HBM-bound: each (sequence, KV head) row reads k blocks of K and V (64 tokens
// x 256 B each) once, and all G query heads of the group share them. The work
// of a row is split over workgroups by block ranges (split-K) so a decode batch
// fills all 256 CUs; a one-wave workgroup streams its blocks:
//   QK  - 16 lanes hold one key row (8 bf16 each), a wave reads 4 keys (1 KiB)
//         per load; G dot products per key via v_dot2_f32_bf16 and a DPP
//         butterfly; scores go to LDS as [key][G].
//   softmax - lane l takes key l: block max and sum per head by wave
//         reductions, running (max, sum) per head (online softmax).
//   PV  - the same lane layout over V; each lane accumulates G x 8 outputs for
//         its key row, reading p[key][0..G) from LDS as one broadcast.
// A combine kernel merges the per-split (max, sum, unnormalised output).
#include "common.h"
#include "launch.h"

namespace sparda {

constexpr int kAttnTargetWaves = 4096;  // aim: ~16 waves per CU over the grid

template <typename Tag, int G>
__global__ __launch_bounds__(64) void attn_decode_kernel(
    const uint8_t* __restrict__ q, const uint8_t* __restrict__ kbuf, const uint8_t* __restrict__ vbuf,
    const int32_t* __restrict__ idx, float* __restrict__ part_o, float2* __restrict__ part_ml,
    uint8_t* __restrict__ out, int T, int nB, int k, int kv_mode, int p, int bps, int splits,
    float scale) {
  constexpr int E = DT<Tag>::kElems;
  constexpr int LPK = kHeadDim / E;  // lanes per key row
  constexpr int KPI = kWave / LPK;   // keys per load instruction
  constexpr int NIT = kBlock / KPI;  // load instructions per block
  constexpr int RB = kHeadDim * DT<Tag>::kBytes;
  __shared__ float s_p[kBlock * G];

  const long row = blockIdx.y;
  const int split = blockIdx.x;
  const int lane = threadIdx.x;
  const int c = lane % LPK;
  const int r = lane / LPK;

  u32x4 qv[G];
#pragma unroll
  for (int g = 0; g < G; ++g) qv[g] = load16(q + (row * G + g) * RB + c * 16);

  float acc[G][E];
  float m_run[G], l_run[G];
#pragma unroll
  for (int g = 0; g < G; ++g) {
    m_run[g] = -INFINITY;
    l_run[g] = 0.f;
#pragma unroll
    for (int e = 0; e < E; ++e) acc[g][e] = 0.f;
  }

  const int j0 = split * bps;
  const int j1 = min(k, j0 + bps);
  for (int j = j0; j < j1; ++j) {
    const int beta = idx[row * k + j];
    if (beta < 0 || beta >= nB) continue;  // -1 padding; out-of-range ignored
    const int nvalid = min(kBlock, p - beta * kBlock + 1);
    if (nvalid <= 0) continue;
    const long tok0 = kv_mode == 0 ? row * (long)T + (long)beta * kBlock : (row * k + j) * (long)kBlock;
    const uint8_t* kb = kbuf + tok0 * RB + c * 16;
    const uint8_t* vb = vbuf + tok0 * RB + c * 16;

    u32x4 kv[NIT], vv[NIT];
#pragma unroll
    for (int it = 0; it < NIT; ++it) kv[it] = load16_nt(kb + (it * KPI + r) * RB);
#pragma unroll
    for (int it = 0; it < NIT; ++it) vv[it] = load16_nt(vb + (it * KPI + r) * RB);

    // scores -> LDS [key][g]
#pragma unroll
    for (int it = 0; it < NIT; ++it) {
      const int key = it * KPI + r;
#pragma unroll
      for (int g = 0; g < G; ++g) {
        const float s = group_sum<LPK>(dot16<Tag>(qv[g], kv[it], 0.f));
        if (c == g) s_p[key * G + g] = key < nvalid ? s * scale : -INFINITY;
      }
    }
    __syncthreads();
    // online softmax, lane = key
    float alpha[G];
#pragma unroll
    for (int g = 0; g < G; ++g) {
      const float s = s_p[lane * G + g];
      const float mb = wave_max(s);
      const float mn = fmaxf(m_run[g], mb);  // finite: key 0 of the block is always valid
      alpha[g] = fast_exp(m_run[g] - mn);    // exp(-inf) = 0 on the first block
      const float pr = fast_exp(s - mn);
      l_run[g] = l_run[g] * alpha[g] + wave_sum(pr);
      m_run[g] = mn;
      s_p[lane * G + g] = pr;
    }
    __syncthreads();
#pragma unroll
    for (int g = 0; g < G; ++g)
#pragma unroll
      for (int e = 0; e < E; ++e) acc[g][e] *= alpha[g];
#pragma unroll
    for (int it = 0; it < NIT; ++it) {
      const int key = it * KPI + r;
      float v[E];
      unpack<Tag>(vv[it], v);
      float pg[G];
#pragma unroll
      for (int g = 0; g < G; ++g) pg[g] = s_p[key * G + g];
#pragma unroll
      for (int g = 0; g < G; ++g)
#pragma unroll
        for (int e = 0; e < E; ++e) acc[g][e] = fmaf(pg[g], v[e], acc[g][e]);
    }
    __syncthreads();
  }

  // reduce the KPI key rows
#pragma unroll
  for (int g = 0; g < G; ++g)
#pragma unroll
    for (int e = 0; e < E; ++e) {
      float x = acc[g][e];
      for (int m = LPK; m < kWave; m <<= 1) x += xor_shfl(x, m);
      acc[g][e] = x;
    }
  if (r != 0) return;

  if (splits == 1) {
    // final: normalise and store in the storage dtype
#pragma unroll
    for (int g = 0; g < G; ++g) {
      const float inv = l_run[g] > 0.f ? 1.f / l_run[g] : 0.f;
      float o[E];
#pragma unroll
      for (int e = 0; e < E; ++e) o[e] = acc[g][e] * inv;
      store16(out + (row * G + g) * RB + c * 16, pack<Tag>(o));
    }
    return;
  }
  const long ps = row * splits + split;
#pragma unroll
  for (int g = 0; g < G; ++g) {
    float* po = part_o + ((ps * G + g) * kHeadDim) + c * E;
#pragma unroll
    for (int e = 0; e < E; e += 4)
      *reinterpret_cast<float4*>(po + e) = make_float4(acc[g][e], acc[g][e + 1], acc[g][e + 2], acc[g][e + 3]);
    if (c == 0) part_ml[ps * G + g] = make_float2(m_run[g], l_run[g]);
  }
}

// One workgroup per (row, head): thread = output channel.
template <typename Tag>
__global__ __launch_bounds__(kHeadDim) void attn_combine_kernel(const float* __restrict__ part_o,
                                                                const float2* __restrict__ part_ml,
                                                                uint8_t* __restrict__ out, int G,
                                                                int splits) {
  const long row = blockIdx.x;
  const int g = blockIdx.y;
  const int ch = threadIdx.x;
  float M = -INFINITY;
  for (int s = 0; s < splits; ++s) M = fmaxf(M, part_ml[(row * splits + s) * G + g].x);
  float L = 0.f, O = 0.f;
  if (M != -INFINITY) {
    for (int s = 0; s < splits; ++s) {
      const float2 ml = part_ml[(row * splits + s) * G + g];
      if (ml.x == -INFINITY) continue;
      const float w = fast_exp(ml.x - M);
      L += ml.y * w;
      O += part_o[(((row * splits + s) * G + g) * kHeadDim) + ch] * w;
    }
  }
  const float o = L > 0.f ? O / L : 0.f;
  const long off = (row * G + g) * kHeadDim + ch;
  if constexpr (DT<Tag>::kBytes == 2) {
    reinterpret_cast<__bf16*>(out)[off] = (__bf16)o;
  } else {
    reinterpret_cast<float*>(out)[off] = o;
  }
}

int decode_attn_splits(const AttnDims& d) {
  const long rows = (long)d.B * d.Hkv;
  long want = (kAttnTargetWaves + rows - 1) / rows;
  if (want < 1) want = 1;
  if (want > d.k) want = d.k;
  // equal block ranges
  const int bps = (int)((d.k + want - 1) / want);
  return (d.k + bps - 1) / bps;
}

static inline size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

size_t decode_attn_ws_bytes(const AttnDims& d) {
  const int splits = decode_attn_splits(d);
  if (splits == 1) return 0;
  const int G = d.Hq / d.Hkv;
  const size_t n = (size_t)d.B * d.Hkv * splits * G;
  return align256(n * kHeadDim * sizeof(float)) + align256(n * sizeof(float2));
}

template <typename Tag, int G>
static void launch_attn_g(const void* q, const void* k, const void* v, const int32_t* idx, void* out,
                          const AttnDims& d, void* ws, hipStream_t s) {
  const int splits = decode_attn_splits(d);
  const int bps = (d.k + splits - 1) / splits;
  const int rows = d.B * d.Hkv;
  float* part_o = nullptr;
  float2* part_ml = nullptr;
  if (splits > 1) {
    const size_t n = (size_t)rows * splits * G;
    part_o = (float*)ws;
    part_ml = (float2*)((char*)ws + align256(n * kHeadDim * sizeof(float)));
  }
  hipLaunchKernelGGL((attn_decode_kernel<Tag, G>), dim3(splits, rows), dim3(kWave), 0, s,
                     (const uint8_t*)q, (const uint8_t*)k, (const uint8_t*)v, idx, part_o, part_ml,
                     (uint8_t*)out, d.T, d.nB, d.k, d.kv_mode, d.q_start, bps, splits, d.scale);
  if (splits > 1)
    hipLaunchKernelGGL(attn_combine_kernel<Tag>, dim3(rows, G), dim3(kHeadDim), 0, s, part_o,
                       part_ml, (uint8_t*)out, G, splits);
}

hipError_t launch_attn_decode(const void* q, const void* k, const void* v, const int32_t* idx,
                              void* out, bool bf16, const AttnDims& d, void* ws, hipStream_t s) {
  const int G = d.Hq / d.Hkv;
#define SPARDA_AT(TAG, GG) launch_attn_g<TAG, GG>(q, k, v, idx, out, d, ws, s)
#define SPARDA_AT_G(TAG)                  \
  switch (G) {                            \
    case 1: SPARDA_AT(TAG, 1); break;     \
    case 2: SPARDA_AT(TAG, 2); break;     \
    case 4: SPARDA_AT(TAG, 4); break;     \
    case 8: SPARDA_AT(TAG, 8); break;     \
    default: return hipErrorInvalidValue; \
  }
  if (bf16) {
    SPARDA_AT_G(BF16Tag)
  } else {
    SPARDA_AT_G(F32Tag)
  }
#undef SPARDA_AT_G
#undef SPARDA_AT
  return hipGetLastError();
}

}  // namespace sparda
