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

constexpr int kAttnTargetWaves = 2048;  // 8 resident waves per CU at ~200 VGPRs
constexpr int kAttnMaxSplits = 64;

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
  constexpr int GR = G < 4 ? 1 : G / 4;  // scores each lane holds after the reduce-scatter
  __shared__ float s_p[kBlock * G];

  const long row = blockIdx.y;
  const int split = blockIdx.x;
  const int lane = threadIdx.x;
  const int c = lane % LPK;
  const int r = lane / LPK;

  u32x4 qs[G];
#pragma unroll
  for (int s = 0; s < G; ++s) qs[s] = load16(q + (row * G + slot_head<G>(s, c & 15)) * RB + c * 16);

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
  const int32_t* idx_row = idx + row * k;
  auto next_valid = [&](int j) {
    for (; j < j1; ++j) {
      const int b = idx_row[j];
      if (b >= 0 && b < nB && b * kBlock <= p) break;  // -1 padding / out of range / future block
    }
    return j;
  };
  auto tok0_of = [&](int j, int beta) -> long {
    return kv_mode == 0 ? row * (long)T + (long)beta * kBlock : (row * k + j) * (long)kBlock;
  };

  u32x4 kv[NIT], vv[NIT];
  int j = next_valid(j0);
  if (j < j1) {
    const uint8_t* kb = kbuf + tok0_of(j, idx_row[j]) * RB + c * 16;
#pragma unroll
    for (int it = 0; it < NIT; ++it) kv[it] = load16_nt(kb + (it * KPI + r) * RB);
  }
  while (j < j1) {
    const int beta = idx_row[j];
    const int nvalid = min(kBlock, p - beta * kBlock + 1);
    const uint8_t* vb = vbuf + tok0_of(j, beta) * RB + c * 16;
#pragma unroll
    for (int it = 0; it < NIT; ++it) vv[it] = load16_nt(vb + (it * KPI + r) * RB);

    // QK: scores -> LDS [key][g]
#pragma unroll
    for (int it = 0; it < NIT; ++it) {
      const int key = it * KPI + r;
      float part[G];
#pragma unroll
      for (int s = 0; s < G; ++s) part[s] = dot16<Tag>(qs[s], kv[it], 0.f);
      if constexpr (LPK == 32) {  // fp32: 32 lanes per key; fold the upper 16 first
#pragma unroll
        for (int s = 0; s < G; ++s) part[s] += xor_shfl(part[s], 16);
      }
      float sc[GR];
      reduce_scatter16<G>(part, sc);
      constexpr int HL = G >= 4 ? 4 : (G == 2 ? 8 : 16);  // lanes per head after the scatter
      if ((c & (HL - 1)) == 0 && c < 16) {
        const int h = (c & 15) / HL;
#pragma unroll
        for (int gr = 0; gr < GR; ++gr)
          s_p[key * G + 4 * gr + h] = key < nvalid ? sc[gr] * scale : -INFINITY;
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
    // prefetch the next block's keys while the values are consumed
    const int jn = next_valid(j + 1);
    if (jn < j1) {
      const uint8_t* kb = kbuf + tok0_of(jn, idx_row[jn]) * RB + c * 16;
#pragma unroll
      for (int it = 0; it < NIT; ++it) kv[it] = load16_nt(kb + (it * KPI + r) * RB);
    }
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
    j = jn;
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

// One 256-thread workgroup per row merges the row's splits for all G heads:
// weights exp(m_s - M) / L per (split, head) go to LDS first, then every
// output channel sums its splits with independent loads.
template <typename Tag>
__global__ __launch_bounds__(256) void attn_combine_kernel(const float* __restrict__ part_o,
                                                           const float2* __restrict__ part_ml,
                                                           uint8_t* __restrict__ out, int G,
                                                           int splits) {
  __shared__ float2 s_ml[kAttnMaxSplits * 8];
  __shared__ float s_w[kAttnMaxSplits * 8];
  __shared__ float s_M[8], s_iL[8];
  const long row = blockIdx.x;
  const int t = threadIdx.x;
  const int n = splits * G;
  for (int i = t; i < n; i += 256) s_ml[i] = part_ml[row * n + i];
  __syncthreads();
  if (t < G) {
    float M = -INFINITY;
    for (int s = 0; s < splits; ++s) M = fmaxf(M, s_ml[s * G + t].x);
    float L = 0.f;
    if (M != -INFINITY)
      for (int s = 0; s < splits; ++s) {
        const float2 ml = s_ml[s * G + t];
        if (ml.x != -INFINITY) L += ml.y * fast_exp(ml.x - M);
      }
    s_M[t] = M;
    s_iL[t] = L > 0.f ? 1.f / L : 0.f;
  }
  __syncthreads();
  for (int i = t; i < n; i += 256) {
    const float2 ml = s_ml[i];
    const int g = i % G;
    s_w[i] = ml.x == -INFINITY ? 0.f : fast_exp(ml.x - s_M[g]) * s_iL[g];
  }
  __syncthreads();
  for (int o = t; o < G * kHeadDim; o += 256) {
    const int g = o / kHeadDim;
    const float* src = part_o + (row * splits * G + g) * kHeadDim + (o % kHeadDim);
    float acc = 0.f;
    int s = 0;
    for (; s + 8 <= splits; s += 8) {
      float x[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) x[u] = src[(long)(s + u) * G * kHeadDim];
#pragma unroll
      for (int u = 0; u < 8; ++u) acc = fmaf(x[u], s_w[(s + u) * G + g], acc);
    }
    for (; s < splits; ++s) acc = fmaf(src[(long)s * G * kHeadDim], s_w[s * G + g], acc);
    const long off = row * G * kHeadDim + o;
    if constexpr (DT<Tag>::kBytes == 2) {
      reinterpret_cast<__bf16*>(out)[off] = (__bf16)acc;
    } else {
      reinterpret_cast<float*>(out)[off] = acc;
    }
  }
}

int decode_attn_splits(const AttnDims& d) {
  const long rows = (long)d.B * d.Hkv;
  long want = (kAttnTargetWaves + rows - 1) / rows;
  if (want < 1) want = 1;
  if (want > d.k) want = d.k;
  if (want > kAttnMaxSplits) want = kAttnMaxSplits;
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
    hipLaunchKernelGGL(attn_combine_kernel<Tag>, dim3(rows), dim3(256), 0, s, part_o, part_ml,
                       (uint8_t*)out, G, splits);
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
