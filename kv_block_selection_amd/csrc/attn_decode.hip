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
//   softmax - lane l takes key l. The running max of a head moves only when
//         a score exceeds it by more than 8 ln 2 (a ballot, wave-uniform), so
//         probabilities stay <= 2^8 and most stages need neither a wave max
//         nor a rescale; each lane keeps its own running sum, reduced over
//         the wave once at the end.
//   PV  - the same lane layout over V; each lane accumulates G x 8 outputs for
//         its key row, reading p[key][0..G) from LDS as one broadcast.
// Each split leaves its (max, sum, unnormalised output); a merge kernel
// (merge_row.h) combines a row's splits. Two more forms of the same kernel:
// four splits per workgroup with the row's top-k taken first by the whole
// workgroup (topk_row.h; the selection then comes from LDS), and the merge
// left to a later launch, such as the next layer's selection. A token mode
// (template flag TOK) reads a list of single tokens instead of blocks, for the
// token-level Forecast variant (techwalker.com article, section 六): each
// lane loads the indices of its stage's keys a stage ahead of their rows.
#include <mutex>
#include <type_traits>

#include "common.h"
#include "launch.h"
#include "merge_row.h"
#include "reduce16.h"
#include "select_row.h"
#include "topk_row.h"

namespace sparda {

#ifndef SPARDA_ATTN_TARGET_WAVES
#define SPARDA_ATTN_TARGET_WAVES 2048
#endif
// Split a decode batch's rows into block ranges until the grid holds about this
// many one-wave workgroups (8 resident per CU at ~250 VGPRs).
constexpr int kAttnTargetWaves = SPARDA_ATTN_TARGET_WAVES;
constexpr int kAttnMaxSplits = 64;
constexpr int kFusedMaxK = 1024;  // top-k fused in front of attention: at most this many blocks
constexpr int SPARDA_KV_CACHE_MODE = 0;  // kv_mode of a cache read at the selected blocks
constexpr float kLazyGrow = 5.545177444479562f;  // 8 ln 2

#ifndef SPARDA_ATTN_WAVES_PER_EU
#define SPARDA_ATTN_WAVES_PER_EU 2
#endif

// WPG waves per workgroup, one split each (split = blockIdx.y * WPG + wave).
// NPT > 0: the workgroup first takes the row's top-k of `scores` itself (all
// WPG x 64 threads, NPT scores per thread; every workgroup of the row computes
// the same selection, the first also writes it to idx_out) and the waves read
// the selection from LDS; NPT = 0: the selection comes from idx.
// LDSM: the workgroup holds all of the row's splits (one per wave; waves past
// the last split contribute nothing) and merges them in LDS, with the merge
// kernel's arithmetic, into the finished output: no partials, no second launch.
template <typename Tag, int G, int WPG, int NPT, bool LDSM = false, bool TOK = false>
__device__ __forceinline__ void attn_decode_body(
    long row, int wg_split, const uint8_t* __restrict__ q, const uint8_t* __restrict__ kbuf,
    const uint8_t* __restrict__ vbuf, const int32_t* __restrict__ idx, int32_t* __restrict__ idx_out,
    const float* __restrict__ scores, float* __restrict__ part_o, float2* __restrict__ part_ml,
    uint8_t* __restrict__ out, int T, int nB, int k, int kv_mode, int p_all, const int* __restrict__ q_pos, int hkv,
    const int32_t* __restrict__ slot_of, int n_slots, int bps, int splits, float scale) {
  constexpr int E = DT<Tag>::kElems;
  constexpr int LPK = kHeadDim / E;  // lanes per key row
  constexpr int KPI = kWave / LPK;   // keys per load instruction
  constexpr int CK = 32;             // keys per pipeline stage (half a block)
  constexpr int NIT = CK / KPI;      // load instructions per stage
  constexpr int RB = kHeadDim * DT<Tag>::kBytes;
  constexpr int GR = G < 4 ? 1 : G / 4;  // scores each lane holds after the reduce-scatter
  constexpr bool kBf16 = DT<Tag>::kBytes == 2;
  __shared__ float s_p_all[WPG][CK * G];          // scores (and fp32 probabilities), per wave
  __shared__ uint32_t s_p2_all[WPG][CK / 2 * G];  // bf16 probability pairs, per wave
  const int wv = WPG == 1 ? 0 : threadIdx.x / kWave;
  float* s_p = s_p_all[wv];
  uint32_t* s_p2 = s_p2_all[wv];

  const int split = wg_split * WPG + wv;
  const int p = row_position(q_pos, row, hkv, p_all, T);  // the row's query position
  const int lane = WPG == 1 ? threadIdx.x : threadIdx.x % kWave;
  const int c = lane % LPK;
  const int r = lane / LPK;

  // TOK: idx holds k * 64 token indices per row (slot j = entries 64 j ..
  // 64 j + 63) instead of k block indices
  const int32_t* idx_row = idx + row * (long)k * (TOK ? kBlock : 1);
  if constexpr (NPT > 0) {
    __shared__ TopkShared<WPG> sh;
    __shared__ int32_t s_sel[kFusedMaxK];
    topk_row<NPT, WPG>(scores + row * nB, wg_split == 0 ? idx_out + row * k : nullptr, s_sel, nB, k, sh,
                       threadIdx.x);
    lds_sync();  // the selection is in LDS
    idx_row = s_sel;
  }
  // a wave past the row's last split: none of the work below (with LDSM it
  // still takes part in the merge, with nothing to add)
  const bool active = split < splits;
  if constexpr (!LDSM) {
    if (!active) return;
  }
  u32x4 qs[G];
#pragma unroll
  for (int s = 0; s < G; ++s) qs[s] = load16(q + (row * G + slot_head<G>(s, c & 15)) * RB + c * 16);
  // Hand-offs through s_p / s_p2 stay inside one wave: with one wave per
  // workgroup a barrier is that wave's own; otherwise waiting for the wave's
  // LDS operations is enough (its lanes run each LDS instruction together, in
  // order), and the other waves of the workgroup run their splits freely.
  auto stage_sync = [&]() {
    if constexpr (WPG == 1) {
      __syncthreads();
    } else {
      asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    }
  };

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
  const int j1 = min(k, j0 + bps);  // >= j0 + 1 for an active split: it owns at least one slot
  // Stage q = half h of slot j0 + q/2: its first token and its number of valid
  // keys. Padding, out-of-range and wholly-future slots read block 0 of the
  // row (a valid address) with every key masked.
  auto stage_of = [&](int q, int& nvalid) -> long {
    const int j = j0 + (q >> 1);
    const int h = q & 1;
    const int b = idx_row[j];
    // kv_mode 2 (staging used as a block cache): the block sits in slot slot_of
    const int sl = kv_mode == 2 ? slot_of[row * k + j] : 0;
    const bool ok = b >= 0 && b < nB && b * kBlock <= p && (kv_mode != 2 || (sl >= 0 && sl < n_slots));
    nvalid = ok ? max(0, min(CK, p - b * kBlock - h * CK + 1)) : 0;
    const long base = kv_mode == 1   ? (row * k + j) * (long)kBlock
                      : kv_mode == 2 ? (row * (long)n_slots + (ok ? sl : 0)) * kBlock
                                     : row * (long)T + (long)(ok ? b : 0) * kBlock;
    return base + h * CK;
  };
  const int nstage = 2 * (j1 - j0);

  // TOK: each stage's keys are the tokens its 32 list entries name; a lane
  // loads the indices of its keys (it KPI + r) a stage ahead of their rows.
  // An entry that is -1 or after the query position reads token 0 (a valid
  // address) and is masked.
  const long tok_row = row * (long)T;
  int tk_cur[TOK ? NIT : 1], tk_nxt[TOK ? NIT : 1];
  uint32_t vm_cur = 0, vm_nxt = 0;  // bit it: key it KPI + r is a valid token
  auto load_tok = [&](int q, int (&tk)[TOK ? NIT : 1], uint32_t& vm) {
    const int e0 = (j0 + (q >> 1)) * kBlock + (q & 1) * CK;
    vm = 0;
#pragma unroll
    for (int it = 0; it < NIT; ++it) {
      const int t = idx_row[e0 + it * KPI + r];
      const bool ok = t >= 0 && t <= p;
      tk[it] = ok ? t : 0;
      vm |= (uint32_t)ok << it;
    }
  };
  auto key_row = [&](long base, int it, const int (&tk)[TOK ? NIT : 1]) -> long {
    if constexpr (TOK) {
      return tok_row + tk[it];
    } else {
      return base + it * KPI + r;
    }
  };

  u32x4 kv[NIT], vv[NIT];
  int nvalid = 0;
  long tok0 = 0;
  if (active) {  // an inactive wave reads no stage
    if constexpr (TOK) {
      load_tok(0, tk_cur, vm_cur);
    } else {
      tok0 = stage_of(0, nvalid);
    }
#pragma unroll
    for (int it = 0; it < NIT; ++it) kv[it] = load16_nt(kbuf + key_row(tok0, it, tk_cur) * RB + c * 16);
  }

  // One stage of 32 keys: V loads go out first, then QK on the keys already in
  // flight, the online softmax, the next stage's key loads (PREFETCH), then PV.
  // The last stage is peeled so that every load in the steady-state body is
  // unconditional and the compiler's wait counts stay exact.
  auto body = [&](int q, auto prefetch) {
#pragma unroll
    for (int it = 0; it < NIT; ++it) vv[it] = load16_nt(vbuf + key_row(tok0, it, tk_cur) * RB + c * 16);
    if constexpr (TOK && decltype(prefetch)::value) load_tok(q + 1, tk_nxt, vm_nxt);

    // QK: scores -> LDS [key][g]
#pragma unroll
    for (int it = 0; it < NIT; ++it) {
      const int key = it * KPI + r;
      float part[G];
#pragma unroll
      for (int s = 0; s < G; ++s) part[s] = dot16<Tag>(qs[s], kv[it], 0.f);
      if constexpr (LPK == 32) {  // fp32: 32 lanes per key; fold the upper 16 first
#pragma unroll
        for (int s = 0; s < G; ++s) part[s] = sum16(part[s]);
      }
      float sc[GR];
      reduce_scatter16<G>(part, sc);
      constexpr int HL = G >= 4 ? 4 : (G == 2 ? 8 : 16);  // lanes per head after the scatter
      if ((c & (HL - 1)) == 0 && c < 16) {
        const int h = (c & 15) / HL;
        const bool valid = TOK ? ((vm_cur >> it) & 1u) != 0 : key < nvalid;
#pragma unroll
        for (int gr = 0; gr < GR; ++gr)
          s_p[key * G + 4 * gr + h] = valid ? sc[gr] * scale : -INFINITY;
      }
    }
    stage_sync();
    // online softmax, lane = key (lanes 32..63 idle)
    float alpha[G], pr[G];
#pragma unroll
    for (int g = 0; g < G; ++g) {
      const float s = lane < CK ? s_p[lane * G + g] : -INFINITY;
      alpha[g] = 1.f;
      if (__ballot(s > m_run[g] + kLazyGrow) != 0) {  // -inf + c stays -inf: the first finite score moves it
        const float mn = fmaxf(m_run[g], wave_max(s));
        alpha[g] = fast_exp(m_run[g] - mn);  // 0 while no valid key was seen
        l_run[g] *= alpha[g];
        m_run[g] = mn;
      }
      pr[g] = m_run[g] == -INFINITY ? 0.f : fast_exp(s - m_run[g]);
      l_run[g] += pr[g];  // this lane's keys only
    }
    if constexpr (kBf16) {
      // bf16 pairs (p[key], p[key + 4]) for the keys with key % 8 < 4; the
      // partner sits 4 lanes up in the same DPP row (row_ror:12)
      float up[G];
#pragma unroll
      for (int g = 0; g < G; ++g) up[g] = dpp<0x12C>(pr[g]);
      if ((lane & 4) == 0 && lane < CK) {
        const int slot = (lane >> 3) * 4 + (lane & 3);
#pragma unroll
        for (int g = 0; g < G; ++g) s_p2[slot * G + g] = pack_bf16(pr[g], up[g]);
      }
    } else {
      if (lane < CK) {
#pragma unroll
        for (int g = 0; g < G; ++g) s_p[lane * G + g] = pr[g];
      }
    }
    stage_sync();
    if constexpr (decltype(prefetch)::value) {
      if constexpr (TOK) {
#pragma unroll
        for (int it = 0; it < NIT; ++it) tk_cur[it] = tk_nxt[it];
        vm_cur = vm_nxt;
      } else {
        tok0 = stage_of(q + 1, nvalid);
      }
#pragma unroll
      for (int it = 0; it < NIT; ++it) kv[it] = load16_nt(kbuf + key_row(tok0, it, tk_cur) * RB + c * 16);
    }
#pragma unroll
    for (int g = 0; g < G; ++g) {
      if (alpha[g] != 1.f) {  // wave-uniform
#pragma unroll
        for (int e = 0; e < E; ++e) acc[g][e] *= alpha[g];
      }
    }
    if constexpr (kBf16) {
      // PV on packed pairs: keys 8jp + r and 8jp + 4 + r come from loads 2jp
      // and 2jp + 1; v_perm_b32 interleaves their channels, v_dot2 applies the
      // pair of probabilities
#pragma unroll
      for (int jp = 0; jp < NIT / 2; ++jp) {
        uint32_t pp[G];
#pragma unroll
        for (int g = 0; g < G; ++g) pp[g] = s_p2[(jp * 4 + r) * G + g];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const uint32_t a = vv[2 * jp][i], b = vv[2 * jp + 1][i];
          const uint32_t lo = __builtin_amdgcn_perm(b, a, 0x05040100u);  // channel 2i of both keys
          const uint32_t hi = __builtin_amdgcn_perm(b, a, 0x07060302u);  // channel 2i + 1
#pragma unroll
          for (int g = 0; g < G; ++g) {
            const bf16x2 pg = __builtin_bit_cast(bf16x2, pp[g]);
            acc[g][2 * i] = __builtin_amdgcn_fdot2_f32_bf16(pg, __builtin_bit_cast(bf16x2, lo), acc[g][2 * i], false);
            acc[g][2 * i + 1] =
                __builtin_amdgcn_fdot2_f32_bf16(pg, __builtin_bit_cast(bf16x2, hi), acc[g][2 * i + 1], false);
          }
        }
      }
    } else {
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
    }
    stage_sync();
  };
  if (active) {
    for (int q = 0; q < nstage - 1; ++q) body(q, std::true_type{});
    body(nstage - 1, std::false_type{});
  }

#pragma unroll
  for (int g = 0; g < G; ++g) l_run[g] = wave_sum(l_run[g]);
  // reduce the KPI key rows
#pragma unroll
  for (int g = 0; g < G; ++g)
#pragma unroll
    for (int e = 0; e < E; ++e) {
      float x = acc[g][e];
      if constexpr (LPK == 16) x = sum16(x);
      acc[g][e] = sum32(x);
    }

  if constexpr (LDSM) {
    // each wave's (max, sum, unnormalised output) per head into LDS, then the
    // merge of merge_row.h over the waves in order: thread t < 32 G takes head
    // t / 32, channels 4 (t % 32) .. + 3
    __shared__ float s_mo[WPG][G][kHeadDim];
    __shared__ float2 s_ml[WPG][G];
    if (r == 0) {
#pragma unroll
      for (int g = 0; g < G; ++g) {
#pragma unroll
        for (int e = 0; e < E; e += 4)
          *reinterpret_cast<float4*>(&s_mo[wv][g][c * E + e]) =
              make_float4(acc[g][e], acc[g][e + 1], acc[g][e + 2], acc[g][e + 3]);
        if (c == 0) s_ml[wv][g] = make_float2(m_run[g], l_run[g]);
      }
    }
    __syncthreads();
    const int t = threadIdx.x;
    if (t < G * (kHeadDim / 4)) {
      const int g = t / (kHeadDim / 4);
      const int ch = (t % (kHeadDim / 4)) * 4;
      float M = -INFINITY;
#pragma unroll
      for (int w = 0; w < WPG; ++w) M = fmaxf(M, s_ml[w][g].x);
      float L = 0.f, O[4] = {0.f, 0.f, 0.f, 0.f};
      if (M != -INFINITY) {
#pragma unroll
        for (int w = 0; w < WPG; ++w) {
          const float2 ml = s_ml[w][g];
          if (ml.x != -INFINITY) {
            const float4 po = *reinterpret_cast<const float4*>(&s_mo[w][g][ch]);
            const float wt = fast_exp(ml.x - M);
            L = fmaf(ml.y, wt, L);
            O[0] = fmaf(po.x, wt, O[0]);
            O[1] = fmaf(po.y, wt, O[1]);
            O[2] = fmaf(po.z, wt, O[2]);
            O[3] = fmaf(po.w, wt, O[3]);
          }
        }
      }
      float o[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) o[e] = L > 0.f ? O[e] / L : 0.f;
      const long off = (row * G + g) * kHeadDim + ch;
      if constexpr (kBf16) {
        uint2 v;
        v.x = pack_bf16(o[0], o[1]);
        v.y = pack_bf16(o[2], o[3]);
        *reinterpret_cast<uint2*>(out + off * 2) = v;
      } else {
        *reinterpret_cast<float4*>(out + off * 4) = make_float4(o[0], o[1], o[2], o[3]);
      }
    }
    return;
  }

  if (splits == 1) {
    // final: normalise and store in the storage dtype
    if (r == 0) {
#pragma unroll
      for (int g = 0; g < G; ++g) {
        const float inv = l_run[g] > 0.f ? 1.f / l_run[g] : 0.f;
        float o[E];
#pragma unroll
        for (int e = 0; e < E; ++e) o[e] = acc[g][e] * inv;
        store16(out + (row * G + g) * RB + c * 16, pack<Tag>(o));
      }
    }
    return;
  }
  const long ps = row * splits + split;
  if (r == 0) {
#pragma unroll
    for (int g = 0; g < G; ++g) {
      float* po = part_o + ((ps * G + g) * kHeadDim) + c * E;
#pragma unroll
      for (int e = 0; e < E; e += 4)
        *reinterpret_cast<float4*>(po + e) = make_float4(acc[g][e], acc[g][e + 1], acc[g][e + 2], acc[g][e + 3]);
      if (c == 0) part_ml[ps * G + g] = make_float2(m_run[g], l_run[g]);
    }
  }
}

// fp32 rows hold twice the bytes in flight: one wave per SIMD, so the
// registers past 256 spill to AGPRs instead of scratch memory
template <typename Tag, int G, int WPG, int NPT, bool TOK = false>
__global__ __launch_bounds__(64 * WPG)
__attribute__((amdgpu_waves_per_eu(DT<Tag>::kBytes == 2 ? SPARDA_ATTN_WAVES_PER_EU : 1)))
void attn_decode_kernel(
    const uint8_t* __restrict__ q, const uint8_t* __restrict__ kbuf, const uint8_t* __restrict__ vbuf,
    const int32_t* __restrict__ idx, int32_t* __restrict__ idx_out, const float* __restrict__ scores,
    float* __restrict__ part_o, float2* __restrict__ part_ml, uint8_t* __restrict__ out, int T, int nB, int k,
    int kv_mode, int p_all, const int* __restrict__ q_pos, int hkv, const int32_t* __restrict__ slot_of, int n_slots,
    int bps, int splits, float scale) {
  // rows on the fast axis: a row's splits share an XCD
  attn_decode_body<Tag, G, WPG, NPT, false, TOK>(blockIdx.x, blockIdx.y, q, kbuf, vbuf, idx, idx_out, scores, part_o,
                                                 part_ml, out, T, nB, k, kv_mode, p_all, q_pos, hkv, slot_of, n_slots,
                                                 bps, splits, scale);
}

// One decode layer in one launch, in an order a model can run: layer l's
// hidden state gives both its queries and the Forecast that scores layer
// l+1's compressed keys, so this layer's top-k + attention and the next
// layer's Forecast selection need the same inputs and nothing from each other
// (bittide.aicompass.dev summary post, paragraph on layer L's Forecast
// choosing layer L+1's blocks). Their workgroups share one 1D grid, and the
// layer's output is complete when the launch ends: the next layer's work
// needs it, through the output projection and the MLP.
//
// Row form (enough rows to fill half the chip): the attention comes first,
// one 8-wave workgroup per (sequence, KV head) row that takes the row's top-k
// with all 512 threads, gives each wave an equal block range and merges the
// eight ranges in LDS; the selection workgroups follow and stream the next
// layer's compressed keys on the CUs the attention leaves free, and on the
// attention's CUs as they finish. Split form (few rows): selection first,
// then 4-wave attention workgroups over shorter block ranges whose results
// go to the workspace; the merge is a second, small launch.
// Both run at the attention's register allocation (2 waves per SIMD), so a
// selection workgroup takes 128 blocks (513 windows) instead of 16.
#ifndef SPARDA_LAYER_SEL_BLOCKS
#define SPARDA_LAYER_SEL_BLOCKS 128
#endif
constexpr int kLayerSelBlocks = SPARDA_LAYER_SEL_BLOCKS;
constexpr int kLayerRowWaves = 8;     // waves of a row-form attention workgroup
constexpr int kLayerRowMinRows = 96;  // fewest rows for the row form

template <typename Tag, int G, int NPT>
__global__ __launch_bounds__(kLayerRowWaves * 64) __attribute__((amdgpu_waves_per_eu(SPARDA_ATTN_WAVES_PER_EU)))
void decode_layer_row_kernel(int rows,
                             // top-k + attention of layer l, one workgroup per row
                             const uint8_t* __restrict__ q, const uint8_t* __restrict__ kbuf,
                             const uint8_t* __restrict__ vbuf, int32_t* __restrict__ idx_out,
                             const float* __restrict__ scores, uint8_t* __restrict__ out, int T, int nB, int k,
                             int p_all, const int* __restrict__ q_pos, int hkv, int bps, int splits, float scale,
                             // selection of layer l+1
                             const uint8_t* __restrict__ f_n, const uint8_t* __restrict__ kc_n,
                             float* __restrict__ scores_n, int W_n, int nB_n, int n_vis_n,
                             const int* __restrict__ q_pos_n, int T_n, float scale_n) {
  constexpr int NT = kLayerRowWaves * 64;
  if ((int)blockIdx.x < rows) {
    attn_decode_body<Tag, G, kLayerRowWaves, NPT, true>(blockIdx.x, 0, q, kbuf, vbuf, nullptr, idx_out, scores,
                                                        nullptr, nullptr, out, T, nB, k, SPARDA_KV_CACHE_MODE, p_all,
                                                        q_pos, hkv, nullptr, 0, bps, splits, scale);
  } else {
    const int r = blockIdx.x - rows;
    __shared__ float s_win[fsel_lds_floats<Tag, kLayerSelBlocks, NT>()];
    fsel_blocks<Tag, kLayerSelBlocks, NT>(f_n, kc_n, scores_n, W_n, nB_n, n_vis_n, q_pos_n, hkv, T_n, scale_n,
                                          r % rows, r / rows, s_win, threadIdx.x);
  }
}

template <typename Tag, int G, int NPT>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(SPARDA_ATTN_WAVES_PER_EU)))
void decode_layer_kernel(int n_sel, int rows,
                         // top-k + attention of layer l, block ranges of 4 splits per workgroup
                         const uint8_t* __restrict__ q, const uint8_t* __restrict__ kbuf,
                         const uint8_t* __restrict__ vbuf, int32_t* __restrict__ idx_out,
                         const float* __restrict__ scores, float* __restrict__ part_o, float2* __restrict__ part_ml,
                         uint8_t* __restrict__ out, int T, int nB, int k, int p_all, const int* __restrict__ q_pos,
                         int hkv, int bps, int splits, float scale,
                         // selection of layer l+1
                         const uint8_t* __restrict__ f_n, const uint8_t* __restrict__ kc_n, float* __restrict__ scores_n,
                         int W_n, int nB_n, int n_vis_n, const int* __restrict__ q_pos_n, int T_n, float scale_n) {
  if ((int)blockIdx.x >= n_sel) {
    const int r = blockIdx.x - n_sel;
    attn_decode_body<Tag, G, 4, NPT>(r % rows, r / rows, q, kbuf, vbuf, nullptr, idx_out, scores, part_o, part_ml, out,
                                     T, nB, k, SPARDA_KV_CACHE_MODE, p_all, q_pos, hkv, nullptr, 0, bps, splits, scale);
  } else {
    const int r = blockIdx.x;
    __shared__ float s_win[fsel_lds_floats<Tag, kLayerSelBlocks>()];
    fsel_blocks<Tag, kLayerSelBlocks>(f_n, kc_n, scores_n, W_n, nB_n, n_vis_n, q_pos_n, hkv, T_n, scale_n, r % rows,
                                      r / rows, s_win, threadIdx.x);
  }
}

template <typename Tag, int MAXS>
__global__ __launch_bounds__(256) void attn_combine_row_kernel(const float* __restrict__ part_o,
                                                               const float2* __restrict__ part_ml,
                                                               uint8_t* __restrict__ out, int G, int splits) {
  merge_row<Tag, MAXS>(blockIdx.x, threadIdx.x, part_o, part_ml, out, G, splits);
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

// Workspace: [partial outputs][partial (max, sum)], 256-byte aligned.
size_t decode_attn_ws_bytes(const AttnDims& d) {
  const int splits = decode_attn_splits(d);
  if (splits == 1) return 0;
  const int G = d.Hq / d.Hkv;
  const size_t n = (size_t)d.B * d.Hkv * splits * G;
  return align256(n * kHeadDim * sizeof(float)) + align256(n * sizeof(float2));
}

DecodePartials decode_attn_partials(void* ws, const AttnDims& d) {
  DecodePartials p{nullptr, nullptr, decode_attn_splits(d), d.Hq / d.Hkv, d.B * d.Hkv};
  if (p.splits > 1) {
    const size_t n = (size_t)p.rows * p.splits * p.G;
    p.part_o = (float*)ws;
    p.part_ml = (float2*)((char*)ws + align256(n * kHeadDim * sizeof(float)));
  }
  return p;
}

template <typename Tag>
static void launch_merge(const DecodePartials& p, void* out, hipStream_t s) {
  if (p.splits <= 1) return;  // one range per row: the attention wrote the output itself
  if (p.splits <= 16)
    hipLaunchKernelGGL((attn_combine_row_kernel<Tag, 16>), dim3(p.rows), dim3(p.G * (kHeadDim / 4)), 0, s, p.part_o,
                       p.part_ml, (uint8_t*)out, p.G, p.splits);
  else
    hipLaunchKernelGGL((attn_combine_row_kernel<Tag, kAttnMaxSplits>), dim3(p.rows), dim3(p.G * (kHeadDim / 4)), 0,
                       s, p.part_o, p.part_ml, (uint8_t*)out, p.G, p.splits);
}

hipError_t launch_merge_partials(void* ws, void* out, bool bf16, const AttnDims& d, hipStream_t s) {
  const DecodePartials p = decode_attn_partials(ws, d);
  if (bf16)
    launch_merge<BF16Tag>(p, out, s);
  else
    launch_merge<F32Tag>(p, out, s);
  return hipGetLastError();
}

template <typename Tag, int G>
static void launch_attn_g(const void* q, const void* k, const void* v, const int32_t* idx, const float* scores,
                          void* out, const AttnDims& d, void* ws, bool merge, hipStream_t s) {
  const DecodePartials pp = decode_attn_partials(ws, d);
  const int splits = pp.splits;
  const int bps = (d.k + splits - 1) / splits;
  const int rows = pp.rows;
  float* part_o = pp.part_o;
  float2* part_ml = pp.part_ml;
  if (scores == nullptr) {
    hipLaunchKernelGGL((attn_decode_kernel<Tag, G, 1, 0>), dim3(rows, splits), dim3(kWave), 0, s,
                       (const uint8_t*)q, (const uint8_t*)k, (const uint8_t*)v, idx, nullptr, nullptr, part_o, part_ml, (uint8_t*)out, d.T, d.nB, d.k, d.kv_mode, d.q_start, d.q_pos, d.q_pos_per_row ? 1 : d.Hkv,
                       d.slot_of, d.n_slots, bps, splits, d.scale);
  } else {
    // top-k fused in front: four splits per workgroup, each workgroup of a
    // row selects the row's blocks itself
    const dim3 grid(rows, (splits + 3) / 4);
#define SPARDA_FUSED(N)                                                                                          \
  hipLaunchKernelGGL((attn_decode_kernel<Tag, G, 4, N>), grid, dim3(4 * kWave), 0, s, (const uint8_t*)q,         \
                     (const uint8_t*)k, (const uint8_t*)v, nullptr, const_cast<int32_t*>(idx), scores, part_o,    \
                     part_ml,                                                                                    \
                     (uint8_t*)out, d.T, d.nB, d.k, d.kv_mode, d.q_start, d.q_pos, d.q_pos_per_row ? 1 : d.Hkv, d.slot_of, d.n_slots, bps, \
                     splits, d.scale)
    if (d.nB <= 256) SPARDA_FUSED(1);
    else if (d.nB <= 2048) SPARDA_FUSED(8);
    else SPARDA_FUSED(32);
#undef SPARDA_FUSED
  }
  if (merge) launch_merge<Tag>(pp, out, s);
}

bool decode_layer_row_form(const AttnDims& d) { return (long)d.B * d.Hkv >= kLayerRowMinRows; }

template <typename Tag, int G>
static void launch_layer_g(const LayerLaunch& L, hipStream_t s) {
  const AttnDims& d = L.attn;
  const int rows = d.B * d.Hkv;
  const int n_sel_chunks = L.f_next ? (L.sel.nB + kLayerSelBlocks - 1) / kLayerSelBlocks : 0;
  const int n_vis_n = L.f_next ? min(L.sel.W, (L.sel.q_start - kKernel + 1) >= 0
                                                  ? (L.sel.q_start - kKernel + 1) / kStride + 1 : 0)
                               : 0;
  if (decode_layer_row_form(d)) {
    // one workgroup per row: eight equal block ranges, merged in LDS
    const int bps = (d.k + kLayerRowWaves - 1) / kLayerRowWaves;
    const int splits = (d.k + bps - 1) / bps;
    const dim3 grid(rows + rows * n_sel_chunks);
#define SPARDA_ROWL(N)                                                                                            \
  hipLaunchKernelGGL((decode_layer_row_kernel<Tag, G, N>), grid, dim3(kLayerRowWaves * 64), 0, s, rows,          \
                     (const uint8_t*)L.q, (const uint8_t*)L.k, (const uint8_t*)L.v, L.idx, L.scores,               \
                     (uint8_t*)L.out, d.T, d.nB, d.k, d.q_start, d.q_pos, d.Hkv, bps, splits, d.scale,             \
                     (const uint8_t*)L.f_next, (const uint8_t*)L.kc_next, L.scores_next, L.sel.W, L.sel.nB,         \
                     n_vis_n, L.sel.q_pos, L.sel.T, L.sel.scale)
    if (d.nB <= 512) SPARDA_ROWL(1);
    else if (d.nB <= 2048) SPARDA_ROWL(4);
    else SPARDA_ROWL(16);
#undef SPARDA_ROWL
    return;
  }
  const DecodePartials pp = decode_attn_partials(L.ws, d);
  const int n_sel = rows * n_sel_chunks;
  const int n_attn = rows * ((pp.splits + 3) / 4);
  const int bps = (d.k + pp.splits - 1) / pp.splits;
  const dim3 grid(n_sel + n_attn);
#define SPARDA_LAYER(N)                                                                                            \
  hipLaunchKernelGGL((decode_layer_kernel<Tag, G, N>), grid, dim3(256), 0, s, n_sel, rows, (const uint8_t*)L.q,   \
                     (const uint8_t*)L.k, (const uint8_t*)L.v, L.idx, L.scores, pp.part_o, pp.part_ml,            \
                     (uint8_t*)L.out, d.T, d.nB, d.k, d.q_start, d.q_pos, d.Hkv, bps, pp.splits, d.scale,          \
                     (const uint8_t*)L.f_next, (const uint8_t*)L.kc_next, L.scores_next, L.sel.W, L.sel.nB,         \
                     n_vis_n, L.sel.q_pos, L.sel.T, L.sel.scale)
  if (d.nB <= 256) SPARDA_LAYER(1);
  else if (d.nB <= 2048) SPARDA_LAYER(8);
  else SPARDA_LAYER(32);
#undef SPARDA_LAYER
  launch_merge<Tag>(pp, L.out, s);  // the output is complete when this launch ends
}

hipError_t launch_decode_layer(const LayerLaunch& L, bool bf16, hipStream_t s) {
  const int G = L.attn.Hq / L.attn.Hkv;
#define SPARDA_LG(TAG, GG) launch_layer_g<TAG, GG>(L, s)
#define SPARDA_LG_G(TAG)                  \
  switch (G) {                            \
    case 1: SPARDA_LG(TAG, 1); break;     \
    case 2: SPARDA_LG(TAG, 2); break;     \
    case 4: SPARDA_LG(TAG, 4); break;     \
    case 8: SPARDA_LG(TAG, 8); break;     \
    default: return hipErrorInvalidValue; \
  }
  // bf16 only: an fp32 selection workgroup of 128 blocks would not fit the
  // attention's register allocation
  if (!bf16) return hipErrorInvalidValue;
  SPARDA_LG_G(BF16Tag)
#undef SPARDA_LG_G
#undef SPARDA_LG
  return hipGetLastError();
}

// Attention over a list of tokens per row (d.k = list length / 64 slots),
// read where they sit in the cache: the split attention in token mode, then
// the merge.
template <typename Tag, int G>
static void launch_attn_tokens_g(const void* q, const void* k, const void* v, const int32_t* tok_idx, void* out,
                                 const AttnDims& d, void* ws, hipStream_t s) {
  const DecodePartials pp = decode_attn_partials(ws, d);
  const int bps = (d.k + pp.splits - 1) / pp.splits;
  hipLaunchKernelGGL((attn_decode_kernel<Tag, G, 1, 0, true>), dim3(pp.rows, pp.splits), dim3(kWave), 0, s,
                     (const uint8_t*)q, (const uint8_t*)k, (const uint8_t*)v, tok_idx, nullptr, nullptr, pp.part_o,
                     pp.part_ml, (uint8_t*)out, d.T, d.nB, d.k, SPARDA_KV_CACHE_MODE, d.q_start, d.q_pos,
                     d.q_pos_per_row ? 1 : d.Hkv, nullptr, 0, bps, pp.splits, d.scale);
  launch_merge<Tag>(pp, out, s);
}

hipError_t launch_attn_tokens(const void* q, const void* k, const void* v, const int32_t* tok_idx, void* out,
                              bool bf16, const AttnDims& d, void* ws, hipStream_t s) {
  const int G = d.Hq / d.Hkv;
#define SPARDA_AT(TAG, GG) launch_attn_tokens_g<TAG, GG>(q, k, v, tok_idx, out, d, ws, s)
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

hipError_t launch_attn_decode(const void* q, const void* k, const void* v, const int32_t* idx,
                              void* out, bool bf16, const AttnDims& d, void* ws, hipStream_t s) {
  return launch_topk_attn_decode(nullptr, q, k, v, const_cast<int32_t*>(idx), out, bf16, d, ws, true, s);
}

hipError_t launch_topk_attn_decode(const float* scores, const void* q, const void* k, const void* v, int32_t* idx,
                                   void* out, bool bf16, const AttnDims& d, void* ws, bool merge, hipStream_t s) {
  const int G = d.Hq / d.Hkv;
#define SPARDA_AT(TAG, GG) launch_attn_g<TAG, GG>(q, k, v, idx, scores, out, d, ws, merge, s)
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

// ---- the decode attention's block-range results in a static device array ----
// For callers that cannot allocate (code under graph capture, serving loops
// that forbid hipMalloc): the partial results live in `scratch`, one copy per
// GPU, held until the process ends. In host code `scratch` names a host-side
// stand-in, not device memory, so the kernels receive the device address
// hipGetSymbolAddress returns for the current device, looked up once per
// device and kept.
static __device__ __align__(256) uint8_t scratch[kStaticScratchBytes];

namespace {
constexpr int kMaxScratchDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxScratchDevices] = {};
}  // namespace

hipError_t static_scratch(void** ptr) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxScratchDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    g_scratch_ptr[dev] = p;
  }
  *ptr = g_scratch_ptr[dev];
  return hipSuccess;
}

}  // namespace sparda
