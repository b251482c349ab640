// Step 4 for a chunk of queries (prefill): GQA block-sparse attention of each
// 64-query tile over the blocks selected for that tile (bittide.aicompass.dev
// summary post, paragraph on block-sparse attention; techwalker.com article,
// section 五: in prefill block-sparse attention is the main cost).
//
// Dense contractions per selected block, on the matrix cores
// (v_mfma_f32_32x32x16_bf16). One workgroup owns one (sequence, KV head, query
// tile); each wave computes one head of the GQA group for 32 of the tile's 64
// queries (two waves per head), so all G heads share every K/V block staged in
// LDS, and a wave's registers (O^T accumulators, Q fragments, scores) fit two
// waves per SIMD: one wave's softmax then runs beside another's MFMAs.
//   S^T = K Q^T  (keys x queries): each lane owns one query column, so the
//                online-softmax statistics of a query stay in one lane (plus
//                its partner 32 lanes away);
//   O^T += V^T P^T: P^T is the S^T accumulator itself, rounded to bf16 in
//                register order. The MFMA k index then runs over the keys in
//                the accumulator's row order (groups of 4); V^T fragments are
//                read from LDS in that same order, so the sum is unchanged.
// Each 64-key block is worked as two 32-key halves in a software pipeline:
// the softmax of half s shares a basic block with the PV products of half s-1
// and the scores of half s+1, so that a wave has matrix-core and vector-ALU
// work in flight together. K and V blocks arrive
// in LDS by direct global->LDS loads two blocks ahead (four K and four V
// buffers; 128 KiB), rows granule-swizzled so that both fragment reads are free
// of bank conflicts: 16-byte granule g of K row r sits at g ^ (r & 15) (a K
// fragment read takes one granule of 16 consecutive rows), of V row r at
// g ^ 4 (r & 3) (a transposed V read takes 4 consecutive granules of 4
// consecutive rows). V^T fragments come straight from row-major V through the LDS
// transpose read ds_read_b64_tr_b16: within each group of 16 lanes, source lane
// 4e + q points at 4 consecutive channels of key kbase + e, and lane j receives
// channel dbase + j of keys kbase .. kbase + 3. A workgroup holds at most 4
// heads; a group of 8 runs as two workgroups.
#include <type_traits>

#include "common.h"
#include "launch.h"
#include "lds_dma.h"

namespace sparda {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef short i16x4 __attribute__((ext_vector_type(4)));

namespace {

constexpr int kRowB = kHeadDim * 2;         // bytes per bf16 row
constexpr int kKBytes = kBlock * kRowB;     // one K (or V) block in LDS

__device__ __forceinline__ bf16x8 as_v8(const u32x4& v) { return __builtin_bit_cast(bf16x8, v); }
__device__ __forceinline__ int swz(int r, int g) { return r * kRowB + ((g ^ (r & 15)) << 4); }
__device__ __forceinline__ int v_swz_granule(int r, int g) { return g ^ ((r & 3) << 2); }

// Two transposed 8-byte reads of a swizzled V block give the V^T MFMA fragment
// of keys {kb .. kb+3, kb+8 .. kb+11} at channel dbase + (lane % 16), where the
// lane's 16-lane group fixes kb and dbase.
__device__ __forceinline__ u32x4 vt_frag(const uint8_t* vblk, int kb, int dbase, int lane) {
  const int r = lane & 15;
  const int key = kb + (r >> 2);
  const int ch = dbase + 4 * (r & 3);
  const int off = (ch & 7) * 2;  // 0 or 8 bytes into the granule
  typedef __attribute__((address_space(3))) i16x4 lds_i16x4;
  const i16x4 a = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (lds_i16x4*)(vblk + key * kRowB + (v_swz_granule(key, ch >> 3) << 4) + off));
  const i16x4 b = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (lds_i16x4*)(vblk + (key + 8) * kRowB + (v_swz_granule(key + 8, ch >> 3) << 4) + off));
  const uint2 ua = __builtin_bit_cast(uint2, a), ub = __builtin_bit_cast(uint2, b);
  return u32x4{ua.x, ua.y, ub.x, ub.y};
}

// A block's 64 rows x 16 granules = 1024 16-byte slots, NT threads filling
// one slot each per load: this lane's source offsets within the block (the
// same for every block), in the K or the V swizzle.
template <int NT, bool kV>
struct BlockOffsets {
  uint32_t off[1024 / NT];
};
template <int NT, bool kV>
__device__ __forceinline__ BlockOffsets<NT, kV> block_lds_offsets() {
  BlockOffsets<NT, kV> o;
  const int wave = threadIdx.x / kWave;
  const int lane = threadIdx.x % kWave;
#pragma unroll
  for (int it = 0; it < 1024 / NT; ++it) {
    const int pos = (it * (NT / kWave) + wave) * kWave + lane;
    const int r = pos >> 4;
    const int g = kV ? v_swz_granule(r, pos & 15) : (pos & 15) ^ (r & 15);
    o.off[it] = (uint32_t)(r * kRowB + g * 16);
  }
  return o;
}
template <int NT, bool kV>
__device__ __forceinline__ void load_block_lds(const uint8_t* __restrict__ src_block, const BlockOffsets<NT, kV>& o,
                                               uint8_t* dst) {
  const int wave = threadIdx.x / kWave;
#pragma unroll
  for (int it = 0; it < 1024 / NT; ++it) dma16_sv(src_block, o.off[it], dst + (it * (NT / kWave) + wave) * kWave * 16);
}

}  // namespace

template <int HPW>
__global__ __launch_bounds__(128 * HPW) void attn_prefill_kernel(
    const uint8_t* __restrict__ q, const uint8_t* __restrict__ kbuf, const uint8_t* __restrict__ vbuf,
    const int32_t* __restrict__ idx, uint8_t* __restrict__ out, int G, int Tq, int q_start, int T, int nB,
    int n_tiles, int k, float scale) {
  constexpr int NT = 128 * HPW;  // threads: two waves (query halves) per head of the workgroup's head group
  constexpr int DMA = 1024 / NT;  // direct-to-LDS load instructions per wave per block
  __shared__ __attribute__((aligned(16))) uint8_t s_k[4][kKBytes];
  __shared__ __attribute__((aligned(16))) uint8_t s_v[4][kKBytes];

  const long row = blockIdx.x;  // (b, kv head)
  const int tile = blockIdx.y;
  const int wv = threadIdx.x / kWave;
  const int g = blockIdx.z * HPW + wv % HPW;  // head within the GQA group
  const int lane = threadIdx.x % kWave;
  const int half = lane >> 5;
  const int l32 = lane & 31;
  const int q0 = tile * kTile + 32 * (wv / HPW);  // this wave's 32 queries
  const int p_tile = q_start + tile * kTile;     // position of the tile's first query
  const int p_first = q_start + q0;              // position of this wave's first query
  const int32_t* sel = idx + (row * n_tiles + tile) * (long)k;

  // Q fragments (B operand of S^T = K Q^T): head g, this wave's 32 queries x 8 k-steps
  const long qrow0 = (row * G + g) * (long)Tq + q0;
  u32x4 qf[8];
  {
    const uint8_t* src = q + (qrow0 + l32) * kRowB + half * 16;
#pragma unroll
    for (int s = 0; s < 8; ++s) qf[s] = load16(src + s * 32);
  }

  f32x16 o[4];
#pragma unroll
  for (int dt = 0; dt < 4; ++dt) o[dt] = f32x16{};
  float m_run = -INFINITY, l_run = 0.f;

  // usable slots: valid, in range, not wholly after the tile (the same for
  // every wave of the workgroup, which shares the staged blocks)
  // Block index of slot j, read with a scalar load (j is wave-uniform): a
  // vector load would count against vmcnt, which tracks the direct-to-LDS
  // loads below.
  auto sel_at = [&](int j) { return sel[__builtin_amdgcn_readfirstlane(j)]; };
  auto usable = [&](int j) {
    const int b = sel_at(j);
    return b >= 0 && b < nB && b * kBlock <= p_tile + kTile - 1;
  };
  auto next_usable = [&](int j) {
    while (j < k && !usable(j)) ++j;
    return j;
  };
  const BlockOffsets<NT, false> k_offs = block_lds_offsets<NT, false>();
  const BlockOffsets<NT, true> v_offs = block_lds_offsets<NT, true>();
  auto load_k = [&](int j, uint8_t* dst) {
    load_block_lds<NT, false>(kbuf + (row * (long)T + (long)sel_at(j) * kBlock) * kRowB, k_offs, dst);
  };
  auto load_v = [&](int j, uint8_t* dst) {
    load_block_lds<NT, true>(vbuf + (row * (long)T + (long)sel_at(j) * kBlock) * kRowB, v_offs, dst);
  };
  // S^T for key half h (keys 32h .. 32h+31 of the block) x this wave's queries;
  // two accumulators (even and odd k-steps) keep two MFMA chains in flight
  auto scores_half = [&](const uint8_t* kblk, int h, f32x16& sa) {
    sa = f32x16{};
#pragma unroll
    for (int s = 0; s < 8; ++s) {
      const u32x4 ka = *reinterpret_cast<const u32x4*>(kblk + swz(32 * h + l32, 2 * s + half));
      sa = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_v8(ka), as_v8(qf[s]), sa, 0, 0, 0);
    }
  };
  // Online softmax of one key half per query column, on raw scores: the
  // reference m_run is kept in raw units and p = exp2(x * c - m * c) with
  // c = scale * log2(e). Only a block that reaches the tile's own positions
  // needs the causal mask (and the guard for a query that sees no key yet).
  // The reference moves only when a score exceeds it by more than 2^8 in exp2
  // units, so most halves leave the accumulators alone; numerator and
  // denominator share it, so the result does not depend on where it sits.
  const float c2 = scale * 1.4426950408889634f;
  // Returns alpha, the factor that moves O and l to the new reference; l is
  // already updated, O is rescaled by the caller once the previous half's PV
  // products have been added to it.
  auto softmax_half = [&](auto kMask, f32x16& sa, int key0, uint32_t (&ph)[8]) -> float {
    const int pq = p_first + l32;  // this lane's query position
    float mx = -INFINITY;
    if constexpr (decltype(kMask)::value) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int key = key0 + 8 * (r >> 2) + 4 * half + (r & 3);
        const float x = key <= pq ? sa[r] : -INFINITY;
        sa[r] = x;
        mx = fmaxf(mx, x);
      }
    } else {
#pragma unroll
      for (int r = 0; r < 16; ++r) mx = fmaxf(mx, sa[r]);
    }
    mx = max32(mx);
    // branch-free (bitwise, selects) so that the stage stays one basic block
    // for the scheduler: exp2(0) = 1 when the reference stays, exp2(-inf) = 0
    // when it is set for the first time
    const bool grow = ((mx - m_run) * c2 > 8.f) | ((m_run == -INFINITY) & (mx != -INFINITY));
    const float mn = grow ? mx : m_run;
    const float alpha = __builtin_amdgcn_exp2f(grow ? (m_run - mn) * c2 : 0.f);
    const float mc = mn == -INFINITY ? 0.f : mn * c2;  // -inf only on a masked block with nothing seen
    float sum = 0.f;
#pragma unroll
    for (int r = 0; r < 16; r += 2) {
      const float p0 = __builtin_amdgcn_exp2f(fmaf(sa[r], c2, -mc));
      const float p1 = __builtin_amdgcn_exp2f(fmaf(sa[r + 1], c2, -mc));
      sum += p0 + p1;
      ph[r >> 1] = pack_bf16(p0, p1);
    }
    sum = sum32(sum);
    l_run = l_run * alpha + sum;
    m_run = mn;
    return alpha;
  };
  // O^T += V^T P^T for key half h: 2 k-steps of 16 keys
  auto pv_half = [&](const uint8_t* vblk, int h, const uint32_t (&ph)[8]) {
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      const int kb = 32 * h + 16 * s + 4 * half;
      const u32x4 pb = {ph[4 * s], ph[4 * s + 1], ph[4 * s + 2], ph[4 * s + 3]};
#pragma unroll
      for (int dt = 0; dt < 4; ++dt) {
        // lane group (lane / 16): channels 32 dt + 16 ((lane / 16) % 2) .. +15
        const u32x4 va = vt_frag(vblk, kb, 32 * dt + 16 * ((lane >> 4) & 1), lane);
        o[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_v8(va), as_v8(pb), o[dt], 0, 0, 0);
      }
    }
  };

  // The work runs in stages, one per key half s of the usable blocks: stage s
  // issues the PV products of half s-1 and the scores of half s+1 on the
  // matrix cores and the softmax of half s on the vector ALUs, in one basic
  // block that the compiler schedules (explicit interleaving by
  // sched_group_barrier measured slower); O is rescaled at the stage's end,
  // after half s-1's products are in. Before the first stage P is all zero
  // (adds exactly 0).
  f32x16 sa_cur;           // scores of the half whose softmax runs now
  uint32_t ph_prev[8];     // P of the previous half, awaiting its PV products
#pragma unroll
  for (int i = 0; i < 8; ++i) ph_prev[i] = 0u;
  auto stage = [&](auto kMask, const uint8_t* __restrict__ k_nxt, int h_nxt, const uint8_t* __restrict__ v_prv,
                   int h_prv, int key0) {
    f32x16 sa_next;
    uint32_t ph[8];
    pv_half(v_prv, h_prv, ph_prev);
    scores_half(k_nxt, h_nxt, sa_next);
    const float alpha = softmax_half(kMask, sa_cur, key0, ph);
    if (__ballot(alpha != 1.f)) {  // wave-uniform; lanes that keep their reference have alpha 1
#pragma unroll
      for (int dt = 0; dt < 4; ++dt) o[dt] *= alpha;
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) ph_prev[i] = ph[i];
    sa_cur = sa_next;
  };

  // Usable blocks t = 0, 1, ...: K(t) in s_k[t % 4], V(t) in s_v[t % 4].
  // Block step t (stages of t's two halves) reads K(t), K(t+1), V(t-1), V(t)
  // and fills K(t+3) and V(t+2) into the buffers of K(t-1) and V(t-2). At its
  // end each wave waits for its loads issued one step earlier (K(t+2),
  // V(t+1)), leaving this step's in flight, and a barrier makes them visible
  // to every wave: a load has two block steps to land.
  int j0 = next_usable(0);
  int j1 = j0 < k ? next_usable(j0 + 1) : k;
  int j2 = j1 < k ? next_usable(j1 + 1) : k;
  if (j0 < k) {
    load_k(j0, s_k[0]);
    load_v(j0, s_v[0]);
  }
  if (j1 < k) {
    load_k(j1, s_k[1]);
    load_v(j1, s_v[1]);
  }
  if (j2 < k) load_k(j2, s_k[2]);
  __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
  __syncthreads();
  if (j0 < k) scores_half(s_k[0], 0, sa_cur);

  int bc = 0;          // t % 4
  int v_last = 0;      // buffer of V(t - 1) (V(0)'s before the first step: P is 0 then)
  while (j0 < k) {
    const int j3 = j2 < k ? next_usable(j2 + 1) : k;
    const int bn = (bc + 1) & 3, bf3 = (bc + 3) & 3, bf2 = (bc + 2) & 3;
    int issued = 0;
    if (j3 < k) {
      load_k(j3, s_k[bf3]);
      issued += DMA;
    }
    if (j2 < k) {
      load_v(j2, s_v[bf2]);
      issued += DMA;
    }
    const int key_base = sel_at(j0) * kBlock;
    // the next block's K buffer holds stale (finite) data after the last block:
    // its scores are computed and never used
    if (key_base + kBlock - 1 > p_first) {  // some key after some query of this wave
      stage(std::true_type{}, s_k[bc], 1, s_v[v_last], 1, key_base);
      stage(std::true_type{}, s_k[bn], 0, s_v[bc], 0, key_base + 32);
    } else {
      stage(std::false_type{}, s_k[bc], 1, s_v[v_last], 1, key_base);
      stage(std::false_type{}, s_k[bn], 0, s_v[bc], 0, key_base + 32);
    }
    if (issued == 2 * DMA) {
      __builtin_amdgcn_s_waitcnt(vmcnt_imm(2 * DMA));
    } else if (issued == DMA) {
      __builtin_amdgcn_s_waitcnt(vmcnt_imm(DMA));
    } else {
      __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
    }
    // No fence: a release fence would also wait for the loads just issued.
    // The memory clobber keeps LDS accesses on their side of the barrier;
    // every fragment read of this step has been consumed by its MFMA.
    asm volatile("s_barrier" ::: "memory");
    v_last = bc;
    j0 = j1;
    j1 = j2;
    j2 = j3;
    bc = bn;
  }
  pv_half(s_v[v_last], 1, ph_prev);  // the last half's products

  // O = O^T / l, written as 4 consecutive channels (8 B) per accumulator group
  {
    const float inv = l_run > 0.f ? 1.f / l_run : 0.f;
    uint8_t* dst = out + (qrow0 + l32) * kRowB;
#pragma unroll
    for (int dt = 0; dt < 4; ++dt)
#pragma unroll
      for (int rg = 0; rg < 4; ++rg) {
        const int d = 32 * dt + 8 * rg + 4 * half;
        uint2 v;
        v.x = pack_bf16(o[dt][4 * rg] * inv, o[dt][4 * rg + 1] * inv);
        v.y = pack_bf16(o[dt][4 * rg + 2] * inv, o[dt][4 * rg + 3] * inv);
        *reinterpret_cast<uint2*>(dst + d * 2) = v;
      }
  }
}

hipError_t launch_attn_prefill(const void* q, const void* k, const void* v, const int32_t* idx, void* out,
                               const AttnDims& d, hipStream_t s) {
  const int G = d.Hq / d.Hkv;
  const int hpw = G < 4 ? G : 4;  // heads per workgroup; G = 8 runs as two groups of 4
  const dim3 grid(d.B * d.Hkv, d.n_tiles, G / hpw);
#define SPARDA_AP(HPW)                                                                                          \
  hipLaunchKernelGGL(attn_prefill_kernel<HPW>, grid, dim3(128 * HPW), 0, s, (const uint8_t*)q, (const uint8_t*)k, \
                     (const uint8_t*)v, idx, (uint8_t*)out, G, d.Tq, d.q_start, d.T, d.nB, d.n_tiles, d.k, d.scale)
  switch (hpw) {
    case 1: SPARDA_AP(1); break;
    case 2: SPARDA_AP(2); break;
    case 4: SPARDA_AP(4); break;
    default: return hipErrorInvalidValue;
  }
#undef SPARDA_AP
  return hipGetLastError();
}

}  // namespace sparda
