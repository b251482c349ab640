// Direct global->LDS loads with a scalar base address: the address of each
// lane is a wave-uniform 64-bit base in SGPRs plus a 32-bit per-lane offset,
// so a kernel that reads the same lane pattern from many bases computes the
// offsets once and spends no vector instructions per load on addresses.
#pragma once

#include "common.h"

namespace sparda {

// One direct load of 16 bytes per lane from sbase + voff (sbase the same in
// every lane of the wave); lane i's bytes land at lds_wave_dst + 16 i. As
// with dma16, the kernel waits for its own loads (vmcnt) before the barrier
// that publishes them.
__device__ __forceinline__ void dma16_sv(const uint8_t* sbase, uint32_t voff, const uint8_t* lds_wave_dst) {
  const uint32_t m0 = __builtin_amdgcn_readfirstlane(
      (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) uint8_t*)lds_wave_dst);
  // readfirstlane returns int: each half goes through uint32_t before it is
  // widened, so the low half is zero-extended, never sign-extended
  const uint64_t b = (uint64_t)(uintptr_t)sbase;
  const uint32_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)(b >> 32));
  const uint32_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)b);
  const uint64_t bs = ((uint64_t)hi << 32) | (uint64_t)lo;
  asm volatile("global_load_lds_dwordx4 %0, %1" ::"v"(voff), "s"(bs), "{m0}"(m0) : "memory");
}

}  // namespace sparda
