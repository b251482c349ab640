// Direct global->LDS loads with a scalar base address: the address of each
// lane is a wave-uniform 64-bit base in SGPRs plus a 32-bit per-lane offset,
// so a kernel that reads the same lane pattern from many bases computes the
// offsets once and spends no vector instructions per load on addresses.
#pragma once

#include "common.h"

namespace sparda {

// LDS address (the 32-bit value a direct load takes in M0) of a pointer into
// shared memory, as a wave-uniform value.
__device__ __forceinline__ uint32_t lds_addr(const uint8_t* p) {
  return __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)(const __attribute__((address_space(3))) uint8_t*)p);
}

// One direct load of 16 bytes per lane from sbase + voff (sbase the same in
// every lane of the wave); lane i's bytes land at LDS address m0 + 16 i (m0
// wave-uniform). As with dma16, the kernel waits for its own loads (vmcnt)
// before the barrier that publishes them.
__device__ __forceinline__ void dma16_sv_m0(const uint8_t* sbase, uint32_t voff, uint32_t m0) {
  // readfirstlane returns int: each half goes through uint32_t before it is
  // widened, so the low half is zero-extended, never sign-extended
  const uint64_t b = (uint64_t)(uintptr_t)sbase;
  const uint32_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)(b >> 32));
  const uint32_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)b);
  const uint64_t bs = ((uint64_t)hi << 32) | (uint64_t)lo;
  asm volatile("global_load_lds_dwordx4 %0, %1" ::"v"(voff), "s"(bs), "{m0}"(m0) : "memory");
}

// The same with the wave's LDS destination as a pointer.
__device__ __forceinline__ void dma16_sv(const uint8_t* sbase, uint32_t voff, const uint8_t* lds_wave_dst) {
  dma16_sv_m0(sbase, voff, lds_addr(lds_wave_dst));
}

}  // namespace sparda
