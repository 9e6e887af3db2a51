// Global -> LDS copies and vmcnt waits shared by the MFMA kernels (gfx950).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace jano {

// s_waitcnt immediate that waits until at most n vector-memory operations are
// outstanding (gfx9 encoding: vmcnt[3:0], expcnt[6:4], lgkmcnt[11:8], vmcnt
// high bits [15:14]; expcnt and lgkmcnt left at their "no wait" maximum).
constexpr int vmcnt_wait(int n) { return 0x0F70 | (n & 15) | ((n >> 4) << 14); }

// One global -> LDS copy of 16 bytes per lane: lane i's bytes land at
// lds_base + 16*i. Issued from asm so that the compiler does not treat every
// later LDS read as dependent on it (it would wait for all copies in flight,
// including the tiles being prefetched); kernels wait on vmcnt themselves.
// The instruction has no register results, only address operands.
__device__ __forceinline__ void copy16_to_lds(const void *gptr, uint32_t lds_base) {
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, off"
               :
               : "s"(lds_base), "v"(gptr)
               : "memory", "m0");
}

// Same copy with a wave-uniform 64-bit base in SGPRs and a per-lane 32-bit
// byte offset (saddr form): advancing the base costs no vector instructions.
__device__ __forceinline__ void copy16_to_lds_s(const void *sbase, uint32_t voff, uint32_t lds_base) {
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, %2"
               :
               : "s"(lds_base), "v"(voff), "s"(sbase)
               : "memory", "m0");
}

// LDS byte address of a __shared__ object (wave-uniform)
__device__ __forceinline__ uint32_t lds_addr(const void *p) {
  const uint32_t a = static_cast<uint32_t>(
      reinterpret_cast<uintptr_t>((__attribute__((address_space(3))) const char *)p));
  return __builtin_amdgcn_readfirstlane(a);
}

}  // namespace jano
