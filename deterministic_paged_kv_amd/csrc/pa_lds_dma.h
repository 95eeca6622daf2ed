// Direct-to-LDS loads (global_load_lds_dwordx4) and their hand-counted waits, shared by the
// prefill attention kernel and the backward kernels.
#pragma once
#include <hip/hip_runtime.h>

#include <cstdint>

namespace pa {

// LDS byte address of a shared-memory pointer (the direct-to-LDS loads take it in M0).
__device__ __forceinline__ uint32_t lds_address(const void* p) {
  return (uint32_t)(uintptr_t)(__attribute__((address_space(3))) const char*)(p);
}

// One wave-wide direct-to-LDS load: lane l reads the 16 bytes at base + voff (voff per lane)
// and they land at LDS byte lds + 16 l.  Issued as inline assembly so that the compiler's
// own wait-count tracking, which cannot tell these writes from the LDS reads of other
// buffers and would wait for every load in flight before any LDS read, leaves them alone:
// completion is waited for explicitly (s_waitcnt vmcnt) before the workgroup barrier that
// publishes a tile.  vmcnt counts these loads with the compiler's own in issue order, so a wait
// the compiler places for its own loads is never too weak, only sometimes stronger.
// lds and base are wave-uniform; readfirstlane keeps them in scalar registers even where the
// compiler's divergence analysis cannot tell.
__device__ __forceinline__ void lds_dma16(uint32_t lds, const void* base, uint32_t voff) {
  // (readfirstlane returns a signed int: each half goes through uint32_t before it is widened,
  // or the low half would be sign-extended into the high one)
  const uint64_t b = (uint64_t)(uintptr_t)base;
  const uint32_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)b);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)(b >> 32));
  const uint64_t bs = ((uint64_t)hi << 32) | (uint64_t)lo;
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, %2" ::"s"(
                   __builtin_amdgcn_readfirstlane(lds)),
               "v"(voff), "s"(bs)
               : "memory");
}
// s_waitcnt vmcnt(N) with the other counters left alone (gfx9 encoding: vmcnt in bits 3:0
// and 15:14, expcnt 6:4, lgkmcnt 11:8)
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | 0x0F70);
}

}  // namespace pa
