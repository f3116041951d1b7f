// Direct global -> LDS copies on gfx950 and the waits around them.
//
// The copies are issued from inline assembly, so the compiler neither counts
// them nor guards LDS reads against them: every wait is explicit.  Loads of
// one wave complete in issue order, so "at most N outstanding" means every
// copy but the last N issued has landed.  The LDS base goes in M0 (one wait
// state before the copy reads it); lane i's bytes land at base + i * size,
// and the base must be the same in every lane of the wave.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace up {

typedef __attribute__((address_space(3))) const char lds_char;

__device__ __forceinline__ uint32_t lds_addr_of(const void* p) {
  return (uint32_t)(uintptr_t)(lds_char*)p;
}
// 16 bytes per lane from global address src to LDS at lds_base + lane * 16
__device__ __forceinline__ void lds_copy16(uintptr_t src, uint32_t lds_base) {
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off"
               :
               : "v"(src), "s"(__builtin_amdgcn_readfirstlane(lds_base))
               : "memory");
}
// 4 bytes per lane from global address src to LDS at lds_base + lane * 4
__device__ __forceinline__ void lds_copy4(uintptr_t src, uint32_t lds_base) {
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dword %0, off"
               :
               : "v"(src), "s"(__builtin_amdgcn_readfirstlane(lds_base))
               : "memory");
}
// 16 bytes per lane from sbase + voff (sbase the same in every lane, voff a
// 32-bit byte offset per lane) to LDS at lds_base + lane * 16
__device__ __forceinline__ void lds_copy16_sv(const void* sbase, uint32_t voff, uint32_t lds_base) {
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1"
               :
               : "v"(voff), "s"(sbase), "s"(__builtin_amdgcn_readfirstlane(lds_base))
               : "memory");
}
// this wave's outstanding global loads (copies included) <= N
template <int N>
__device__ __forceinline__ void lds_copy_wait() {
  static_assert(N >= 0 && N < 16, "vmcnt immediate");
  asm volatile("s_waitcnt vmcnt(%0)" : : "n"(N) : "memory");
}
// workgroup barrier that orders LDS only (no wait for outstanding copies)
__device__ __forceinline__ void lds_only_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" : : : "memory");
}

}  // namespace up
