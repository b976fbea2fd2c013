// Direct global-to-LDS copies (GLOBAL_LOAD_LDS) and explicit vmcnt waits for gfx950.
#pragma once

#include "common.hpp"

namespace mxq {

typedef __attribute__((address_space(3))) void* lds_ptr_t;

// Byte address of an LDS object as the M0 register takes it.
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return uint32_t(reinterpret_cast<uintptr_t>((lds_ptr_t)(const_cast<void*>(p))));
}

// GLOBAL_LOAD_LDS: each active lane's `size` bytes land at M0 + lane * size (lanes switched
// off by the exec mask write nothing).  `lds` must be the same in every lane of the wave.  Issued as inline asm so that the compiler does not
// treat every LDS read that follows as a hazard of the copy (it cannot tell buffers apart and
// would wait for the copy before each one); the caller waits on vmcnt itself before the
// barrier that publishes the data.  The compiler's own vmcnt waits for register loads stay
// correct because vector memory operations complete in issue order: an unseen copy can only
// make such a wait stricter.
__device__ __forceinline__ void lds_dma16(const void* g, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off" ::"v"(g), "s"(__builtin_amdgcn_readfirstlane(lds))
               : "memory", "m0");
}
__device__ __forceinline__ void lds_dma4(const void* g, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dword %0, off" ::"v"(g), "s"(__builtin_amdgcn_readfirstlane(lds))
               : "memory", "m0");
}

// The same copies addressed as a wave-uniform base (kept in SGPRs) plus a 32-bit per-lane byte
// offset, so a loop that walks a matrix only moves the base.
__device__ __forceinline__ void lds_dma16(const void* base, uint32_t off, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1" ::"v"(off), "s"(base),
               "s"(__builtin_amdgcn_readfirstlane(lds))
               : "memory", "m0");
}
__device__ __forceinline__ void lds_dma4(const void* base, uint32_t off, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dword %0, %1" ::"v"(off), "s"(base),
               "s"(__builtin_amdgcn_readfirstlane(lds))
               : "memory", "m0");
}

// Wait until at most N vector memory operations of this wave are outstanding.
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt immediate");
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

}  // namespace mxq
