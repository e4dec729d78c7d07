// Direct global -> LDS copies and explicit completion tracking for gfx950 kernels that
// stream operands through multi-stage LDS pipelines.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mla {

// Wait until at most N vector-memory operations of this wave are outstanding.
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}
// Workgroup barrier without the compiler's implicit wait for all outstanding memory.
__device__ __forceinline__ void barrier_only() { asm volatile("s_barrier" ::: "memory"); }

// 16-byte global -> LDS copy per lane (lane l writes lds_addr + 16 l).  Issued as inline
// assembly so the compiler does not drain all outstanding copies (vmcnt(0)) before every
// LDS read it cannot disambiguate; completion is tracked explicitly with wait_vmcnt<>.
__device__ __forceinline__ void dma16(const void* gptr, uint32_t lds_addr) {
  asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dwordx4 %0, off" ::"v"(gptr), "s"(lds_addr) : "memory", "m0");
}

__device__ __forceinline__ int bitrev4(int x) {
  return ((x & 1) << 3) | ((x & 2) << 1) | ((x & 4) >> 1) | ((x & 8) >> 3);
}

__device__ __forceinline__ uint32_t lds_addr_of(const void* p) {
  return (uint32_t)reinterpret_cast<uintptr_t>((__attribute__((address_space(3))) const unsigned char*)p);
}

}  // namespace mla
