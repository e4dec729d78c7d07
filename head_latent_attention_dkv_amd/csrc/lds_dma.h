// Direct global -> LDS copies and explicit completion tracking for gfx950 kernels that
// stream operands through multi-stage LDS pipelines.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mla {

// Copy-phase rule (every kernel that issues the copies below follows it):
//
//   While any copy of a wave is in flight, that wave has no other vector-memory operation
//   (global or buffer load, store or atomic that the compiler emits) in flight.
//
// One counter, vmcnt, tracks every vector-memory operation of a wave.  The pipelines wait
// for "all but the newest N copies" with explicit wait_vmcnt<N>, which is exact only if
// every counted operation is a copy: the ISA returns loads of one kind in issue order, but
// a copy (which completes when its data is written to LDS) and a load into VGPRs, or a
// store, are not ordered with respect to each other, so with both kinds in flight a count
// of N no longer says which operations are done.  The compiler, for its part, computes the
// waits before the uses of its own loads without seeing the copies (they are inline
// assembly).  So a kernel
//   1. issues and consumes its own loads (query fragments, table reads) first and calls
//      copies_begin() -- which drains them -- before its first copy;
//   2. issues no compiler-visible vector-memory operation inside the copy loop (the loop
//      body reads LDS only);
//   3. calls copies_end() -- which drains the copies -- before the first compiler-visible
//      vector-memory operation after the loop (partial-result stores, the epilogue).
//   4. may instead issue its first copies, then its own loads, and drain everything
//      (drain_all()) before it uses any loaded value or copied tile: with nothing outstanding
//      after the drain, the count is exact again for the copy loop that follows.  The loads'
//      latency then overlaps the first copies'.
// A kernel that once issued later tiles' copies behind its query loads and waited for them
// with partial counts, against rules 1 and 4, read wrong tiles although the bytes in HBM
// were right.
//
// Stores are the one exception a kernel may take to rules 2 and 3 (the persistent K/V
// up-projection stores a tile while the next tile's copies are in flight): copies complete
// in issue order among themselves, so while an awaited copy is outstanding every later copy
// is too, and the count stays above N whatever the stores do; an outstanding store only
// holds the count above N longer.  The compiler emits no wait of its own for a store.  Loads
// into VGPRs stay excluded: the compiler's waits for them would be wrong.

// Wait until at most N vector-memory operations of this wave are outstanding.
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

// Opens a copy phase (rule 1): no compiler-visible vector-memory operation stays in flight.
__device__ __forceinline__ void copies_begin() { wait_vmcnt<0>(); }
// Closes a copy phase (rule 3): every copy has landed in LDS.
__device__ __forceinline__ void copies_end() { wait_vmcnt<0>(); }
// Rule 4: every vector-memory operation of the wave, copy or load, has completed.
__device__ __forceinline__ void drain_all() { wait_vmcnt<0>(); }
// Workgroup barrier without the compiler's implicit wait for all outstanding memory.
__device__ __forceinline__ void barrier_only() { asm volatile("s_barrier" ::: "memory"); }

// 16-byte global -> LDS copy per lane (lane l writes lds_addr + 16 l).  Issued as inline
// assembly so the compiler does not drain all outstanding copies (vmcnt(0)) before every
// LDS read it cannot disambiguate; completion is tracked explicitly with wait_vmcnt<>.
// The copy takes its LDS address from M0, and on this GPU family an LDS-DMA instruction
// needs one wait state after the SALU write of M0 (the compiler cannot see into the asm to
// insert it), hence the s_nop.
__device__ __forceinline__ void dma16(const void* gptr, uint32_t lds_addr) {
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off" ::"v"(gptr), "s"(lds_addr) : "memory", "m0");
}

// Same copy addressed as wave-uniform base (SGPR pair) + 32-bit per-lane byte offset, which
// keeps the 64-bit address arithmetic off the vector ALU.
__device__ __forceinline__ void dma16_s(const void* sbase, uint32_t voff, uint32_t lds_addr) {
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1" ::"v"(voff), "s"(sbase), "s"(lds_addr) : "memory", "m0");
}

// Non-temporal forms of the two copies above, for data a launch reads exactly once (cache
// rows in decode, projection weights): the lines stream past the L2 instead of evicting the
// lines that are read again (query blocks, activation rows).  On the decode step this took
// 202 -> 187 us, on the MLRA decode unit 236 -> 220 us.
__device__ __forceinline__ void dma16_nt(const void* gptr, uint32_t lds_addr) {
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off nt" ::"v"(gptr), "s"(lds_addr) : "memory", "m0");
}
__device__ __forceinline__ void dma16_s_nt(const void* sbase, uint32_t voff, uint32_t lds_addr) {
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1 nt" ::"v"(voff), "s"(sbase), "s"(lds_addr) : "memory", "m0");
}

// 4-byte form (64 lanes x 4 bytes = 256 contiguous LDS bytes), for narrow rows.
//
// Every lane of the wave must be active for any of these copies: an LDS-DMA issued under a
// partial exec mask still fills the LDS slots of the inactive lanes, which would overwrite
// the neighbouring rows.
__device__ __forceinline__ void dma4_s(const void* sbase, uint32_t voff, uint32_t lds_addr) {
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dword %0, %1" ::"v"(voff), "s"(sbase), "s"(lds_addr) : "memory", "m0");
}

__device__ __forceinline__ int bitrev4(int x) {
  return ((x & 1) << 3) | ((x & 2) << 1) | ((x & 4) >> 1) | ((x & 8) >> 3);
}

__device__ __forceinline__ uint32_t lds_addr_of(const void* p) {
  return (uint32_t)reinterpret_cast<uintptr_t>((__attribute__((address_space(3))) const unsigned char*)p);
}

}  // namespace mla
