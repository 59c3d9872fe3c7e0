// Workgroup pipeline helpers shared by the attention kernels: direct
// global->LDS copies and the phase barrier of the two-group ping-pong.
//
// The kernels run 8 waves per workgroup in two groups of four (one wave of
// each group per SIMD).  Group 1 runs one phase behind group 0, so while one
// wave of a SIMD issues matrix instructions (Q.K^T, P.V) the other runs the
// vector softmax/encode work, and the two execution units overlap.  Phases are
// separated by a plain s_barrier (no memory fence: LDS tiles arrive by DMA and
// each wave waits for its own DMA with an explicit vmcnt wait).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace attn {

// 32-bit LDS address of a pointer into __shared__ memory.
__device__ inline uint32_t lds_address(const void* p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)p;
}

// Copy 16 bytes per lane from global memory straight into LDS: lane i of the
// wave reads base + off (base wave-uniform, off a per-lane byte offset below
// 4 GiB) and writes LDS bytes [lds + 16 i, lds + 16 i + 16).  `lds` must be
// wave-uniform.  Written as inline assembly so that the compiler does not
// insert a wait for the copy before unrelated LDS reads; completion is
// awaited explicitly with dma_wait().
__device__ inline void dma16(const void* base, uint32_t off, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, %2"
               :
               : "s"(__builtin_amdgcn_readfirstlane(lds)), "v"(off), "s"(base)
               : "memory");
}
// Same for 4 bytes per lane (lane i writes [lds + 4 i, lds + 4 i + 4)).
__device__ inline void dma4(const void* base, uint32_t off, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dword %1, %2"
               :
               : "s"(__builtin_amdgcn_readfirstlane(lds)), "v"(off), "s"(base)
               : "memory");
}
// The same two copies with the non-temporal hint (nt): for data that is read
// exactly once, such as a decode step's KV cache.
__device__ inline void dma16_nt(const void* base, uint32_t off, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, %2 nt"
               :
               : "s"(__builtin_amdgcn_readfirstlane(lds)), "v"(off), "s"(base)
               : "memory");
}
__device__ inline void dma4_nt(const void* base, uint32_t off, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dword %1, %2 nt"
               :
               : "s"(__builtin_amdgcn_readfirstlane(lds)), "v"(off), "s"(base)
               : "memory");
}
// Wait until every global load (and LDS copy) this wave issued has landed.
__device__ inline void dma_wait() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

// Workgroup barrier without a memory fence (the compiler may not move memory
// operations across it; no waits are emitted).
__device__ inline void phase_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// Wait for this wave's copies and join the workgroup barrier, but only when
// `take` (wave-uniform, in a scalar register) is nonzero.  The test and the
// branch around the barrier sit inside one asm statement, so that the code
// around it stays a single basic block for the compiler's scheduler and
// register allocator.  Each wave must still join the same number of barriers.
__device__ inline void dma_wait_barrier_if(int take) {
  asm volatile(
      "s_cmp_eq_u32 %0, 0\n\t"
      "s_cbranch_scc1 1f\n\t"
      "s_waitcnt vmcnt(0)\n\t"
      "s_barrier\n"
      "1:"
      :
      : "s"(take)
      : "memory", "scc");
}

// Set this wave's issue priority to PRIO when `take` (wave-uniform) is nonzero.
template <int PRIO>
__device__ inline void setprio_if(int take) {
  asm volatile(
      "s_cmp_eq_u32 %0, 0\n\t"
      "s_cbranch_scc1 1f\n\t"
      "s_setprio %1\n"
      "1:"
      :
      : "s"(take), "n"(PRIO)
      : "scc");
}

}  // namespace attn
