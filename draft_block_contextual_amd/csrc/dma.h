// Direct global -> LDS loads for gfx950 (global_load_lds_dwordx4): one wave
// instruction copies 64 lanes x 16 bytes into 1 KB of LDS starting at the
// wave-uniform address in M0 (lane l writes bytes 16 l .. 16 l + 15), so
// staging costs no VGPRs.  The loads and the waits on them are issued as
// inline asm: the compiler then neither counts these loads nor guards LDS
// reads with blanket waits, and the explicit vmcnt waits are the only
// synchronisation (vector memory loads complete in issue order, so
// vmcnt <= N means all but the N most recent have landed).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dcoco {

__device__ __forceinline__ uint32_t lds_offset(const void* p) {
  return static_cast<uint32_t>(reinterpret_cast<uintptr_t>(p));
}

// lds must be wave-uniform
__device__ __forceinline__ void dma16(const void* g, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off"
               :
               : "v"(g), "s"(lds)
               : "memory", "m0");
}

// wait until at most N of this wave's vector loads are in flight, then barrier
template <int N>
__device__ __forceinline__ void wait_vmcnt_barrier() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  asm volatile("s_waitcnt vmcnt(%0)\n\ts_barrier" : : "n"(N) : "memory");
}

// wait for every vector load and LDS access of this wave, then barrier
__device__ __forceinline__ void wait_all_barrier() {
  asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)\n\ts_barrier" : : : "memory");
}

}  // namespace dcoco
