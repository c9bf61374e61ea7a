// Device helpers for global-to-LDS transfers (gfx950), shared by the GEMM and
// decode kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <cstdint>

namespace qk {

// One 128-bit global-to-LDS load: this lane's 16 bytes at g go to LDS byte
// lds_base + 16 * lane (lds_base is the wave-uniform LDS address in m0).
// Written as inline assembly so that the compiler does not treat every later
// LDS read as possibly aliasing the transfer (which makes it wait for all
// outstanding loads before each read); completion is tracked explicitly with
// wait_vmcnt before the data is read.  The instruction
// has no register results.  m0 is written here and nowhere else in the kernel.
__device__ __forceinline__ void lds_dma16(const void* g, uint32_t lds_base) {
  asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dwordx4 %0, off"
               :
               : "v"(g), "s"(lds_base)
               : "memory", "m0");
}

// The same load with its address split into a wave-uniform 64-bit base in
// scalar registers and this lane's unsigned 32-bit offset: advancing the base
// is then scalar arithmetic, not a 64-bit vector add per instruction.
__device__ __forceinline__ void lds_dma16_split(const void* sbase, uint32_t voff, uint32_t lds_base) {
  asm volatile("s_mov_b32 m0, %2\n\tglobal_load_lds_dwordx4 %0, %1"
               :
               : "v"(voff), "s"(sbase), "s"(lds_base)
               : "memory", "m0");
}

__device__ __forceinline__ uint32_t lds_addr(const char* p) {
  return __builtin_amdgcn_readfirstlane(
      static_cast<uint32_t>(reinterpret_cast<uintptr_t>((__attribute__((address_space(3))) const char*)p)));
}

// s_waitcnt on the vector-memory counter only (gfx9 encoding: vmcnt in bits
// 3:0 and 15:14, expcnt 6:4, lgkmcnt 11:8).  Global-to-LDS loads complete on
// this counter, so this is how a wave knows its DMA into LDS has landed.
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | ((N >> 4) << 14));
}

}  // namespace qk
