// Direct global -> LDS copy for the gfx950 MFMA kernels.
#pragma once

#include <cstdint>

#include <hip/hip_runtime.h>

namespace gemmf32 {
namespace mfma {

// One global_load_lds_dwordx4: lane l copies 16 bytes from g into LDS at
// lds_wave + 16 l (lds_wave is the same for the whole wave).  The instruction
// takes its LDS address from M0, which is saved and restored around it.
//
// It is written as inline assembly on purpose: the compiler cannot tell which
// LDS buffer a load through its builtin writes, and so makes every later LDS
// read wait for all loads still in flight, including loads into the other
// buffer.  The kernels wait themselves (s_waitcnt vmcnt(0) before the barrier
// that publishes a buffer), so reads of one buffer overlap loads into the
// other.
__device__ __forceinline__ void load_lds16(const float* g, float* lds_wave) {
  const uint32_t lds_addr = __builtin_amdgcn_readfirstlane(
      (uint32_t)(uintptr_t)((__attribute__((address_space(3))) float*)lds_wave));
  uint32_t saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %2\n\t"
      "global_load_lds_dwordx4 %1, off\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(saved)
      : "v"(g), "s"(lds_addr)
      : "memory");
}

}  // namespace mfma
}  // namespace gemmf32
