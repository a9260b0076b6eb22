// lds_dma.h -- HBM -> LDS copies (global_load_lds_dwordx4) issued as inline assembly, for the
// kernels that stage K/V tiles in LDS. Device code only.
//
// The compiler cannot tell which LDS buffer an in-flight global_load_lds writes, so when the copy
// is issued through the builtin it waits for every outstanding load before each later LDS read --
// including the copy of the next tile into the other pipeline stage, which serialises the
// pipeline. Issued as inline assembly the copy is invisible to that analysis; each kernel orders
// it with its own s_waitcnt + barrier before reading the stage. M0 holds the wave's LDS
// destination (lane i lands at M0 + 16 i); the kernels that include this use M0 for nothing else.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace blasst {

#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"  // M0 is reserved to the compiler; see above
__device__ __forceinline__ void lds_dma16(const void *g, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off"
               :
               : "v"(g), "s"(lds)
               : "memory", "m0");
}

// The same copy from a wave-uniform base address (SGPR pair) plus a per-lane 32-bit byte offset:
// the address arithmetic of a row-per-instruction copy stays on the scalar unit.
__device__ __forceinline__ void lds_dma16_s(const void *base, uint32_t voff, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1"
               :
               : "v"(voff), "s"(base), "s"(lds)
               : "memory", "m0");
}
#pragma clang diagnostic pop

// The 32-bit LDS address of a __shared__ object, as a wave-uniform value.
__device__ __forceinline__ uint32_t lds_addr(const void *p) {
  return __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)p);
}

}  // namespace blasst
