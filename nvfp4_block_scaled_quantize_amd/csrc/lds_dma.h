// lds_dma.h -- gfx950 helpers for kernels that stream operands straight from
// global memory into LDS (global_load_lds_dwordx4 / _dword) several stages
// ahead and wait for them with the vector-memory counter.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace nvfp4 {

// s_waitcnt with only the vector-memory counter constrained (gfx9 encoding:
// vmcnt[3:0] | expcnt[6:4]=7 | lgkmcnt[11:8]=15 | vmcnt[5:4] in bits [15:14]).
template <int N>
__device__ __forceinline__ void wait_vmcnt_le() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt(0x0F70 | (N & 0xF) | ((N >> 4) << 14));
}

// LDS byte address of a shared-memory pointer.
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) unsigned char*)p;
}

// Direct global -> LDS copies of 16 (4) bytes per lane: lane i's bytes land at
// LDS address lds + 16*i (4*i).  Written as inline assembly so that the
// compiler does not treat every later LDS read as dependent on these
// asynchronous writes (it would wait for all outstanding vector-memory
// operations, including the loads of the stages in flight).  The kernel waits
// for them itself with s_waitcnt vmcnt + s_barrier before reading a stage.
// These instructions produce no VGPR result.
__device__ __forceinline__ void dma16(const void* sbase, uint32_t vofs, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, %2"
               :: "s"(lds), "v"(vofs), "s"(sbase) : "memory", "m0");
}
__device__ __forceinline__ void dma4(const void* sbase, uint32_t vofs, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dword %1, %2"
               :: "s"(lds), "v"(vofs), "s"(sbase) : "memory", "m0");
}
// The same 16-byte copy from a full 64-bit address per lane (gathers of rows
// that share no base within 4 GiB).
__device__ __forceinline__ void dma16_at(const void* gaddr, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, off"
               :: "s"(lds), "v"(gaddr) : "memory", "m0");
}

}  // namespace nvfp4
