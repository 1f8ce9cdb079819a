// Global -> LDS copies through the buffer unit on gfx950, shared by the kernels
// that stage operands without passing them through registers.
#pragma once

#include "common.h"

namespace dflash {

// s_waitcnt vmcnt(N) with expcnt/lgkmcnt left at their no-wait maxima (gfx9 encoding:
// vmcnt bits 3:0 and 15:14).
template <int N>
__device__ __forceinline__ void wait_vmem() {
  static_assert(N >= 0 && N < 64, "vmcnt immediate");
  __builtin_amdgcn_s_waitcnt(0x0F70 | (N & 15) | ((N >> 4) << 14));
}

// s_waitcnt lgkmcnt(N) with vmcnt/expcnt left at their no-wait maxima.
template <int N>
__device__ __forceinline__ void wait_lgkm() {
  static_assert(N >= 0 && N < 16, "lgkmcnt immediate");
  __builtin_amdgcn_s_waitcnt(0xC07F | (N << 8));
}

// 16 bytes per lane from a buffer straight into LDS at lds_base + OFF + 16*lane; reads past
// the descriptor's num_records return zeros.  Issued as inline asm so the compiler
// does not treat the in-flight LDS write as a dependency of unrelated LDS reads
// (it would otherwise wait for it before every ds_read); completion is awaited
// explicitly (wait_vmem) before the barrier that publishes the slot.  No memory
// clobber: the slot it writes is not read before that barrier.
template <int OFF>
__device__ __forceinline__ void dma16(u32x4_t rsrc, uint32_t lds_base, uint32_t voff, uint32_t soff) {
  asm volatile("s_add_u32 m0, %3, %4\n\tbuffer_load_dwordx4 %0, %1, %2 offen lds"
               :: "v"(voff), "s"(rsrc), "s"(__builtin_amdgcn_readfirstlane(soff)),
                  "s"(__builtin_amdgcn_readfirstlane(lds_base)), "i"(OFF) : "scc");
}

// dma16 with the LDS address given as the sum of two scalar values (a ring slot
// and a region offset): the one add into M0 forms it.
__device__ __forceinline__ void dma16s(u32x4_t rsrc, uint32_t lds_a, uint32_t lds_b, uint32_t voff, uint32_t soff) {
  asm volatile("s_add_u32 m0, %3, %4\n\tbuffer_load_dwordx4 %0, %1, %2 offen lds"
               :: "v"(voff), "s"(rsrc), "s"(__builtin_amdgcn_readfirstlane(soff)),
                  "s"(__builtin_amdgcn_readfirstlane(lds_a)), "s"(__builtin_amdgcn_readfirstlane(lds_b)) : "scc");
}

__device__ __forceinline__ u32x4_t buffer_desc(const void* base, uint32_t bytes) {
  const uint64_t p = reinterpret_cast<uint64_t>(base);
  u32x4_t d = {static_cast<uint32_t>(p), static_cast<uint32_t>(p >> 32) & 0xFFFFu, bytes, 0x00020000u};
#pragma unroll
  for (int i = 0; i < 4; ++i) d[i] = __builtin_amdgcn_readfirstlane(d[i]);
  return d;
}

}  // namespace dflash
