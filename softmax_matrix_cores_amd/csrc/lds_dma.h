// lds_dma.h -- gfx950 helpers shared by the attention kernels: LDS DMA
// (buffer_load ... lds) issued as inline assembly, raw buffer descriptors,
// explicit vmcnt waits and a workgroup barrier that does not drain them.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "mx_device.h"

namespace fsattn {

constexpr int RSRC_W3 = 0x00020000;  // descriptor word 3 (gfx9): raw buffer, 32-bit data format

template <int N> __device__ __forceinline__ void wait_vm() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  // s_waitcnt: vmcnt[3:0] | expcnt[6:4] | lgkmcnt[11:8] | vmcnt[5:4] at [15:14]
  __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | ((N >> 4) << 14));
}
// wait for every outstanding LDS instruction (ds_write results included)
__device__ __forceinline__ void wait_lgkm0() {
  __builtin_amdgcn_s_waitcnt(15 | (7 << 4) | (0 << 8) | (3 << 14));
}
// workgroup barrier without the memory fence of __syncthreads (which would
// wait for every outstanding DMA); the clobber keeps LDS reads below it
__device__ __forceinline__ void barrier() { asm volatile("s_barrier" ::: "memory"); }

// Buffer descriptor (raw, stride 0) of `bytes` bytes at `base`, in SGPRs.
// Reads at or beyond `bytes` return zeros.
__device__ __forceinline__ v4i rsrc(uint64_t b, int bytes) {
  const int nrec = bytes < 0 ? 0 : bytes;
  return v4i{(int)__builtin_amdgcn_readfirstlane((uint32_t)b), (int)__builtin_amdgcn_readfirstlane((uint32_t)(b >> 32) & 0xFFFFu),
             __builtin_amdgcn_readfirstlane(nrec), RSRC_W3};
}

// buffer_load ... lds: each lane's 16 (or 4) bytes at voff land in LDS at
// M0 + 16 (or 4) * lane.  Issued as inline asm so that the compiler does not
// treat the asynchronous LDS write as aliasing every later LDS read (it would
// wait for all outstanding loads before each one); completion is tracked
// explicitly with s_waitcnt vmcnt and published with s_barrier.  A group of
// loads is bracketed by m0_save / m0_restore (M0 is the LDS destination).
__device__ __forceinline__ uint32_t m0_save() {
  uint32_t k;
  asm volatile("s_mov_b32 %0, m0" : "=s"(k));
  return k;
}
__device__ __forceinline__ void m0_restore(uint32_t k) { asm volatile("s_mov_b32 m0, %0" ::"s"(k)); }
__device__ __forceinline__ void dma_x4(const v4i& rs, uint32_t slot, uint32_t off, int voff) {
  asm volatile("s_add_u32 m0, %0, %1\n\tbuffer_load_dwordx4 %2, %3, 0 offen lds" ::"s"(slot), "s"(off), "v"(voff),
               "s"(rs)
               : "scc");
}
__device__ __forceinline__ void dma_x1(const v4i& rs, uint32_t slot, uint32_t off, int voff) {
  asm volatile("s_add_u32 m0, %0, %1\n\tbuffer_load_dword %2, %3, 0 offen lds" ::"s"(slot), "s"(off), "v"(voff),
               "s"(rs)
               : "scc");
}

__device__ __forceinline__ uint32_t lds_addr(const uint8_t* p) {
  return __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)p);
}

}  // namespace fsattn
