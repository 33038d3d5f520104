// Helpers shared by the prefill kernels: raw buffer descriptors, buffer
// loads with the LDS-DMA flag, and empty asm statements that pin a value.
#pragma once
#include "device_common.h"

namespace inkattn {

// Raw buffer descriptor (gfx9 family) of `bytes` bytes at p, in scalar
// registers (p and bytes must be wave-uniform).  Word 3 selects untyped
// access; reads past `bytes` return zero.
__device__ __forceinline__ u32x4 make_buf_rsrc(const void* p, uint32_t bytes) {
  const uint64_t a = reinterpret_cast<uint64_t>(p);
  return u32x4{(uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)a),
               (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)(a >> 32) & 0xffffu),
               (uint32_t)__builtin_amdgcn_readfirstlane(bytes), 0x00020000u};
}
// One 16-byte buffer load straight into LDS: lane l writes its 16 bytes at
// LDS byte address lds + 16 l (M0 holds lds; it is set here and used by
// nothing else in these kernels).  rsrc is a raw buffer descriptor, voff the
// lane's byte offset, soff a wave-uniform byte offset.
__device__ __forceinline__ void lds_dma16(u32x4 rsrc, uint32_t lds, uint32_t voff, uint32_t soff) {
  asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dwordx4 %1, %2, %3 offen lds"
               :: "s"(lds), "v"(voff), "s"(rsrc), "s"(soff) : "memory");
}
// Four 16-byte buffer loads into LDS under one M0 value: load j writes lane
// l's bytes at LDS lds + 1024 j + 16 l.  The instruction offset 1024 j is
// added to the memory address too, so the caller passes voff_j less 1024 j
// (on a descriptor that starts 4 KiB early, so the difference stays
// positive).  Rewriting M0 before every load costs the issuing wave about
// 110 cycles per load (it waits for the previous load's use of M0); one M0
// per four loads issues them at the memory pipeline's rate.
__device__ __forceinline__ void lds_dma16x4(u32x4 rsrc, uint32_t lds, uint32_t v0, uint32_t v1,
                                            uint32_t v2, uint32_t v3, uint32_t soff) {
  asm volatile("s_mov_b32 m0, %0\n\t"
               "buffer_load_dwordx4 %1, %5, %6 offen lds\n\t"
               "buffer_load_dwordx4 %2, %5, %6 offen offset:1024 lds\n\t"
               "buffer_load_dwordx4 %3, %5, %6 offen offset:2048 lds\n\t"
               "buffer_load_dwordx4 %4, %5, %6 offen offset:3072 lds"
               :: "s"(lds), "v"(v0), "v"(v1), "v"(v2), "v"(v3), "s"(rsrc), "s"(soff) : "memory");
}
// Three such loads under one M0 value (instruction offsets 0, 1024, 2048).
__device__ __forceinline__ void lds_dma16x3(u32x4 rsrc, uint32_t lds, uint32_t v0, uint32_t v1,
                                            uint32_t v2, uint32_t soff) {
  asm volatile("s_mov_b32 m0, %0\n\t"
               "buffer_load_dwordx4 %1, %4, %5 offen lds\n\t"
               "buffer_load_dwordx4 %2, %4, %5 offen offset:1024 lds\n\t"
               "buffer_load_dwordx4 %3, %4, %5 offen offset:2048 lds"
               :: "s"(lds), "v"(v0), "v"(v1), "v"(v2), "s"(rsrc), "s"(soff) : "memory");
}
// An empty asm that reads a fragment: forces its load to have completed here.
__device__ __forceinline__ void keep_live(const Frag8<bf16>& f) { asm volatile("" :: "v"(f.v)); }
__device__ __forceinline__ void keep_live(const Frag8<float>& f) {
  asm volatile("" :: "v"(f.lo), "v"(f.hi));
}
__device__ __forceinline__ void keep_live(int x) { asm volatile("" :: "v"(x)); }
__device__ __forceinline__ void keep_live(float x) { asm volatile("" :: "v"(x)); }
__device__ __forceinline__ void keep_live(bf16 x) { asm volatile("" :: "v"(x.bits)); }
// One 4-byte buffer load straight into LDS: lane l writes at lds + 4 l.
__device__ __forceinline__ void lds_dma4(u32x4 rsrc, uint32_t lds, uint32_t voff, uint32_t soff) {
  asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dword %1, %2, %3 offen lds"
               :: "s"(lds), "v"(voff), "s"(rsrc), "s"(soff) : "memory");
}
// Wait until every load this wave issued (including the LDS-DMA ones) landed.
__device__ __forceinline__ void wait_all_loads() {
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
}

}  // namespace inkattn
