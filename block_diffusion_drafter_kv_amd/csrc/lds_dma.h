// Direct global -> LDS copies and the waits / barrier that order them.
#pragma once
#include "common.h"

namespace dfl {

typedef __attribute__((address_space(3))) void lds_void_t;
typedef __attribute__((address_space(1))) void glob_void_t;

// 16-byte global -> LDS copy: lane l of the wave lands at lds_wave_base + 16 * l.
// Issued through inline asm so that the compiler's wait insertion does not treat
// the copy as an LDS store aliasing every later LDS read (it would drain all
// copies in flight); ordering is provided by the explicit vmcnt waits and
// barriers of the ring loop, which contains no other vector-memory operation.
__device__ __forceinline__ void copy16_to_lds(const void* g, void* lds_wave_base) {
  const uint32_t lds = __builtin_amdgcn_readfirstlane(
      (uint32_t)(uintptr_t)(__attribute__((address_space(3))) void*)lds_wave_base);
  // M0 carries the LDS base; it is saved and restored around the copy (the
  // compiler reserves M0), with the one wait state an M0 write needs before an
  // LDS-DMA instruction reads it.
  uint32_t saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\ts_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %2, off\n\ts_mov_b32 m0, %0"
      : "=&s"(saved)
      : "s"(lds), "v"(g)
      : "memory");
}

// LDS byte address of a __shared__ object (32-bit, as M0 takes it)
__device__ __forceinline__ uint32_t lds_addr(const void* lds_ptr) {
  return (uint32_t)(uintptr_t)(__attribute__((address_space(3))) const void*)lds_ptr;
}

// Copies to an integer LDS byte address (wave-uniform) that declare M0 clobbered
// instead of saving and restoring it around every copy (the compiler sets M0
// again wherever it needs it; s_nop 0 is the wait state an M0 write needs
// before an LDS-DMA instruction reads it), and carry no memory clobber: for ring loops
// whose explicit waits and barriers order the copies against the LDS reads.
// The compiler keeps no value of its own in M0 on gfx950 unless it emits one of
// the few instructions that read it (indirect register moves, add-tid LDS
// operations, messages, GWS, buffer-to-LDS loads), none of which these kernels
// contain; a device-code test over the built library checks exactly that.
// sv: wave-uniform 64-bit global base in SGPRs plus a per-lane 32-bit offset.
__device__ __forceinline__ void copy16_to_lds_sv_m0(const void* sbase, uint32_t voff, uint32_t lds_wave_base) {
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, %2"
               :
               : "s"(lds_wave_base), "v"(voff), "s"(sbase)
               : "m0");
}
__device__ __forceinline__ void copy16_to_lds_m0(const void* g, uint32_t lds_wave_base) {
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, off"
               :
               : "s"(lds_wave_base), "v"(g)
               : "m0");
}

// s_waitcnt vmcnt(N) leaving the other counters unconstrained (gfx9 encoding)
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 0xF) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}

// s_waitcnt lgkmcnt(0) leaving the other counters unconstrained
__device__ __forceinline__ void wait_lgkmcnt0() { __builtin_amdgcn_s_waitcnt(0xC07F); }

// Workgroup barrier that is also a compiler memory fence (no LDS access moves
// across it) but, unlike __syncthreads, emits no wait on outstanding copies.
__device__ __forceinline__ void lds_barrier() { asm volatile("s_barrier" ::: "memory"); }

}  // namespace dfl
