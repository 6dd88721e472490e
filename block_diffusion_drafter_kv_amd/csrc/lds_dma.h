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

// Same copy with a wave-uniform 64-bit base in SGPRs and a per-lane 32-bit byte
// offset (global_load_lds with saddr): no per-copy 64-bit address arithmetic.
__device__ __forceinline__ void copy16_to_lds_sv(const void* sbase, uint32_t voff, void* lds_wave_base) {
  const uint32_t lds = __builtin_amdgcn_readfirstlane(
      (uint32_t)(uintptr_t)(__attribute__((address_space(3))) void*)lds_wave_base);
  uint32_t saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\ts_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %2, %3\n\ts_mov_b32 m0, %0"
      : "=&s"(saved)
      : "s"(lds), "v"(voff), "s"(sbase)
      : "memory");
}

// The same two copies without a memory clobber, for loops whose barriers
// (lds_barrier, which clobbers memory) already order every copy against the LDS
// reads of its stage: the clobber would make the compiler reload kernel
// arguments after each copy and wait for all outstanding LDS reads first.
// Volatile asm statements keep their order among themselves.
__device__ __forceinline__ void copy16_to_lds_nc(const void* g, void* lds_wave_base) {
  const uint32_t lds = __builtin_amdgcn_readfirstlane(
      (uint32_t)(uintptr_t)(__attribute__((address_space(3))) void*)lds_wave_base);
  uint32_t saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\ts_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %2, off\n\ts_mov_b32 m0, %0"
      : "=&s"(saved)
      : "s"(lds), "v"(g));
}
__device__ __forceinline__ void copy16_to_lds_sv_nc(const void* sbase, uint32_t voff, void* lds_wave_base) {
  const uint32_t lds = __builtin_amdgcn_readfirstlane(
      (uint32_t)(uintptr_t)(__attribute__((address_space(3))) void*)lds_wave_base);
  uint32_t saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\ts_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %2, %3\n\ts_mov_b32 m0, %0"
      : "=&s"(saved)
      : "s"(lds), "v"(voff), "s"(sbase));
}

// The same copy to an LDS byte address (wave-uniform) given as an integer: a
// ring addressed through a run-time stage index would otherwise turn the address
// into a generic pointer that must be cast back.
__device__ __forceinline__ uint32_t lds_addr(const void* lds_ptr) {
  return (uint32_t)(uintptr_t)(__attribute__((address_space(3))) const void*)lds_ptr;
}
__device__ __forceinline__ void copy16_to_lds_at(const void* g, uint32_t lds_wave_base) {
  const uint32_t lds = __builtin_amdgcn_readfirstlane(lds_wave_base);
  uint32_t saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\ts_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %2, off\n\ts_mov_b32 m0, %0"
      : "=&s"(saved)
      : "s"(lds), "v"(g));
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
