// Storage order of keys and values (drafter KV cache and the block's own K/V).
//
// A head's keys are stored in blocks of 32 consecutive positions; one block is
// 32 x D contiguous elements, permuted into the order in which the attention
// kernel's MFMA operand loads consume them, so that every load instruction of a
// wave reads one contiguous span (64 lanes x 8 elements).
//
// K block: the kernel reads K as the A operand of S^T = K Q^T, 16 keys x 32
// dims per fragment, lane (r16, grp) holding key r16 of the fragment and dims
// 8*grp .. 8*grp+7.  Within a 32-key group the two 16-key fragments t = 0, 1
// take keys 8*(r16>>2) + 4*t + (r16&3), a permutation that lets the score
// tile's rows (4 consecutive per lane group) line up with the B operand of the
// P V product without register shuffles.
//   element (key j, dim e) -> ((t*KS + s)*64 + 16*grp + r16)*8 + (e & 7)
//   t = (j>>2)&1, r16 = ((j>>3)<<2) | (j&3), s = e>>5, grp = (e>>3)&3, KS = D/32
// V block: the kernel reads V^T as the A operand of O^T = V^T P^T, 16 dims x 32
// keys per fragment, lane (r16, grp) holding dim 16*dt + r16, keys 8*grp .. +7.
//   element (key j, dim e) -> ((e>>4)*64 + 16*(j>>3) + (e&15))*8 + (j & 7)
#pragma once
#include <stdint.h>

namespace dfl {

constexpr int KV_BLOCK = 32;   // positions per storage block

__host__ __device__ __forceinline__ int kblk_off(int j, int e, int D) {
  const int t = (j >> 2) & 1, r16 = ((j >> 3) << 2) | (j & 3);
  return (((t * (D >> 5) + (e >> 5)) * 64 + 16 * ((e >> 3) & 3) + r16) << 3) + (e & 7);
}

__host__ __device__ __forceinline__ int vblk_off(int j, int e) {
  return ((((e >> 4) * 64) + 16 * (j >> 3) + (e & 15)) << 3) + (j & 7);
}

// offsets of (position, dim) inside one head's region of ctx_alloc * D elements
__host__ __device__ __forceinline__ int64_t k_off(int64_t pos, int e, int D) {
  return (pos >> 5) * (int64_t)(KV_BLOCK * D) + kblk_off((int)(pos & 31), e, D);
}
__host__ __device__ __forceinline__ int64_t v_off(int64_t pos, int e, int D) {
  return (pos >> 5) * (int64_t)(KV_BLOCK * D) + vblk_off((int)(pos & 31), e);
}

}  // namespace dfl
