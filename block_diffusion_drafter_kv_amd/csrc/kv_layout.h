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

// Paged storage (optional): a page holds page_size consecutive positions (a
// multiple of KV_BLOCK) of one sequence for every layer and kv head, as
// [layer][kv][page_size * D] with the 32-key blocks above inside; the caller's
// table maps (slot, position / page_size) to a page id.  Elements per page:
// n_layers * n_kv * page_size * D.  Contiguous storage is [layer][slot][kv]
// [ctx_alloc * D].
struct KvPages {
  const int32_t* table;   // [table_rows][per_slot] page ids, or null: contiguous
  int per_slot, page_size, n_pages, table_rows;
  int64_t page_elems;
};

// first element of (layer, slot, kv) holding `pos`, and pos's offset from it; false when unmapped
__device__ __forceinline__ bool kv_locate(const KvPages& pg, int64_t contig_head_elems, int max_slots, int n_kv,
                                          int D, int layer, int slot, int kv, int pos, int64_t* base,
                                          int* pos_in) {
  if (!pg.table) {
    *base = (((int64_t)layer * max_slots + slot) * n_kv + kv) * contig_head_elems;
    *pos_in = pos;
    return true;
  }
  const int page = slot < pg.table_rows ? pg.table[(int64_t)slot * pg.per_slot + pos / pg.page_size] : -1;
  if ((unsigned)page >= (unsigned)pg.n_pages) return false;
  *base = page * pg.page_elems + ((int64_t)layer * n_kv + kv) * pg.page_size * D;
  *pos_in = pos % pg.page_size;
  return true;
}

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
