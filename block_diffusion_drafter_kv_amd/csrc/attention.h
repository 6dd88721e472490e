// Block attention: the K+1 block rows of every request attend, without a mask
// inside the block, to [context K/V ; block K/V] ([P4 §5.3 table], [P1
// "关键创新" Step 3]).  Few queries (g*(K+1) per kv head) against a long context:
// the kernel streams K and V exactly once per (request, kv head) from HBM.
//
// Work split, decided on the device from the actual context lengths (no host
// sync).  A segment is one (request, kv head, q-row part); its keys form
// ceil(C/32) cache groups of 32 keys plus one group holding the block's own
// R <= 32 keys.  The groups of all segments are laid end to end and cut into
// equal ranges, one per work-group, so every work-group streams about the same
// number of bytes whatever the mix of context lengths.
//   16-bit K/V (attn_wave_kernel): ranges are not snapped, so a range may start
//   or end inside a segment; each (work-group, segment) piece writes one partial
//   record (O / l in fp16, fragment order; m and l in fp32) at index w + s.
//   fp32 K/V (attn_kernel): each segment is cut into chunks of cg = max(chunk_min,
//   ceil(groups / chunk_max)) groups and the range ends are snapped to chunk
//   starts, so a chunk's partial record (unnormalised O, m, l in fp32, row
//   layout) depends on its request alone.
// A combine kernel merges each segment's records in order.
//
// K and V are stored in 32-key blocks in MFMA operand order (kv_layout.h), so
// every 64-lane fragment is one contiguous 1 KB span, copied straight into a ring
// of LDS stages shared by the work-group's waves.  Scores are computed
// transposed, S^T = K Q^T, so that the softmax probabilities land in registers
// as the B operand of O^T = V^T P^T.
#pragma once
#include "common.h"
#include "kv_layout.h"

namespace dfl {

struct AttnPlan {          // written by attn_plan_kernel
  int32_t total;           // 32-key groups over all segments
  int32_t per_wg;          // groups per work-group range
  int32_t n_wg;            // work-groups with a non-empty range
};

struct AttnArgs {
  const void* qb;          // [n_req][n_kv][QRpad][D]
  const void* cache_k;     // layer base: [slot][n_kv][ctx_alloc * D], 32-key blocks
  const void* cache_v;     // layer base: [slot][n_kv][ctx_alloc * D], 32-key blocks
  const void* kb;          // block's own keys   [n_req][n_kv][Rpad * D] (Rpad == 32: one block)
  const void* vb;          // block's own values [n_req][n_kv][Rpad * D]
  const int32_t* slots;
  const int32_t* ctx_len;
  const AttnPlan* plan;
  const int32_t* seg_start;   // [n_seg + 1] first group of each segment (segment s = (r*n_kv + kv)*splits + z)
  const int32_t* chunk_base;  // [n_seg] first partial-result record (chunk) of each segment
  const int4* seg_desc;       // [n_seg] (slot, context length, first group, group count)
  const int4* wg_range;       // [work-groups] (first group, end group, segment of the first group, -)
  float* o_part;              // fp32: [chunk][QRT*16][D]; 16-bit: fp16 O/l [piece][QRT][D/16][64 lanes][4]
  float* m_part;              // [chunk or piece][QRT*16]   running max (exp2 domain)
  float* l_part;              // [chunk or piece][QRT*16]   sum of exp2(s - m)
  int n_seg, n_kv, R, Rpad, QRpad, rows_per_split, splits;
  int chunk_min, chunk_max;   // chunk size rule (groups), see above
  int64_t ctx_alloc;
  float scale_log2;        // log2(e) / sqrt(D)
  int causal;              // 1: block row j sees block keys 0..j only (context keys always)
  // paged cache (page_table null: contiguous); cache_k / cache_v then point at the
  // layer's part of page 0 and a kv head's part of a page is page_size * D elements
  const int32_t* page_table;   // [table_rows][pages_per_slot]
  int pages_per_slot, gpp, n_pages, table_rows;   // gpp: 32-key groups per page
  int64_t page_elems;
};

struct AttnCombineArgs {
  const float* o_part; const float* m_part; const float* l_part;
  const int32_t* seg_start; const int32_t* chunk_base;
  void* out;               // [n_req*R][q_dim] activations (T)
  int n_kv, group, R, rows_per_split, splits, QRT16, q_dim, D;
  int chunk_min, chunk_max;
  // wave-range records (16-bit K/V), or null: the plan's per_wg is the groups per wave range;
  // segment s has one record per wave range it meets, at w + s for those waves w (attn_wave_kernel)
  const AttnPlan* wave_plan;
};

// groups per chunk of a segment of `len` groups
__host__ __device__ __forceinline__ int attn_chunk_groups(int len, int chunk_min, int chunk_max) {
  const int c = (len + chunk_max - 1) / chunk_max;
  return c > chunk_min ? c : chunk_min;
}

}  // namespace dfl
