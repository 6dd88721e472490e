// Block attention: the K+1 block rows of every request attend, without a mask
// inside the block, to [context K/V ; block K/V] ([P4 §5.3 table], [P1
// "关键创新" Step 3]).  Few queries (g*(K+1) per kv head) against a long context:
// the kernel streams K and V exactly once per (request, kv head) from HBM.
//
// Work split (decided on the device from the actual context lengths, no host
// sync): the context keys of each request are cut into chunks of CK keys; one
// work-group handles (chunk, kv head[, q-row part]) with 4 waves taking a
// quarter of the chunk each.  Scores are computed transposed, S^T = K Q^T, so
// that the softmax probabilities land in registers exactly as the B operand of
// O^T = V^T P^T.  K and V are stored in 32-key blocks in MFMA operand order
// (kv_layout.h), so every fragment load of a wave is one contiguous 1 KB read;
// each wave keeps the next two key groups in flight in registers while it
// computes on the current one.  Waves merge through LDS in a fixed order, and a
// combine kernel merges the chunks of a request (log-sum-exp rescaling, fixed
// order).
#pragma once
#include "common.h"
#include "kv_layout.h"

namespace dfl {

struct AttnPlan {          // written by attn_plan_kernel
  int32_t count;           // number of work items
  int32_t ck;              // chunk size (keys)
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
  const int4* items;       // (req, key_begin, key_end, is_last)
  float* o_part;           // [item][n_kv][splits][QRT*16][D]
  float* m_part;           // [item][n_kv][splits][QRT*16]
  float* l_part;
  int n_kv, R, Rpad, QRpad, rows_per_split, splits;
  int64_t ctx_alloc;
  float scale_log2;        // log2(e) / sqrt(D)
};

struct AttnCombineArgs {
  const float* o_part; const float* m_part; const float* l_part;
  const int32_t* first_item; const int32_t* n_items;
  void* out;               // [n_req*R][q_dim] activations (T)
  int n_kv, group, R, rows_per_split, splits, QRT16, q_dim, D;
};

}  // namespace dfl
