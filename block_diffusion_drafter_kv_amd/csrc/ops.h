// Internal launch interface between the host library and the kernels.
#pragma once
#include "common.h"
#include "gemm.h"
#include "epilogues.h"
#include "attention.h"

namespace dfl {

// drafter element type (dflash_config.dtype): fp32, or bf16 inputs with fp16 operands
enum { DT_F32 = 0, DT_BF16 = 1 };
// operand type of one matrix product
enum OpType { OP_F32 = 0, OP_BF16 = 1, OP_F16 = 2 };

// ---- GEMM (gemm_inst.hip) ----
enum EpiKind { EPI_STORE_F32 = 0, EPI_STORE_T, EPI_RESADD, EPI_SWIGLU, EPI_QKV, EPI_KVINJECT, EPI_LMHEAD,
               EPI_STORE_SPLIT };

struct GemmPlan {
  int bm = 128, bn = 128, splits = 1;
  int sb = 0;   // 16-bit 128 x 128 tiles: B ring depth 3 (with a 2-deep A ring), else 2
};
// output tile width of the products whose epilogue keeps per-tile statistics
// (the LM head): the column width of its statistics tiles
inline int gemm_bn(int) { return 128; }
// Choose tile/split for an M x N x K product (K multiple of the slab); wide = the
// vocabulary product (widest tiles).
// big_ok: the product's epilogue has a 256 x 256 instantiation (fc store, K|V
// injection, LM head).
GemmPlan plan_gemm(int op, int M, int N, int K, int num_cus, bool wide = false, bool big_ok = false);
// Fill tiles/splits/partials fields of g and launch kernel (+ reduce when split,
// unless g.keep_partials).  Returns the launched split count and partial-tile
// shape: with keep_partials and splits > 1 the unscaled partial sums of output
// (m, n) are partials[s * Mpad * Npad + m * Npad + n], s < splits, and the
// epilogue did not run.
// op: operand type; OP_BF16 supports only EPI_STORE_F32 (the fc product).
struct GemmShape {
  int splits, Mpad, Npad;
};
GemmShape launch_gemm(int op, EpiKind kind, GemmArgs g, const void* epi_params, const GemmPlan& plan,
                      float* partials, size_t partials_elems, hipStream_t s);

// ---- attention (attention.hip) ----
// attention work plan: per-segment group starts, equal group ranges for up to
// n_wg_max work-groups (at least min_per_wg groups each), per-segment chunk bases
void launch_attn_plan(const int32_t* slots, const int32_t* ctx_len, int n_req, int n_kv, int splits, int n_wg_max,
                      int min_per_wg, int chunk_min, int chunk_max, AttnPlan* plan, int32_t* seg_start,
                      int32_t* chunk_base, int4* seg_desc, int4* wg_range, hipStream_t s);
// fp32 K/V: LDS-ring work-groups over chunk-snapped group ranges
void launch_attn(int D, int qrt, const AttnArgs& a, int grid, hipStream_t s);
// 16-bit K/V: work-groups of up to two waves sharing an LDS ring, over equal
// group ranges (plan built without chunk snapping)
void launch_attn_waves(int D, int qrt, const AttnArgs& a, int grid, hipStream_t s);
// work-groups of the 16-bit streamed attention that fit one CU at once (its LDS ring and registers)
int attn_waves_wg_per_cu();
void launch_attn_combine(int dtype, int D, const AttnCombineArgs& a, dim3 grid, hipStream_t s);

// Top-p set of one row over the whole vocabulary (no top-k): the ids in
// probability-descending order (ties: ascending id) up to the one whose
// cumulative probability reaches top_p.  Members: ids whose key(z / T) exceeds
// key, or equals it with id <= cut (key: order-preserving uint32 image of the
// float); mass = sum of exp(z / T - row max) over the members.
struct Nucleus {
  uint32_t key;
  int32_t cut;
  float mass;
  float pad;
};

// X rows += scale * (sum of a split product's partials, in split order), then
// RMSNorm of the updated rows into h_out (rmsnorm's row mapping); H <= 8192
void launch_partials_add_norm(int dtype, int n_rows, int H, float* X, int map_mask, int K, int R, const float* P, int ld,
                              int splits, int64_t split_stride, float scale, const void* gain, void* h_out, float eps,
                              hipStream_t s);
// ---- elementwise / row kernels (kernels.hip) ----
void launch_rope_table(float2* table, int n_pos, int d, double theta, hipStream_t s);
void launch_embed_norm(int dtype, int n_rows, int R, const int32_t* anchors, int mask_id, int vocab, const void* embed,
                       const void* mask_emb, float scale, int H, float* X, const void* gain, void* h_out, float eps,
                       int32_t* err, hipStream_t s, float* rs_out = nullptr);
// out row o reads X row (map_mask ? (o / K) * R + 1 + o % K : o); rows at or past
// (*n_valid - valid_base) are skipped when n_valid is given (device-side row count);
// rs_out (or null) receives each output row's RMS scale rsqrt(mean(x^2) + eps)
void launch_rmsnorm(int dtype, int n_rows, int H, const float* X, int map_mask, int K, int R, const void* gain,
                    void* h_out, float eps, hipStream_t s, const int32_t* n_valid = nullptr, int valid_base = 0,
                    float* rs_out = nullptr);
void launch_inject_scan(int n_req, const int32_t* slots, const int32_t* row_start, const int32_t* row_count,
                        int32_t* ctx_len, int max_ctx, int max_batch, int64_t rows_upper, int32_t* req_off,
                        int32_t* req_pos, int32_t* err, hipStream_t s);
// gemm row table of an injection; source rows at or past max_row (not addressable
// with 32-bit byte offsets) are skipped and flag the error word
void launch_inject_fill(int n_req, int64_t rows_upper, const int32_t* slots, const int32_t* row_start,
                        const int32_t* path_nodes, int max_path, int tree_stride, const int32_t* req_off,
                        const int32_t* req_pos, int64_t max_row, int32_t* a_rows, int32_t* row_slot,
                        int32_t* row_pos, int32_t* err, hipStream_t s);
void launch_row_finalize(int n_rows, int n_tiles, const float* tmax, const float* tsum, const int32_t* targ,
                         float* row_max, float* row_lse, int32_t* argmax_out, float* out_row_max, float* out_row_lse,
                         hipStream_t s);
// tile_w: column width of the LM-head statistics tiles (the GEMM's BN)
void launch_sample(int n_rows, int K, const int32_t* slots, uint64_t seed, uint64_t step, float inv_temp,
                   const float* logits, int V, int n_tiles, int tile_w, const float* tmax, const float* tsum,
                   const float* row_max, int32_t* draft_ids, hipStream_t s);
void launch_topk(int n_rows, int V, int k, const float* logits, const float* tmax, int n_tiles, int tile_w,
                 float inv_temp, const float* row_max, const float* row_lse, int32_t* ids_out, float* probs_out,
                 hipStream_t s);
void launch_tree(int n_req, int L, int Kc, int stride, int B, const float* probs, const int32_t* ids, const int32_t* anchors,
                 int32_t* tokens, int32_t* parents, int32_t* depth, uint64_t* mask, hipStream_t s);
void launch_verify_greedy(int n_req, int K, int V, const int32_t* draft_ids, const float* target, int32_t* post,
                          int32_t* out_tokens, int32_t* out_len, int32_t* accept_len, int32_t* next_anchor,
                          hipStream_t s);
// draft-tree verifier walk: greedy (row argmax of every node, then the walk) or sampled
void launch_verify_tree(int n_req, int n_nodes, int max_out, int V, const int32_t* slots, const int32_t* tokens,
                        const int32_t* parents, const float* target, float temperature, uint64_t seed, uint64_t step,
                        int32_t* out_tokens, int32_t* out_len, int32_t* accept_len, int32_t* next_anchor,
                        int32_t* path_out, int32_t* err, hipStream_t s);
// LDS segments (8 bytes each) the sampling tree walk keeps for a vocabulary of V ids.
int tree_walk_segments(int V);
// DFlash 2: rejection against candidate-subset draft distributions (C <= 64)
// Row statistics of fp32 rows (max z/T and sum exp(z/T - max), or its log), with
// optional per-128-id tile maxima; row m lands at (m / per) * group + off + m % per.
void launch_row_stats(int rows, int V, const float* x, float inv_temp, float* tmax, int n_tiles, float* out_max,
                      float* out_b, int os, int per, int group, int off, int want_log, hipStream_t s);
// whether the verification draws' LDS chunk table fits for this vocabulary
int draw_vocab_ok(int V);
// number of 256-id chunks of the verification draws (chunk-sum scratch: 2 * n_req * chunks floats)
int draw_chunks(int V);
// stats [n_req * (K+1) * 2], acc [n_req], chunks [n_req * draw_chunks(V)] floats
void launch_verify_subset(int n_req, int K, int C, int V, const int32_t* slots, const int32_t* draft_ids,
                          const int32_t* cand_ids, const float* cand_probs, const float* target, float inv_temp,
                          uint64_t seed, uint64_t step, float* stats, int32_t* acc, float* chunks,
                          int32_t* out_tokens, int32_t* out_len, int32_t* accept_len, int32_t* next_anchor,
                          int32_t* err, hipStream_t s, Nucleus* nuc = nullptr, float top_p = 1.f);
// DFlash 2: y = dynamic two-tap conv of x = X * rs * gain [M, H] (blocks of R rows, rs [M] the
// rows' RMS scales) with kernel corrections [M, 2H/G] = scale * sum over s < splits of
// corr[s * split_stride + m * corr_ld + j] (the split partials of the correction product)
void launch_dyn_conv(int dtype, int M, int R, int H, int G, const float* X, const float* rs, const void* gain,
                     const float* corr, int corr_ld, int splits, int64_t split_stride, float scale, const void* base,
                     void* y, hipStream_t s);
// DFlash 2: X[rows] += two-tap conv of the sub-layer output o (fp32 [M, H]) with corrections corr
// [M, 2H/G], then RMSNorm of the updated rows into h_out (row mapping as launch_rmsnorm)
void launch_conv_post_norm(int dtype, int n_rows, int H, int G, float* X, int map_mask, int K, int R, const float* o,
                           const float* corr, const void* base, const void* gain, void* h_out, float eps,
                           float* rs_out, hipStream_t s);
// DFlash 2: selector pair-score table (scratch [n_req*K, C, C]) and walk over cand [n_req*K, C] with
// gate [n_req*K, rank] and codebooks A, B [V, rank]
void launch_sel_walk(int dtype, int n_req, int K, int C, int rank, int V, const int32_t* slots,
                     const int32_t* anchors, const float* logits, const int32_t* cand, const float* gate,
                     const void* A, const void* B, float temperature, uint64_t seed, uint64_t step, float* table,
                     int32_t* draft_ids, int32_t* cand_out, float* probs_out, int32_t* err, hipStream_t s);
// symmetric top-k / top-p truncation: rows of top-k (ids, full-vocabulary probabilities), k <= 64 ->
// kept ids (-1 elsewhere) and renormalised probabilities
// top-p sets over whole rows: row i of logits [rows, V] (z / T with T = 1 / inv_temp) with its
// statistics at index j = (i / per) * nrow + off + i % per of st_max (row max of z / T, stride
// st_stride); the set goes to out[j]
void launch_nucleus(int rows, int V, const float* logits, int per, int nrow, int off, const float* st_max,
                    int st_stride, float inv_temp, float top_p, Nucleus* out, hipStream_t s);
// draft draws from the top-p sets of rows [rows = n_req * K] (Philox as launch_sample)
void launch_nucleus_sample(int rows, int K, int V, const int32_t* slots, uint64_t seed, uint64_t step,
                           float inv_temp, const float* logits, const float* row_max, const Nucleus* nuc,
                           int32_t* draft_ids, hipStream_t s);
void launch_trunc_rows(int rows, int k, float top_p, const int32_t* ids_in, const float* probs_in,
                       int32_t* ids_out, float* probs_out, hipStream_t s);
// draft tokens drawn from truncated rows (row j of request r: Philox(seed; j+1, slot, step, 0))
void launch_sparse_sample(int rows, int K, int k, const int32_t* slots, uint64_t seed, uint64_t step,
                          const int32_t* ids, const float* probs, int32_t* draft_ids, hipStream_t s);
// rejection with sparse p rows [n][K+1][kp] and q rows [n][K][kq]
void launch_verify_sparse(int n_req, int K, int kp, int kq, const int32_t* slots, const int32_t* draft_ids,
                          const int32_t* p_ids, const float* p_probs, const int32_t* q_ids, const float* q_probs,
                          uint64_t seed, uint64_t step, int32_t* out_tokens, int32_t* out_len, int32_t* accept_len,
                          int32_t* next_anchor, int32_t* err, hipStream_t s);
// fp32 copy of n 16-bit (fp16) or fp32 values
void launch_to_f32(int dtype, int64_t n, const void* src, float* dst, hipStream_t s);
// n fp32 values rounded to the activation type (fp16 for a bf16 drafter)
void launch_from_f32(int dtype, int64_t n, const float* src, void* dst, hipStream_t s);
// stats [n_req * (2K+1) * 2], acc [n_req], chunks [2 * n_req * draw_chunks(V)] floats
void launch_verify_rejection(int n_req, int K, int V, const int32_t* slots, const int32_t* draft_ids,
                             const float* draft_logits, const float* target, float inv_temp, uint64_t seed,
                             uint64_t step, float* stats, int32_t* acc, float* chunks, int32_t* out_tokens,
                             int32_t* out_len, int32_t* accept_len, int32_t* next_anchor, int32_t* err,
                             hipStream_t s, Nucleus* nuc = nullptr, float top_p = 1.f);
// out[i] = in[i] if in [0, max_batch) else max_batch (a spare empty slot), flagging the error word
void launch_sanitize_slots(int n, const int32_t* in, int32_t* out, int max_batch, int32_t* err, hipStream_t s);
void launch_synth_target(int n_req, int K, int V, const float* draft_logits, float sigma, uint64_t seed,
                         uint64_t step, float* out, hipStream_t s);
void launch_copy_cache(int dtype, const void* cache_k, const void* cache_v, int layer, int slot, int start, int n,
                       int max_batch, int n_kv, int d, int64_t ctx_alloc, const KvPages& pages, void* k_out,
                       void* v_out, hipStream_t s);
// paged cache: flags ERR_PAGE when a request's context occupies an unmapped page
void launch_page_check(int n_req, const int32_t* slots, const int32_t* ctx_len, int max_batch, const KvPages& pages,
                       int32_t* err, hipStream_t s);
void launch_reset_slots(int n, const int32_t* slots, int32_t* ctx_len, int max_batch, int32_t* err, hipStream_t s);
// bf16 drafter weights: *out = max over w of the fp32 bit pattern of |w| (atomic max;
// *out must start at 0), and out = fp16(w * scale)
void launch_absmax_bf16(const void* w, int64_t n, uint32_t* out, hipStream_t s);
void launch_convert_bf16_f16(const void* w, int64_t n, float scale, void* out, hipStream_t s);
void launch_absmax_f32(const float* w, int64_t n, uint32_t* out, hipStream_t s);
void launch_convert_f32_f16(const float* w, int64_t n, float scale, void* out, hipStream_t s);
// C [Rn, J] = A [Rn, Kn] . B [Kn, J] in fp32 (weights in the model dtype; create-time products)
void launch_matmul_nn(int dtype, int Rn, int J, int Kn, const void* A, const void* B, float* C, hipStream_t s);
void launch_philox_fill(int n, uint64_t seed, uint32_t slot, uint64_t step, uint32_t purpose, float* out,
                        hipStream_t s);

}  // namespace dfl
