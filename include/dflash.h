/*
 * dflash.h -- C ABI of the MI355X (gfx950) DFlash drafter hot path.
 *
 * The library implements the three steps of block-diffusion speculative
 * drafting with target-feature KV injection, as the following public pages
 * describe them (cited by key throughout the sources):
 *
 *   [P1] "LLM的推理加速-DFlash" (wnma3mz.github.io blog)
 *   [P2] "一次前向，白赚 4 个 token：DFlash 2 块扩散投机解码技术详解" (forceinjection.github.io)
 *   [P3] "DFlash：块扩散 + KV 注入，让投机解码的草稿不再串行" (rainlin-top.pages.dev)
 *   [P4] "【大模型】DFlash：把串行 Draft 变成并行“填空”" (developer.horizon.auto)
 *   [P5] "DDTree 深度解析:从 Block Diffusion 到 Diffusion Draft Tree" (zhichai.net)
 *
 * Conventions shared by every call:
 *  - Pointers documented "device" are HIP device memory (hipMalloc'ed or a
 *    torch CUDA tensor's data_ptr()); "host" pointers are ordinary memory.
 *  - `stream` is a hipStream_t passed as void* (NULL = the default stream).
 *    Every call only enqueues work on `stream` and returns; none synchronises
 *    except dflash_get_error and dflash_destroy.  Calls on one handle must be
 *    ordered on one stream; a handle is not thread-safe.
 *  - Host-side argument validation runs before anything is enqueued; on a
 *    negative return value nothing was enqueued.
 *  - Conditions only the device can see (a slot whose context would overflow,
 *    an out-of-range slot or token id) never fault: the affected request is
 *    skipped or clamped and a bit is OR-ed into the handle's sticky error
 *    word, read (and cleared) by dflash_get_error.
 *  - Weights are borrowed: the caller keeps them alive and unchanged for the
 *    handle's lifetime.  The handle owns the drafter KV cache, the per-slot
 *    context lengths and all scratch memory (allocated in dflash_create), and
 *    for a bf16 drafter its own fp16 copies of the weight matrices (below).
 *  - Element types.  cfg.dtype = DFLASH_F32: weights, target hidden states,
 *    activations and KV cache are fp32.  cfg.dtype = DFLASH_BF16: weights and
 *    target hidden states are bf16; every matrix product except the fc takes
 *    fp16 operands with fp32 accumulation, so dflash_create converts q/k/v/o/
 *    gate/up/down of every layer and the LM head once into fp16 copies, each
 *    group of matrices that one product reads scaled by its own power of two
 *    (exact for every weight of at least 2^-28 times the group's largest |w|;
 *    the products are scaled back exactly), and the KV cache and
 *    activations are fp16.  The fc product multiplies the given bf16 operands.
 *    The residual stream is fp32 in both.  Logits, probabilities and
 *    statistics are fp32; token ids, lengths and tree indices are int32.
 */
#ifndef DFLASH_H
#define DFLASH_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum dflash_status {
  DFLASH_OK = 0,
  DFLASH_E_INVALID = -1,     /* bad argument (null pointer, size out of range)            */
  DFLASH_E_NOMEM = -2,       /* device allocation failed in dflash_create                  */
  DFLASH_E_CAPACITY = -3,    /* request exceeds a limit fixed in dflash_config             */
  DFLASH_E_UNSUPPORTED = -4, /* shape the kernels do not handle (see dflash_create)        */
  DFLASH_E_HIP = -5          /* a HIP runtime call failed                                  */
};

enum dflash_dtype { DFLASH_F32 = 0, DFLASH_BF16 = 1 };

/* Device error word bits (dflash_get_error). */
enum dflash_device_error {
  DFLASH_DEV_CAPACITY = 1,   /* an injection would exceed max_ctx: that request's rows were skipped */
  DFLASH_DEV_BAD_SLOT = 2,   /* a slot id outside [0, max_batch): that request was skipped          */
  DFLASH_DEV_ROWS = 4,       /* row counts negative or above rows_upper_bound: rows skipped         */
  DFLASH_DEV_BAD_TOKEN = 8,  /* an anchor id outside [0, vocab): id 0 was embedded instead          */
  DFLASH_DEV_PAGE = 16,      /* paged cache: a position maps to an unmapped page (table entry outside
                                [0, num_pages)): injected rows there were skipped; a draft reading
                                such a page read page 0 instead (its outputs are not meaningful)     */
  DFLASH_DEV_NONFINITE = 32  /* bf16 drafter: a value stored in 16 bits (SwiGLU output, q/k/v of the
                                block, K/V written to the cache) was beyond fp16's largest finite
                                magnitude 65504, or NaN: it was stored saturated to +-65504 (NaN as
                                NaN), so later kernels stay finite, and the results that depend on
                                it are not meaningful                                               */
};

/* Model shape, numerics and capacity, fixed at create time.
 * Drafter: Qwen3-style decoder layers (GQA attention with per-head q/k
 * RMSNorm and RoPE, SwiGLU MLP), fed by context K/V projected from the
 * hidden states of n_target_layers target layers [P1 "关键创新"; P2 §2.2]. */
typedef struct dflash_config {
  int32_t dtype;              /* DFLASH_F32 or DFLASH_BF16                                      */
  int32_t n_layers;           /* drafter decoder layers L_d (1..64)                             */
  int32_t hidden;             /* H, multiple of 128                                              */
  int32_t n_q_heads;          /* multiple of n_kv_heads                                           */
  int32_t n_kv_heads;
  int32_t head_dim;           /* d: 64 or 128                                                     */
  int32_t ffn;                /* SwiGLU width F, multiple of 64                                   */
  int32_t vocab;              /* V (shared embedding and LM head rows)                            */
  int32_t n_target_layers;    /* L_t (1..8): hidden states concatenated in ascending layer order */
  int32_t target_hidden;      /* H_t, multiple of 64                                              */
  int32_t mask_token_id;      /* id embedded at the K mask positions [P2 §2.1; P4 §5.2]          */
  float rms_eps;              /* RMSNorm epsilon (e.g. 1e-6)                                      */
  float rope_theta;           /* RoPE base (rotate-half pairing (i, i + d/2))                     */
  float input_embedding_scale;/* multiplies the shared embedding of the block [P2 §2.2]          */
  float output_multiplier;    /* logits *= output_multiplier (1 = off) [P2 §2.2]                  */
  float logit_softcap;        /* > 0: logits = c * tanh(logits / c); 0 = off [P2 §2.2]             */
  int32_t max_batch;          /* number of request slots                                          */
  int32_t max_ctx;            /* context positions per slot                                        */
  int32_t max_k;              /* largest K (masks per block), 1..31                                */
  int32_t max_inject_rows;    /* largest rows_upper_bound accepted by dflash_inject_context       */
  int32_t max_top_k;          /* largest top_k of dflash_draft_block (0..256)                      */
  int32_t max_tree;           /* largest tree_budget (0..256)                                      */
  /* DFlash 2 modules [P2 §3.1-3.2]; all zero = DFlash 1. */
  int32_t conv_group;         /* > 0: each layer applies two-tap dynamic depthwise convolutions to its
                                 attention and MLP sub-layer inputs; channels per kernel-correction
                                 group (a multiple of 4 dividing hidden, 2*hidden/conv_group a multiple
                                 of 8); 0 = off                                                        */
  int32_t sel_rank;           /* > 0: path selector with codebooks of this rank (1..4096); 0 = off   */
  int32_t sel_cands;          /* selector candidates per position (1..64, <= vocab) when sel_rank > 0 */
  int32_t causal_block;       /* 1: block row j attends to the context and to block rows 0..j only
                                 (the pages differ on the block-internal mask [P2 §2.2 vs P4 §5.3]);
                                 0: no mask inside the block (default)                               */
  /* Paged KV cache (engine integration [P3 §4]); page_size 0 = one contiguous region per slot. */
  int32_t page_size;          /* positions per page: 0, or a multiple of 32 up to 8192; a page holds
                                 those positions of one sequence for every layer and kv head        */
  int32_t num_pages;          /* pages in the handle's pool when page_size > 0 (>= 1)                */
} dflash_config;

/* Per-layer weights, all [out_features, in_features] row-major, cfg.dtype.
 * Matrices and norm gains are read at create time (a bf16 drafter converts the
 * matrices into its own fp16 copies then); the gains, embedding and fc are
 * read again on every call. */
typedef struct dflash_layer_weights {
  const void* in_norm;        /* [H]          pre-attention RMSNorm gain          */
  const void* q_w;            /* [n_q*d, H]                                       */
  const void* k_w;            /* [n_kv*d, H]  used for block rows and context     */
  const void* v_w;            /* [n_kv*d, H]  used for block rows and context     */
  const void* o_w;            /* [H, n_q*d]                                       */
  const void* q_norm;         /* [d]          per-head RMSNorm gain of q          */
  const void* k_norm;         /* [d]          per-head RMSNorm gain of k          */
  const void* post_norm;      /* [H]          pre-MLP RMSNorm gain                */
  const void* gate_w;         /* [F, H]                                           */
  const void* up_w;           /* [F, H]                                           */
  const void* down_w;         /* [H, F]                                           */
  /* DFlash 2 dynamic convolutions (read when cfg.conv_group > 0, else ignored) [P2 §3.2.3]:
   * y_t = k_t0 * x_t + k_t1 * x_{t-1} over the block rows (x_{-1} = 0), with
   * k_tj[c] = base[j][c] + (x_t . proj^T)[j * H/G + c/G], x being the
   * convolution's own input.  One convolution before and one after each
   * sub-layer: attn_* acts on the RMS-normalised input of q/k/v, mlp_* on that
   * of gate/up (both required); attn_conv_post_* on the attention output (after
   * o, before the residual add), mlp_conv_post_* on the MLP output (after down,
   * before the residual add) -- each post pair optional (both pointers, or
   * neither). */
  const void* attn_conv_base; /* [2, H]        per-channel kernels of the two taps (current, previous) */
  const void* attn_conv_proj; /* [2*H/G, H]    kernel corrections: rows [0,H/G) tap 0, [H/G,2H/G) tap 1 */
  const void* mlp_conv_base;  /* [2, H]                                           */
  const void* mlp_conv_proj;  /* [2*H/G, H]                                       */
  const void* attn_conv_post_base;  /* [2, H]      or NULL                        */
  const void* attn_conv_post_proj;  /* [2*H/G, H]  or NULL                        */
  const void* mlp_conv_post_base;   /* [2, H]      or NULL                        */
  const void* mlp_conv_post_proj;   /* [2*H/G, H]  or NULL                        */
} dflash_layer_weights;

typedef struct dflash_weights {
  const void* embed;          /* [V, H] shared with the target [P1 "架构设计"]   */
  const void* lm_head;        /* [V, H] shared with the target                   */
  const void* fc;             /* [H, L_t*H_t] fusion of the target features      */
  const void* hidden_norm;    /* [H] RMSNorm gain after fc                        */
  const void* final_norm;     /* [H] RMSNorm gain before the LM head              */
  int32_t n_layers;           /* must equal cfg.n_layers                          */
  const dflash_layer_weights* layers; /* host array [n_layers] of device pointers */
  /* DFlash 2 path selector (read when cfg.sel_rank > 0) [P2 §3.1.2]:
   * S_t(a, b) = z_t(b) + <A(a) * (W_H h_t), B(b)>. */
  const void* sel_pred;       /* [V, rank] predecessor codebook A                 */
  const void* sel_succ;       /* [V, rank] successor codebook B                   */
  const void* sel_hidden;     /* [rank, H] W_H, applied to the final-normalised hidden state */
  const void* mask_embedding; /* [H] or NULL: trained vector embedded at the mask positions in place of
                                 the embedding row of mask_token_id (times input_embedding_scale) [P4 §5.2] */
} dflash_weights;

typedef struct dflash_handle dflash_handle;

/* Create a handle: validates the shapes, allocates and zeroes the KV cache
 * (n_layers x max_batch x n_kv_heads x max_ctx positions of K and V), the
 * per-slot context lengths and the scratch memory, and (bf16 drafter) makes the
 * fp16 weight copies; synchronises the device.  Returns DFLASH_OK and *out, or
 * a negative status (nothing allocated): DFLASH_E_INVALID also when a weight
 * matrix holds Inf or NaN. */
int dflash_create(const dflash_config* cfg, const dflash_weights* w, dflash_handle** out);

/* Synchronises the device and frees everything the handle owns. */
int dflash_destroy(dflash_handle* h);

/* Set the context length of the n slots in slots_dev (device int32[n]) to 0. */
int dflash_reset_slots(dflash_handle* h, void* stream, int32_t n, const int32_t* slots_dev);

/* Context injection [P1 "关键创新" Steps 1-3; P2 §2.2; P3 §四; P4 §5.1, §5.6].
 * For request r (0 <= r < n_req) take row_count[r] rows starting at row
 * row_start[r] of every target-layer buffer, concatenate the layers (ascending
 * order of target_hidden[]), project with fc, RMSNorm (hidden_norm), then for
 * every drafter layer project with k_w / v_w, RMSNorm each k head (k_norm),
 * rotate k with RoPE at positions ctx_len[slot]..ctx_len[slot]+count-1, and
 * write K and V into the slot's cache; ctx_len[slot] += count.
 *   slots, row_start, row_count : device int32[n_req]; slots may repeat (rows append in order)
 *   rows_upper_bound            : host bound >= sum(row_count), <= cfg.max_inject_rows
 *   target_hidden               : host array [n_target_layers] of device pointers; layer l's
 *                                 rows are target_hidden[l] + row * row_stride (elements)
 *   row_stride                  : elements between rows (>= target_hidden, multiple of 8) */
int dflash_inject_context(dflash_handle* h, void* stream, int32_t n_req, const int32_t* slots,
                          const int32_t* row_start, const int32_t* row_count, int64_t rows_upper_bound,
                          const void* const* target_hidden, int64_t row_stride);

/* Per-call parameters of a draft. */
typedef struct dflash_draft_params {
  int32_t K;                  /* masks per block, 1..max_k; the block has K+1 rows [P4 §4]   */
  float temperature;          /* 0: greedy argmax; > 0: sample from softmax(z / T)           */
  uint64_t seed;              /* Philox4x32-10 key                                           */
  uint64_t step;              /* Philox counter word (low 32 bits used)                      */
  int32_t top_k;              /* 0 or 1..max_top_k: report the top_k tokens per position     */
  int32_t tree_budget;        /* 0 or 1..max_tree: build a best-first prefix tree [P5 §2.3]  */
} dflash_draft_params;

/* Outputs of a draft (device pointers; NULL where optional). */
typedef struct dflash_draft_outputs {
  int32_t* draft_ids;         /* [n_req, K] required: d_1..d_K                                  */
  int32_t* topk_ids;          /* [n_req, K, top_k]   if top_k > 0: logit desc, ties lower id    */
  float* topk_probs;          /* [n_req, K, top_k]   full-vocabulary softmax(z/T') probability  */
  float* row_max;             /* [n_req, K] or NULL  max of z/T'                                 */
  float* row_lse;             /* [n_req, K] or NULL  log sum exp(z/T' - row_max)                 */
  float* logits;              /* [n_req, K, V] or NULL: z (after output_multiplier / softcap)    */
  int32_t* tree_tokens;       /* [n_req, B+1] if tree_budget = B > 0; node 0 = anchor            */
  int32_t* tree_parents;      /* [n_req, B+1] parent node index (-1 for the root / unused)       */
  int32_t* tree_depth;        /* [n_req, B+1] depth (root 0; -1 unused)                           */
  uint64_t* tree_mask;        /* [n_req, B+1, ceil((B+1)/64)] bit j of row i: i may attend to j  */
  /* selector (cfg.sel_rank > 0): the walk's candidates and its distribution over them */
  int32_t* cand_ids;          /* [n_req, K, sel_cands] or NULL: top-sel_cands ids (logit desc, id asc) */
  float* cand_probs;          /* [n_req, K, sel_cands] or NULL: softmax(S/T) (one-hot when T = 0)       */
  float* hidden;              /* [n_req, K, H] or NULL: final-normalised hidden rows of the masks (fp32) */
} dflash_draft_outputs;
/* T' = temperature if > 0, else 1.  A tree needs top_k >= min(B, V). */

/* One drafter forward over the block [anchor | mask x K] of each request
 * [P2 §2.1-2.2; P4 §4-4.4]: embedding x input_embedding_scale at positions
 * C..C+K (C = ctx_len[slot]), n_layers decoder layers whose queries attend to
 * the slot's context K/V plus the block's own K/V with no mask inside the
 * block [P4 §5.3], final RMSNorm, LM head on the K mask rows, per-position
 * softmax, top-k, draft tokens (argmax, or inverse-CDF sampling with
 * u = Philox(seed; position j, slot, step, 0)), and optionally the prefix tree
 * and its ancestor-only mask [P5 §2.3, §3.3].  Does not modify the cache.
 *   slots, anchor_ids : device int32[n_req] (distinct slots in [0, max_batch)) */
int dflash_draft_block(dflash_handle* h, void* stream, int32_t n_req, const int32_t* slots,
                       const int32_t* anchor_ids, const dflash_draft_params* params,
                       const dflash_draft_outputs* out);

/* With cfg.sel_rank > 0, dflash_draft_block's draft tokens come from the DFlash 2
 * path selector [P2 §3.1.2-3.1.3]: per mask position t (0-based) the top
 * sel_cands ids of the logits are the candidates, scored S_t(a, b) = z_t(b) +
 * <A(a) * (W_H h_t), B(b)> with a the anchor (t = 0) or the token picked at t-1
 * and h_t the final-normalised hidden row; temperature 0 picks the best score
 * (lowest id on ties), T > 0 draws from softmax(S/T) over the candidates by
 * inverse CDF in candidate order with u = Philox(seed; t+1, slot, step, 0).
 * cand_ids / cand_probs then feed dflash_verify_subset. */

/* The selection stage of dflash_draft_block alone, from caller logits
 * [n_req, K, V] (device fp32): row statistics, top-k, draft tokens, tree. */
int dflash_select_from_logits(dflash_handle* h, void* stream, int32_t n_req, const int32_t* slots,
                              const int32_t* anchor_ids, const float* logits,
                              const dflash_draft_params* params, const dflash_draft_outputs* out);

/* The DFlash 2 path selector alone, from caller logits [n_req, K, V] and
 * final-normalised hidden rows [n_req, K, H] (device fp32; a bf16 drafter rounds
 * the hidden rows to fp16 before the W_H product): writes draft_ids [n_req, K],
 * cand_ids and cand_probs [n_req, K, sel_cands].  Needs cfg.sel_rank > 0
 * (else DFLASH_E_INVALID). */
int dflash_select_path(dflash_handle* h, void* stream, int32_t n_req, int32_t K, const int32_t* slots,
                       const int32_t* anchor_ids, const float* logits, const float* hidden, float temperature,
                       uint64_t seed, uint64_t step, int32_t* draft_ids, int32_t* cand_ids, float* cand_probs);

/* Paged KV cache [P3 §4: the drafter's cache managed by the serving engine's
 * pages]: table is a device array [max_batch][pages_per_slot] of int32 page ids
 * (pages_per_slot = ceil(max_ctx / page_size)); entry (s, p) holds positions
 * [p * page_size, (p+1) * page_size) of slot s.  Borrowed: the caller owns it,
 * keeps it alive and may rewrite entries between calls (stream-ordered); -1 or
 * any id outside [0, num_pages) = unmapped (see DFLASH_DEV_PAGE).  Pages may be
 * shared between slots only for positions both hold identically (a common
 * prefix); injecting into a shared page overwrites it for both.  Required
 * before any call that reads or writes the cache of a paged handle
 * (DFLASH_E_INVALID otherwise); DFLASH_E_UNSUPPORTED on a contiguous handle. */
int dflash_set_page_table(dflash_handle* h, const int32_t* table);

/* Symmetric sampling truncation [P2 §3.3]: from this call on, every draw at
 * temperature > 0 uses distributions cut to their top_k ids (probability
 * descending, id ascending), renormalised, then to the shortest prefix of that
 * order whose cumulative probability reaches top_p (the crossing id kept), and
 * renormalised: the draft's sampling (not the selector's walk), and in
 * dflash_verify both p and q, in dflash_verify_subset p.  Truncated draws are
 * inverse CDFs in ascending id order.  top_k 0 = off (the default); 1..64;
 * top_p in (0, 1] (1 = off).  top_p < 1 with top_k 0 cuts the whole row:
 * the set is the shortest prefix of the full probability-descending order
 * (ties: ascending id) that reaches top_p, found by a radix select over the
 * row, and draws and verification run over the full vocabulary with the ids
 * outside it at probability 0 (needs vocab <= 2^21, else DFLASH_E_CAPACITY). */
int dflash_set_sampling(dflash_handle* h, int32_t top_k, float top_p);

/* Verification of one drafted block per request [P2 §2.3, §4.2; P1 "验证"].
 * target_logits [n_req, K+1, V]: row j is the target's distribution after
 * the anchor and d_1..d_j.  temperature 0: greedy prefix match, emitting
 * d_1..d_a and the target's argmax of row a.  temperature > 0: rejection
 * sampling against draft_logits [n_req, K, V] (row i-1 for d_i) with accept
 * uniforms Philox(seed; i, slot, step, 1) and a residual / bonus draw with
 * Philox(seed; a+1, slot, step, 2); an exhausted residual (mass < 2^-20)
 * falls back to p.  Outputs (device): out_tokens [n_req, K+1] (unused -1),
 * out_len [n_req] = a+1, accept_len [n_req] = a.  Does not touch the cache:
 * inject the a+1 committed rows next (row_count = out_len on the device).
 * temperature > 0 needs vocab <= 2^21 (DFLASH_E_CAPACITY otherwise: the draw
 * keeps one float per 256 ids in LDS); draft_logits and slots must be given. */
int dflash_verify(dflash_handle* h, void* stream, int32_t n_req, int32_t K, const int32_t* slots,
                  const int32_t* draft_ids, const float* draft_logits, const float* target_logits,
                  float temperature, uint64_t seed, uint64_t step, int32_t* out_tokens, int32_t* out_len,
                  int32_t* accept_len, int32_t* next_anchor);
/* next_anchor [n_req] (device, or NULL) receives out_tokens[r][out_len[r]-1]: the
 * token that anchors the next block [P4 §4.2; P1 "核心推理伪代码"]. */

/* For callers that cannot allocate device memory (code under HIP graph capture,
 * serving loops or harnesses that forbid hipMalloc): the verification of
 * dflash_verify without a handle.  Same arguments, outputs, Philox streams and
 * results as dflash_verify on a handle of this vocabulary, except: the
 * vocabulary is passed here; no top-k / top-p truncation (as after
 * dflash_set_sampling(h, 0, 1)); draft ids outside [0, vocab) are rejected
 * without an error bit (there is no error word).  Its scratch (about 2.3 MB)
 * is one static array per GPU, resolved on the first call on each device and
 * kept until the process ends; nothing is allocated.  Limits: n_req <= 256,
 * 1 <= K <= 31, vocab <= 262144 (DFLASH_E_CAPACITY beyond).  Every call on a
 * GPU uses that GPU's one array: calls that may overlap on one GPU (different
 * streams without ordering) race and must not be made. */
int dflash_verify_noalloc(void* stream, int32_t n_req, int32_t K, int32_t vocab, const int32_t* slots,
                          const int32_t* draft_ids, const float* draft_logits, const float* target_logits,
                          float temperature, uint64_t seed, uint64_t step, int32_t* out_tokens, int32_t* out_len,
                          int32_t* accept_len, int32_t* next_anchor);

/* Rejection verification of a selector draft [P2 §3.1.3, §4.2]: the drafter's
 * distribution at position i is given over C candidates (cand_ids / cand_probs
 * [n_req, K, C], device; C <= 64), projected onto token ids (q_full(v) = summed
 * probability of the candidates with id v, 0 elsewhere); accept d_i iff
 * u * q_full(d_i) < p_{i-1}(d_i) with u = Philox(seed; i, slot, step, 1); at the
 * first rejection draw from max(0, p - q_full) renormalised (from p when that
 * mass is below 2^-20) with Philox(seed; i, slot, step, 2); after K acceptances
 * the bonus from p_K.  temperature 0: the greedy prefix match of dflash_verify.
 * Outputs and the vocabulary limit as dflash_verify. */
int dflash_verify_subset(dflash_handle* h, void* stream, int32_t n_req, int32_t K, int32_t C, const int32_t* slots,
                         const int32_t* draft_ids, const int32_t* cand_ids, const float* cand_probs,
                         const float* target_logits, float temperature, uint64_t seed, uint64_t step,
                         int32_t* out_tokens, int32_t* out_len, int32_t* accept_len, int32_t* next_anchor);

/* Verifier walk down a draft tree [P5 §3.5] (one
 * tree per request, as dflash_draft_block builds it: node 0 = root / anchor,
 * siblings carrying distinct tokens).  From the root, the target's own decoding rule picks the
 * next token from target_logits row u (the target's distribution after the
 * path root..u, i.e. the tree evaluated under its ancestor-only mask
 * [P5 §3.3]); the walk moves to the child of u carrying that token, if any, and
 * otherwise stops with the pick as the new bonus token.  temperature 0: row
 * argmax (lowest id on ties); > 0: inverse-CDF draw from softmax(t_u / T) in
 * ascending id order with u = Philox(seed; depth(u) + 1, slot, step, 4).
 *   n_nodes        : B + 1 (1 .. cfg.max_tree + 1); K: the draft's K (tree depth <= K)
 *   tree_tokens, tree_parents : device int32 [n_req, n_nodes] (parent -1: root or unused)
 *   target_logits  : device fp32 [n_req, n_nodes, V]
 * Outputs (device): out_tokens [n_req, K+1] (accepted tokens, then the bonus;
 * unused -1), out_len [n_req] = a + 1, accept_len [n_req] = a, next_anchor
 * [n_req] (or NULL) = the bonus, path_nodes [n_req, K+1] (or NULL) = node
 * indices of the accepted path, root first (unused -1).  A walk deeper than K
 * stops there and sets DFLASH_DEV_ROWS in the error word.  Only the rows of
 * the visited nodes are read (one work-group per request).  temperature > 0
 * needs V <= 2^21 (else DFLASH_E_CAPACITY).
 * Does not touch the cache: inject the path's a + 1 rows next
 * (dflash_inject_tree_path with path_len = out_len). */
int dflash_verify_tree(dflash_handle* h, void* stream, int32_t n_req, int32_t K, int32_t n_nodes,
                       const int32_t* slots, const int32_t* tree_tokens, const int32_t* tree_parents,
                       const float* target_logits, float temperature, uint64_t seed, uint64_t step,
                       int32_t* out_tokens, int32_t* out_len, int32_t* accept_len, int32_t* next_anchor,
                       int32_t* path_nodes);

/* Injection of the rows of an accepted tree path [P5 §3.4-3.5; P3 §四]: the
 * same computation as dflash_inject_context, with request r's i-th new row
 * (i < path_len[r]) read from row r * tree_stride + path_nodes[r * max_path + i]
 * of target_hidden (the target's hidden states in tree order, tree_stride rows
 * per request).  A node index outside [0, tree_stride) sets DFLASH_DEV_ROWS in
 * the error word and leaves that row's cache entry unwritten (the slot's
 * context length still advances by path_len, as for any injected row).
 *   path_nodes : device int32 [n_req, max_path]; path_len: device int32 [n_req]
 *   rows_upper_bound : host bound >= sum(path_len), <= cfg.max_inject_rows */
int dflash_inject_tree_path(dflash_handle* h, void* stream, int32_t n_req, const int32_t* slots,
                            const int32_t* path_nodes, const int32_t* path_len, int32_t max_path,
                            int32_t tree_stride, int64_t rows_upper_bound, const void* const* target_hidden,
                            int64_t row_stride);

/* Synchronise `stream`, return the sticky device error word in *code and clear it. */
int dflash_get_error(dflash_handle* h, void* stream, int32_t* code);

/* Human-readable name of a status code. */
const char* dflash_status_str(int status);

/* ---- inspection and benchmark helpers (not part of the drafting path) ---- */

/* Per-phase timing: when enabled, HIP events are recorded on the call's
 * stream around each group of kernels below; dflash_profile_read synchronises,
 * writes the accumulated milliseconds and launch counts of the first n phases
 * since the last read (host arrays, either may be NULL) and resets them. */
enum dflash_phase {
  DFLASH_PH_INJECT_PREP = 0, /* row tables                                  */
  DFLASH_PH_INJECT_FC,       /* fc GEMM over the concatenated target layers */
  DFLASH_PH_INJECT_NORM,     /* RMSNorm of the fused feature               */
  DFLASH_PH_INJECT_KV,       /* per-layer K|V GEMM + k-norm/RoPE/cache store */
  DFLASH_PH_EMBED,           /* block embedding + first RMSNorm             */
  DFLASH_PH_QKV,             /* q|k|v GEMM + head norm + RoPE               */
  DFLASH_PH_ATTN,            /* block attention kernel                      */
  DFLASH_PH_ATTN_COMBINE,    /* merge of context chunks                     */
  DFLASH_PH_O,               /* output projection + residual                */
  DFLASH_PH_NORM,            /* RMSNorms between sub-layers                 */
  DFLASH_PH_GATE_UP,         /* gate|up GEMM + SwiGLU                       */
  DFLASH_PH_DOWN,            /* down GEMM + residual                        */
  DFLASH_PH_LM_HEAD,         /* LM-head GEMM + tile statistics              */
  DFLASH_PH_SELECT,          /* row statistics, sampling, top-k, tree       */
  DFLASH_PH_VERIFY,          /* verification                                */
  DFLASH_PH_ATTN_PLAN,       /* context-chunk work list of the attention    */
  DFLASH_PH_CONV,            /* DFlash 2 kernel-correction GEMMs + dynamic convolutions */
  DFLASH_PH_SELECTOR,        /* DFlash 2 candidates, W_H product and walk   */
  DFLASH_PH_COUNT
};
int dflash_profile(dflash_handle* h, int32_t enable);
int dflash_profile_read(dflash_handle* h, int32_t n, double* ms, int32_t* launches);

/* Copy ctx_len[0..max_batch) to device int32 buffer out_dev. */
int dflash_ctx_lens(dflash_handle* h, void* stream, int32_t* out_dev);

/* Copy cache positions [start, start+n) of (layer, slot) as K and V, each
 * [n, n_kv_heads, head_dim] in the cache element type (fp32, or fp16 for a
 * bf16 drafter), to device buffers k_out / v_out.  Paged cache: positions in
 * unmapped pages read as 0. */
int dflash_copy_cache(dflash_handle* h, void* stream, int32_t layer, int32_t slot, int32_t start, int32_t n,
                      void* k_out, void* v_out);

/* Synthetic target logits for benchmarks and tests (a stand-in for the target
 * model): out[r, j] = draft_logits[r, j] + sigma * N(0,1) for j < K and
 * out[r, K] = sigma * N(0,1), normals from Philox (purpose 3) + Box-Muller. */
int dflash_synth_target_logits(void* stream, int32_t n_req, int32_t K, int32_t vocab, const float* draft_logits,
                               float sigma, uint64_t seed, uint64_t step, float* out);

/* out[i] = Philox uniform (seed; position i, slot, step, purpose), i < n (device fp32). */
int dflash_philox_uniforms(void* stream, int32_t n, uint64_t seed, uint32_t slot, uint64_t step, uint32_t purpose,
                           float* out);

#ifdef __cplusplus
}
#endif
#endif /* DFLASH_H */
