// Host library: handle, validation, scratch ownership and the launch sequence
// of the three drafting calls.  No host synchronisation on the drafting path;
// every device-dependent size is bounded on the host and resolved on the device.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstring>
#include <vector>

#include "../../include/dflash.h"
#include "ops.h"

using namespace dfl;

struct dflash_handle {
  dflash_config cfg{};
  int esize = 4;
  int device = 0, num_cus = 256;
  // borrowed weights
  const void* sel_hidden_src = nullptr;   // caller's W_H
  const void* mask_emb = nullptr;         // caller's mask-embedding override (or null)
  const void *embed = nullptr, *lm_head = nullptr, *fc = nullptr, *hidden_norm = nullptr, *final_norm = nullptr;
  std::vector<dflash_layer_weights> layers;
  // matrices as the products read them: the caller's (fp32 drafter) or the
  // handle's fp16 copies, each group of them scaled by its own power of two (bf16 drafter)
  // s_*: 2^-(the copy's scale exponent), multiplied into every product that reads the copy
  struct Mats {
    const void *q, *k, *v, *o, *gate, *up, *down, *conv_a, *conv_m;
    // after-sub-layer convolutions (or null): their corrections o . P^T are taken
    // as A . (P . W)^T, the product's extra output columns, so what is kept is
    // P . W_o [2H/G, q_dim] and P . W_down [2H/G, ffn] (scaled with o / down)
    const void *conv_ap = nullptr, *conv_mp = nullptr;
    float s_o = 1.f, s_gu = 1.f, s_down = 1.f, s_ca = 1.f, s_cm = 1.f;
  };
  std::vector<Mats> mats;
  const void* lm = nullptr;
  int op = OP_F32, op_fc = OP_F32;  // operand type of the products / of the fc product
  // scales shared across layers: q | k | v of every layer (the draft reads one layer's q | k | v in
  // one product, the injection every layer's k | v), the LM head, the selector's W_H
  float s_qkv = 1.f, s_lm = 1.f, s_selh = 1.f;
  const void** d_k_gains = nullptr;       // device array of per-layer k_norm pointers
  // cache and state
  void* cache_k = nullptr;
  void* cache_v = nullptr;
  int64_t ctx_alloc = 0;
  // paged cache (cfg.page_size > 0): the caller's page table and its geometry
  const int32_t* page_table = nullptr;
  int pages_per_slot = 0;
  int64_t page_elems = 0;   // elements of one page (all layers and kv heads)
  KvPages pages() const {
    KvPages p;
    p.table = cfg.page_size > 0 ? page_table : nullptr;
    p.per_slot = pages_per_slot;
    p.page_size = cfg.page_size;
    p.n_pages = cfg.num_pages;
    p.table_rows = cfg.max_batch;
    p.page_elems = page_elems;
    return p;
  }
  int32_t* ctx_len = nullptr;
  int32_t* err = nullptr;
  float2* rope = nullptr;
  int n_rope = 0;
  // draft scratch
  int maxM = 0, Rpad = 0, QRpad = 0, attn_splits = 1, attn_wg = 0, piece_cap = 0, qrt_max = 5;
  bool attn_waves = false;     // 16-bit K/V: ring work-groups, attn_wg = attn_waves_wg_per_cu() per CU
  float* X = nullptr;
  void *hbuf = nullptr, *attn_out = nullptr, *act = nullptr, *qb = nullptr, *kb = nullptr, *vb = nullptr;
  float *o_part = nullptr, *m_part = nullptr, *l_part = nullptr;
  AttnPlan* plan = nullptr;
  int32_t *seg_start = nullptr, *chunk_base = nullptr;
  int4 *seg_desc = nullptr, *wg_range = nullptr;
  int32_t* dslots = nullptr;              // validated slot ids of the current draft
  float* partials = nullptr;
  size_t partials_elems = 0;
  // LM head
  int n_vtiles = 0, lm_tile = 128;
  float *logits_ws = nullptr, *tmax = nullptr, *tsum = nullptr, *row_max = nullptr, *row_lse = nullptr;
  int32_t* targ = nullptr;
  int32_t* tk_ids = nullptr;
  float* tk_probs = nullptr;
  // injection
  int inject_chunk = 0;
  float* y = nullptr;
  void* g = nullptr;
  int32_t *a_rows = nullptr, *row_slot = nullptr, *row_pos = nullptr, *req_off = nullptr, *req_pos = nullptr;
  // DFlash 2 modules
  void* hbuf2 = nullptr;                  // convolved sub-layer input
  float* obuf = nullptr;                  // fp32 sub-layer output ahead of an after-sub-layer convolution
  float* cbuf = nullptr;                  // kernel corrections [maxM, 2H/G]
  float* rsbuf = nullptr;                 // RMS scales of the rows the last norm pass produced [maxM]
  const void* sel_h = nullptr;            // W_H (fp16 copy for a bf16 drafter)
  const void *sel_pred = nullptr, *sel_succ = nullptr;
  float *sel_gate = nullptr, *sel_cprob = nullptr, *sel_probs_ws = nullptr, *sel_table = nullptr;
  int32_t *sel_cand = nullptr, *sel_ids_ws = nullptr;
  void* sel_hin = nullptr;                // caller hidden rows in the operand type
  // symmetric sampling truncation (dflash_set_sampling)
  int trunc_k = 0;
  float trunc_p = 1.f;
  Nucleus* nuc = nullptr;                 // top-p sets over whole rows (trunc_k 0, trunc_p < 1)
  float *vt_max = nullptr, *vrow_max = nullptr, *vrow_lse = nullptr;   // tile maxima, row max / log-sum
  int32_t *tr_ids = nullptr, *kp_ids = nullptr;
  float *tr_probs = nullptr, *kp_probs = nullptr;
  // verification
  int32_t* post = nullptr;
  float* vstats = nullptr;
  int32_t* vacc = nullptr;     // accepted count per request (T > 0 verification)
  float* vchunks = nullptr;    // chunk sums of p and of the residual
  std::vector<void*> allocs;
  // optional per-phase timing
  struct Mark { int phase; hipEvent_t a, b; };
  bool prof = false;
  std::vector<Mark> marks;
  std::vector<hipEvent_t> event_pool;
};

namespace {

constexpr int kAttnMinGroups = 8;   // fewest 32-key groups per attention work-group range
constexpr int kAttnMinGroupsWave = 2;   // ... per single-wave range (16-bit K/V)
constexpr int kAttnChunkMin = 16;   // chunk of a segment: at least 16 groups (512 keys) ...
constexpr int kAttnChunkMax = 16;   // ... and at most 16 chunks per segment

// Records a pair of HIP events around a group of launches when timing is enabled.
struct Phase {
  dflash_handle* h;
  hipStream_t s;
  int phase;
  hipEvent_t a = nullptr;
  static hipEvent_t take(dflash_handle* h) {
    if (!h->event_pool.empty()) {
      hipEvent_t e = h->event_pool.back();
      h->event_pool.pop_back();
      return e;
    }
    hipEvent_t e = nullptr;
    (void)hipEventCreate(&e);
    return e;
  }
  Phase(dflash_handle* h_, hipStream_t s_, int ph) : h(h_), s(s_), phase(ph) {
    if (h->prof) {
      a = take(h);
      (void)hipEventRecord(a, s);
    }
  }
  ~Phase() {
    if (h->prof) {
      hipEvent_t b = take(h);
      (void)hipEventRecord(b, s);
      h->marks.push_back({phase, a, b});
    }
  }
};

int alloc(dflash_handle* h, void** p, size_t bytes) {
  if (bytes == 0) bytes = 256;
  if (hipMalloc(p, bytes) != hipSuccess) return DFLASH_E_NOMEM;
  h->allocs.push_back(*p);
  if (hipMemset(*p, 0, bytes) != hipSuccess) return DFLASH_E_HIP;
  return DFLASH_OK;
}

template <typename P>
int alloc_t(dflash_handle* h, P** p, size_t count, size_t elem) {
  void* v = nullptr;
  const int rc = alloc(h, &v, count * elem);
  *p = (P*)v;
  return rc;
}

// free one allocation of the handle before destroy (create-time temporaries)
void free_one(dflash_handle* h, void* p) {
  for (size_t i = 0; i < h->allocs.size(); ++i)
    if (h->allocs[i] == p) {
      (void)hipFree(p);
      h->allocs.erase(h->allocs.begin() + i);
      return;
    }
}

void free_all(dflash_handle* h) {
  for (void* p : h->allocs) (void)hipFree(p);
  h->allocs.clear();
}

int check_config(const dflash_config& c) {
  if (c.dtype != DFLASH_F32 && c.dtype != DFLASH_BF16) return DFLASH_E_INVALID;
  if (c.n_layers < 1 || c.n_layers > 64 || c.hidden <= 0 || c.n_q_heads <= 0 || c.n_kv_heads <= 0 ||
      c.ffn <= 0 || c.vocab <= 0 || c.n_target_layers < 1 || c.target_hidden <= 0)
    return DFLASH_E_INVALID;
  if (c.max_batch < 1 || c.max_ctx < 1 || c.max_k < 1 || c.max_inject_rows < 1 || c.max_top_k < 0 ||
      c.max_tree < 0)
    return DFLASH_E_INVALID;
  if (c.mask_token_id < 0 || c.mask_token_id >= c.vocab) return DFLASH_E_INVALID;
  if (!(c.rms_eps > 0.f) || !(c.rope_theta > 0.f)) return DFLASH_E_INVALID;
  if (c.head_dim != 64 && c.head_dim != 128) return DFLASH_E_UNSUPPORTED;
  if (c.n_q_heads % c.n_kv_heads) return DFLASH_E_UNSUPPORTED;
  if (c.hidden % 128 || (c.n_q_heads * c.head_dim) % 128 || (c.n_kv_heads * c.head_dim) % 128)
    return DFLASH_E_UNSUPPORTED;
  if (c.ffn % 64 || c.target_hidden % 64) return DFLASH_E_UNSUPPORTED;
  if (c.n_target_layers > MAX_ASEG) return DFLASH_E_UNSUPPORTED;
  if (c.max_k > 31) return DFLASH_E_UNSUPPORTED;
  if (c.max_top_k > 256 || c.max_tree > 256) return DFLASH_E_UNSUPPORTED;
  if (c.conv_group < 0 || c.sel_rank < 0 || c.causal_block < 0 || c.causal_block > 1) return DFLASH_E_INVALID;
  if (c.page_size < 0 || (c.page_size > 0 && c.num_pages < 1)) return DFLASH_E_INVALID;
  if (c.page_size > 0 && (c.page_size % 32 || c.page_size > 8192)) return DFLASH_E_UNSUPPORTED;
  if (c.conv_group > 0 && (c.conv_group % 4 || c.hidden % c.conv_group || (2 * c.hidden / c.conv_group) % 8))
    return DFLASH_E_UNSUPPORTED;
  if (c.sel_rank > 0 && (c.sel_rank > 4096 || c.sel_cands < 1 || c.sel_cands > 64 || c.sel_cands > c.vocab))
    return DFLASH_E_UNSUPPORTED;
  if ((int64_t)c.max_batch * (c.max_k + 1) > (1 << 20)) return DFLASH_E_UNSUPPORTED;
  // the bf16 GEMM addresses each operand with 32-bit byte offsets from a base
  const int64_t es = c.dtype == DFLASH_BF16 ? 2 : 4, lim = (int64_t)1 << 32;
  const int64_t widest = std::max<int64_t>(c.ffn, std::max<int64_t>(c.hidden, (int64_t)c.n_q_heads * c.head_dim));
  if ((int64_t)c.vocab * c.hidden * es >= lim || (int64_t)c.ffn * c.hidden * es >= lim ||
      (int64_t)c.hidden * c.n_target_layers * c.target_hidden * es >= lim ||
      (int64_t)c.n_q_heads * c.head_dim * c.hidden * es >= lim ||
      (int64_t)c.max_batch * (c.max_k + 1) * widest * es >= lim)
    return DFLASH_E_UNSUPPORTED;
  return DFLASH_OK;
}

// q-row splits so that one attention work-group holds at most 16*qrt_cap query rows
int choose_attn_splits(const dflash_config& c, int qrt_cap) {
  const int g = c.n_q_heads / c.n_kv_heads;
  for (int s = 1; s <= g; s *= 2) {
    if (g % s) continue;
    if ((g / s) * (c.max_k + 1) <= 16 * qrt_cap) return s;
  }
  return -1;
}

GemmArgs gemm_a1(const void* a, int64_t lda, int M, int N, int K) {
  GemmArgs g;
  std::memset(&g, 0, sizeof(g));
  g.M = M;
  g.N = N;
  g.K = K;
  g.a_ptr[0] = a;
  g.a_ld[0] = lda;
  g.a_nseg = 1;
  g.a_segk = K;
  g.b_nseg = 1;
  g.splits = 1;
  g.out_scale = 1.f;
  return g;
}

void set_b(GemmArgs& g, std::initializer_list<std::pair<const void*, int>> segs, int64_t ld) {
  int s = 0, begin = 0;
  for (auto& p : segs) {
    g.b_ptr[s] = p.first;
    g.b_begin[s] = begin;
    begin += p.second;
    ++s;
  }
  g.b_begin[s] = begin;
  g.b_nseg = s;
  g.b_ld = ld;
}

inline hipStream_t S(void* s) { return (hipStream_t)s; }

// The matrices every product reads.  fp32 drafter: the caller's.  bf16 drafter:
// fp16 copies of q/k/v/o/gate/up/down of every layer, the convolution
// projections, the LM head and the selector's W_H.  Each group of matrices that
// one product reads (q|k|v of all layers, since the injection reads every
// layer's k|v at once; o, gate|up, down and each projection per layer; the LM
// head; W_H) is scaled by its own power of two 2^s, chosen from the group's
// largest |w| so that it lies in [2^14, 2^15).  A bf16 value has 8 significant
// bits, so w * 2^s is exact in fp16 whenever it is at least 2^-14, which holds
// for every |w| of at least 2^-28 times the group's largest; smaller weights
// round to fp16's subnormal grid (absolute error at most 2^(-25-s)).  The
// epilogues multiply each product by its group's 2^-s (exact).
//
// An after-sub-layer convolution's correction o . P^T is computed as A . (P . W)^T,
// extra output columns of the sub-layer's output product (o = A . W^T), so its
// P . W (fp32, made here once) joins W's scale group.
int prepare_weights(dflash_handle* h) {
  const dflash_config& c = h->cfg;
  h->mats.resize(c.n_layers);
  const int64_t H = c.hidden, qdim = (int64_t)c.n_q_heads * c.head_dim, kvdim = (int64_t)c.n_kv_heads * c.head_dim;
  const int64_t F = c.ffn, V = c.vocab;
  const int64_t nc = c.conv_group > 0 ? 2 * H / c.conv_group : 0;
  // P . W products of the after-sub-layer convolutions, fp32 [nc, q_dim] / [nc, ffn]
  std::vector<float*> pw_o(c.n_layers, nullptr), pw_d(c.n_layers, nullptr);
  int rc = DFLASH_OK;
  for (int l = 0; l < c.n_layers && c.conv_group > 0; ++l) {
    const dflash_layer_weights& L = h->layers[l];
    if (L.attn_conv_post_proj) {
      if ((rc = alloc_t(h, &pw_o[l], (size_t)(nc * qdim), 4))) return rc;
      launch_matmul_nn(c.dtype, (int)nc, (int)qdim, (int)H, L.attn_conv_post_proj, L.o_w, pw_o[l], nullptr);
    }
    if (L.mlp_conv_post_proj) {
      if ((rc = alloc_t(h, &pw_d[l], (size_t)(nc * F), 4))) return rc;
      launch_matmul_nn(c.dtype, (int)nc, (int)F, (int)H, L.mlp_conv_post_proj, L.down_w, pw_d[l], nullptr);
    }
  }
  if (hipGetLastError() != hipSuccess) return DFLASH_E_HIP;
  if (c.dtype != DFLASH_BF16) {
    for (int l = 0; l < c.n_layers; ++l) {
      const dflash_layer_weights& L = h->layers[l];
      h->mats[l] = {L.q_w, L.k_w, L.v_w, L.o_w, L.gate_w, L.up_w, L.down_w, L.attn_conv_proj, L.mlp_conv_proj,
                    pw_o[l], pw_d[l]};
    }
    h->lm = h->lm_head;
    h->sel_h = h->sel_hidden_src;
    return DFLASH_OK;
  }
  // Each group of matrices read by one product gets its own power-of-two scale,
  // chosen from the group's largest |w|, so one large matrix does not shrink the
  // exact range of the others.
  struct Job { const void* src; int64_t n; const void** dst; int group; bool f32 = false; };
  std::vector<Job> jobs;
  std::vector<float*> group_scale;           // where each group's 2^-s goes
  auto group = [&](float* out) { group_scale.push_back(out); return (int)group_scale.size() - 1; };
  const int g_qkv = group(&h->s_qkv);
  for (int l = 0; l < c.n_layers; ++l) {
    const dflash_layer_weights& L = h->layers[l];
    dflash_handle::Mats& m = h->mats[l];
    jobs.push_back({L.q_w, qdim * H, &m.q, g_qkv});
    jobs.push_back({L.k_w, kvdim * H, &m.k, g_qkv});
    jobs.push_back({L.v_w, kvdim * H, &m.v, g_qkv});
    const int g_o = group(&m.s_o);
    jobs.push_back({L.o_w, H * qdim, &m.o, g_o});
    if (pw_o[l]) jobs.push_back({pw_o[l], nc * qdim, &m.conv_ap, g_o, true});
    const int g_gu = group(&m.s_gu);
    jobs.push_back({L.gate_w, F * H, &m.gate, g_gu});
    jobs.push_back({L.up_w, F * H, &m.up, g_gu});
    const int g_d = group(&m.s_down);
    jobs.push_back({L.down_w, H * F, &m.down, g_d});
    if (pw_d[l]) jobs.push_back({pw_d[l], nc * F, &m.conv_mp, g_d, true});
    m.conv_a = m.conv_m = nullptr;
    if (c.conv_group > 0) {
      jobs.push_back({L.attn_conv_proj, 2 * H / c.conv_group * H, &m.conv_a, group(&m.s_ca)});
      jobs.push_back({L.mlp_conv_proj, 2 * H / c.conv_group * H, &m.conv_m, group(&m.s_cm)});
    }
  }
  jobs.push_back({h->lm_head, V * H, &h->lm, group(&h->s_lm)});
  if (c.sel_rank > 0) jobs.push_back({h->sel_hidden_src, (int64_t)c.sel_rank * H, &h->sel_h, group(&h->s_selh)});
  const int ng = (int)group_scale.size();
  uint32_t* d_max = nullptr;
  if ((rc = alloc_t(h, &d_max, (size_t)ng, 4))) return rc;
  if (hipMemset(d_max, 0, (size_t)ng * 4) != hipSuccess) return DFLASH_E_HIP;
  for (auto& j : jobs) {
    if (j.f32) launch_absmax_f32((const float*)j.src, j.n, d_max + j.group, nullptr);
    else launch_absmax_bf16(j.src, j.n, d_max + j.group, nullptr);
  }
  std::vector<uint32_t> bits(ng);
  if (hipMemcpy(bits.data(), d_max, (size_t)ng * 4, hipMemcpyDeviceToHost) != hipSuccess) return DFLASH_E_HIP;
  std::vector<float> scale(ng);
  for (int gi = 0; gi < ng; ++gi) {
    float amax;
    std::memcpy(&amax, &bits[gi], 4);
    if (!(amax <= 3.0e38f)) return DFLASH_E_INVALID;   // Inf or NaN among the weights
    int s = 0;
    if (amax > 0.f) {
      int e;
      std::frexp(amax, &e);     // amax in [2^(e-1), 2^e)
      s = 15 - e;               // amax * 2^s in [2^14, 2^15)
    }
    *group_scale[gi] = std::ldexp(1.0f, -s);
    scale[gi] = std::ldexp(1.0f, s);
  }
  for (auto& j : jobs) {
    void* dst = nullptr;
    if ((rc = alloc(h, &dst, (size_t)j.n * 2))) return rc;
    if (j.f32) launch_convert_f32_f16((const float*)j.src, j.n, scale[j.group], dst, nullptr);
    else launch_convert_bf16_f16(j.src, j.n, scale[j.group], dst, nullptr);
    *j.dst = dst;
  }
  for (int l = 0; l < c.n_layers; ++l) {   // the fp32 products now live in their fp16 copies
    if (pw_o[l]) free_one(h, pw_o[l]);
    if (pw_d[l]) free_one(h, pw_d[l]);
  }
  return DFLASH_OK;
}

}  // namespace

extern "C" {

const char* dflash_status_str(int st) {
  switch (st) {
    case DFLASH_OK: return "ok";
    case DFLASH_E_INVALID: return "invalid argument";
    case DFLASH_E_NOMEM: return "out of device memory";
    case DFLASH_E_CAPACITY: return "capacity exceeded";
    case DFLASH_E_UNSUPPORTED: return "unsupported shape";
    case DFLASH_E_HIP: return "HIP runtime error";
    default: return "unknown status";
  }
}

int dflash_create(const dflash_config* cfg, const dflash_weights* w, dflash_handle** out) {
  if (!cfg || !w || !out) return DFLASH_E_INVALID;
  *out = nullptr;
  int rc = check_config(*cfg);
  if (rc) return rc;
  const dflash_config& c = *cfg;
  if (w->n_layers != c.n_layers || !w->layers || !w->embed || !w->lm_head || !w->fc || !w->hidden_norm ||
      !w->final_norm)
    return DFLASH_E_INVALID;
  for (int l = 0; l < c.n_layers; ++l) {
    const dflash_layer_weights& L = w->layers[l];
    if (!L.in_norm || !L.q_w || !L.k_w || !L.v_w || !L.o_w || !L.q_norm || !L.k_norm || !L.post_norm ||
        !L.gate_w || !L.up_w || !L.down_w)
      return DFLASH_E_INVALID;
    if (c.conv_group > 0 && (!L.attn_conv_base || !L.attn_conv_proj || !L.mlp_conv_base || !L.mlp_conv_proj))
      return DFLASH_E_INVALID;
    // an after-sub-layer convolution needs both its pointers
    if (c.conv_group > 0 && (!L.attn_conv_post_base != !L.attn_conv_post_proj ||
                             !L.mlp_conv_post_base != !L.mlp_conv_post_proj))
      return DFLASH_E_INVALID;
  }
  if (c.sel_rank > 0 && (!w->sel_pred || !w->sel_succ || !w->sel_hidden)) return DFLASH_E_INVALID;
  const int qrt_cap = 5;  // attention work-groups hold at most 5 tiles of 16 query rows
  const int splits = choose_attn_splits(c, qrt_cap);
  if (splits < 0) return DFLASH_E_UNSUPPORTED;

  dflash_handle* h = new dflash_handle();
  h->cfg = c;
  h->esize = c.dtype == DFLASH_BF16 ? 2 : 4;
  h->qrt_max = qrt_cap;
  h->attn_splits = splits;
  (void)hipGetDevice(&h->device);
  hipDeviceProp_t prop;
  if (hipGetDeviceProperties(&prop, h->device) == hipSuccess && prop.multiProcessorCount > 0)
    h->num_cus = prop.multiProcessorCount;
  h->embed = w->embed;
  h->lm_head = w->lm_head;
  h->fc = w->fc;
  h->hidden_norm = w->hidden_norm;
  h->final_norm = w->final_norm;
  h->layers.assign(w->layers, w->layers + c.n_layers);
  h->mask_emb = w->mask_embedding;
  if (c.sel_rank > 0) {
    h->sel_pred = w->sel_pred;
    h->sel_succ = w->sel_succ;
    h->sel_hidden_src = w->sel_hidden;
  }

  const int H = c.hidden, d = c.head_dim, nkv = c.n_kv_heads, g = c.n_q_heads / nkv;
  const int qdim = c.n_q_heads * d, kvdim = nkv * d;
  const size_t es = h->esize;
  const int R = c.max_k + 1;
  h->maxM = c.max_batch * R;
  h->Rpad = ((R + 31) / 32) * 32;
  h->QRpad = ((g * R + 15) / 16) * 16 + 80;
  h->ctx_alloc = ((int64_t)(c.max_ctx + 63) / 64) * 64 + 64;
  // attention work-groups: for 16-bit K/V as many ring work-groups as fit the CUs
  // at once (equal group ranges, one partial record per (work-group, segment)
  // piece); for fp32 two LDS-ring work-groups per CU with at most kAttnChunkMax
  // partial records (chunks) per segment
  h->attn_waves = c.dtype == DFLASH_BF16;
  h->attn_wg = (h->attn_waves ? attn_waves_wg_per_cu() : 2) * h->num_cus;
  h->piece_cap = h->attn_waves ? h->attn_wg + c.max_batch * nkv * splits : c.max_batch * nkv * splits * kAttnChunkMax;
  h->op = c.dtype == DFLASH_BF16 ? OP_F16 : OP_F32;
  h->op_fc = c.dtype == DFLASH_BF16 ? OP_BF16 : OP_F32;
  h->lm_tile = gemm_bn(h->op);
  h->n_vtiles = (c.vocab + h->lm_tile - 1) / h->lm_tile;
  h->inject_chunk = std::min(c.max_inject_rows, 16384);

  if (c.page_size > 0) {
    h->pages_per_slot = (c.max_ctx + c.page_size - 1) / c.page_size;
    h->page_elems = (int64_t)c.n_layers * nkv * c.page_size * d;
  }
  const size_t cache_elems = c.page_size > 0 ? (size_t)c.num_pages * h->page_elems
                                             : (size_t)c.n_layers * (c.max_batch + 1) * nkv * h->ctx_alloc * d;
  do {
    if ((rc = alloc(h, &h->cache_k, cache_elems * es))) break;
    if ((rc = alloc(h, &h->cache_v, cache_elems * es))) break;
    if ((rc = alloc_t(h, &h->ctx_len, c.max_batch + 1, 4))) break;
    if ((rc = alloc_t(h, &h->err, 1, 4))) break;
    h->n_rope = (int)h->ctx_alloc;
    if ((rc = alloc_t(h, &h->rope, (size_t)h->n_rope * (d / 2), sizeof(float2)))) break;
    void* kg = nullptr;
    if ((rc = alloc(h, &kg, sizeof(void*) * c.n_layers))) break;
    h->d_k_gains = (const void**)kg;
    if ((rc = alloc_t(h, &h->X, (size_t)h->maxM * H, 4))) break;
    if ((rc = alloc(h, &h->hbuf, (size_t)h->maxM * H * es))) break;
    if ((rc = alloc(h, &h->attn_out, (size_t)h->maxM * qdim * es))) break;
    if ((rc = alloc(h, &h->act, (size_t)h->maxM * c.ffn * es))) break;
    if ((rc = alloc(h, &h->qb, (size_t)c.max_batch * nkv * h->QRpad * d * es))) break;
    if ((rc = alloc(h, &h->kb, (size_t)c.max_batch * nkv * h->Rpad * d * es))) break;
    if ((rc = alloc(h, &h->vb, (size_t)c.max_batch * nkv * h->Rpad * d * es))) break;
    const size_t prow = (size_t)h->piece_cap * 16 * h->qrt_max;
    if ((rc = alloc_t(h, &h->o_part, prow * d, 4))) break;
    if ((rc = alloc_t(h, &h->m_part, prow, 4))) break;
    if ((rc = alloc_t(h, &h->l_part, prow, 4))) break;
    if ((rc = alloc_t(h, &h->plan, 1, sizeof(AttnPlan)))) break;
    if ((rc = alloc_t(h, &h->seg_start, (size_t)c.max_batch * nkv * splits + 1, 4))) break;
    if ((rc = alloc_t(h, &h->chunk_base, (size_t)c.max_batch * nkv * splits, 4))) break;
    if ((rc = alloc_t(h, &h->seg_desc, (size_t)c.max_batch * nkv * splits, 16))) break;
    if ((rc = alloc_t(h, &h->wg_range, (size_t)h->attn_wg, 16))) break;
    if ((rc = alloc_t(h, &h->dslots, c.max_batch, 4))) break;
    // split-K partials: grids of at most 2 * CUs tiles, or a five-way split of the
    // long-K products over the draft's rows (M x H each, rows padded to 128- or
    // 192-row tiles); a product needing more runs with fewer splits
    // (H columns, plus the kernel corrections of DFlash 2 after-sub-layer convolutions)
    const size_t mpad = std::max((h->maxM + 127) / 128 * 128, (h->maxM + 191) / 192 * 192);
    const size_t ncols = H + (c.conv_group > 0 ? 2 * (H / c.conv_group) : 0);
    h->partials_elems = std::max((size_t)(2 * h->num_cus + 8) * 128 * gemm_bn(h->op), (size_t)5 * mpad * ncols);
    // ... and the per-step injection (a row bound of at most 1024 on 64-row tiles,
    // the true row count on the device): the partial tiles cover every row tile
    // of the bound, for the fc product's K split in up to eight and the K|V
    // product's in up to eight (a smaller buffer silently cut both splits)
    const size_t inj_rows = (size_t)(std::min(c.max_inject_rows, 1024) + 63) / 64 * 64;
    const size_t kv_cols = (size_t)2 * kvdim * std::min(c.n_layers, MAX_BSEG / 2);
    h->partials_elems = std::max(h->partials_elems, 8 * inj_rows * std::max((size_t)H, kv_cols));
    if ((rc = alloc_t(h, &h->partials, h->partials_elems, 4))) break;
    const size_t lrows = (size_t)c.max_batch * c.max_k;
    if ((rc = alloc_t(h, &h->logits_ws, lrows * c.vocab, 4))) break;
    if ((rc = alloc_t(h, &h->tmax, lrows * h->n_vtiles, 4))) break;
    if ((rc = alloc_t(h, &h->tsum, lrows * h->n_vtiles, 4))) break;
    if ((rc = alloc_t(h, &h->targ, lrows * h->n_vtiles, 4))) break;
    if ((rc = alloc_t(h, &h->row_max, lrows, 4))) break;
    if ((rc = alloc_t(h, &h->row_lse, lrows, 4))) break;
    const int kc = std::max(1, std::min(c.max_tree, c.vocab));
    if ((rc = alloc_t(h, &h->tk_ids, lrows * kc, 4))) break;
    {   // truncation scratch: rows of a verification (K+1 target and K draft rows per request)
      const size_t vrows = (size_t)c.max_batch * (2 * c.max_k + 1);
      if ((rc = alloc_t(h, &h->vt_max, vrows * h->n_vtiles, 4))) break;
      if ((rc = alloc_t(h, &h->vrow_max, vrows, 4))) break;
      if ((rc = alloc_t(h, &h->vrow_lse, vrows, 4))) break;
      if ((rc = alloc_t(h, &h->tr_ids, vrows * 64, 4))) break;
      if ((rc = alloc_t(h, &h->tr_probs, vrows * 64, 4))) break;
      if ((rc = alloc_t(h, &h->kp_ids, vrows * 64, 4))) break;
      if ((rc = alloc_t(h, &h->kp_probs, vrows * 64, 4))) break;
      if ((rc = alloc_t(h, &h->nuc, vrows, sizeof(Nucleus)))) break;
    }
    if (c.conv_group > 0) {
      if ((rc = alloc(h, &h->hbuf2, (size_t)h->maxM * H * es))) break;
      if ((rc = alloc_t(h, &h->cbuf, (size_t)h->maxM * 2 * (H / c.conv_group), 4))) break;
      if ((rc = alloc_t(h, &h->obuf, (size_t)h->maxM * H, 4))) break;
      if ((rc = alloc_t(h, &h->rsbuf, (size_t)h->maxM, 4))) break;
    }
    if (c.sel_rank > 0) {
      const size_t C = c.sel_cands;
      if ((rc = alloc_t(h, &h->sel_gate, lrows * c.sel_rank, 4))) break;
      if ((rc = alloc_t(h, &h->sel_cand, lrows * C, 4))) break;
      if ((rc = alloc_t(h, &h->sel_cprob, lrows * C, 4))) break;
      if ((rc = alloc_t(h, &h->sel_ids_ws, lrows * C, 4))) break;
      if ((rc = alloc_t(h, &h->sel_probs_ws, lrows * C, 4))) break;
      if ((rc = alloc_t(h, &h->sel_table, lrows * C * C, 4))) break;
      if ((rc = alloc(h, &h->sel_hin, lrows * H * es))) break;
    }
    if ((rc = alloc_t(h, &h->tk_probs, lrows * kc, 4))) break;
    if ((rc = alloc_t(h, &h->y, (size_t)h->inject_chunk * H, 4))) break;
    if ((rc = alloc(h, &h->g, (size_t)h->inject_chunk * H * es))) break;
    if ((rc = alloc_t(h, &h->a_rows, c.max_inject_rows, 4))) break;
    if ((rc = alloc_t(h, &h->row_slot, c.max_inject_rows, 4))) break;
    if ((rc = alloc_t(h, &h->row_pos, c.max_inject_rows, 4))) break;
    if ((rc = alloc_t(h, &h->req_off, c.max_batch + 1, 4))) break;
    if ((rc = alloc_t(h, &h->req_pos, c.max_batch, 4))) break;
    if ((rc = alloc_t(h, &h->post, (size_t)c.max_batch * R, 4))) break;
    if ((rc = alloc_t(h, &h->vstats, (size_t)c.max_batch * (2 * c.max_k + 1) * 2, 4))) break;
    if ((rc = alloc_t(h, &h->vacc, (size_t)c.max_batch, 4))) break;
    if ((rc = alloc_t(h, &h->vchunks, (size_t)2 * c.max_batch * draw_chunks(c.vocab), 4))) break;
  } while (0);
  if (rc) {
    free_all(h);
    delete h;
    return rc;
  }
  if (!rc) rc = prepare_weights(h);
  std::vector<const void*> kg(c.n_layers);
  for (int l = 0; l < c.n_layers; ++l) kg[l] = h->layers[l].k_norm;
  if (!rc && hipMemcpy(h->d_k_gains, kg.data(), sizeof(void*) * c.n_layers, hipMemcpyHostToDevice) != hipSuccess)
    rc = DFLASH_E_HIP;
  if (!rc) {
    launch_rope_table(h->rope, h->n_rope, d, (double)c.rope_theta, nullptr);
    if (hipDeviceSynchronize() != hipSuccess || hipGetLastError() != hipSuccess) rc = DFLASH_E_HIP;
  }
  if (rc) {
    free_all(h);
    delete h;
    return rc;
  }
  *out = h;
  return DFLASH_OK;
}

int dflash_destroy(dflash_handle* h) {
  if (!h) return DFLASH_E_INVALID;
  (void)hipDeviceSynchronize();
  free_all(h);
  delete h;
  return DFLASH_OK;
}

int dflash_reset_slots(dflash_handle* h, void* stream, int32_t n, const int32_t* slots_dev) {
  if (!h || n < 0 || (n > 0 && !slots_dev)) return DFLASH_E_INVALID;
  launch_reset_slots(n, slots_dev, h->ctx_len, h->cfg.max_batch, h->err, S(stream));
  return hipGetLastError() == hipSuccess ? DFLASH_OK : DFLASH_E_HIP;
}

}  // extern "C"

namespace {

// Common checks of the injection entry points.
int validate_inject(dflash_handle* h, int n_req, const int32_t* slots, const int32_t* row_count,
                    int64_t rows_upper_bound, const void* const* target_hidden, int64_t row_stride) {
  const dflash_config& c = h->cfg;
  if (!slots || !row_count || !target_hidden) return DFLASH_E_INVALID;
  if (n_req > c.max_batch || rows_upper_bound > c.max_inject_rows) return DFLASH_E_CAPACITY;
  if (row_stride < c.target_hidden || row_stride % 8) return DFLASH_E_INVALID;
  if (c.page_size > 0 && !h->page_table) return DFLASH_E_INVALID;
  for (int l = 0; l < c.n_target_layers; ++l)
    if (!target_hidden[l]) return DFLASH_E_INVALID;
  return DFLASH_OK;
}

// K splits of the per-step injection products (planned for one 64-row tile, the
// true row count on the device), measured at batch 32: K|V 4 (inject_kv 64 us
// per step with 2, 50 with 4, 57 with 8), fc 16 (63 us with 8, 61 with 16)
static constexpr int KV_STEP_SPLITS = 4;
static constexpr int FC_STEP_SPLITS = 16;

// The products of an injection once its row tables (a_rows, row_slot, row_pos,
// req_off) are on the device: fc, RMSNorm, per-layer K|V with k-norm + RoPE into the cache.
int inject_rows(dflash_handle* h, hipStream_t s, int n_req, int64_t rows_upper_bound, const void* const* target_hidden,
                int64_t row_stride) {
  const dflash_config& c = h->cfg;
  const int dt = c.dtype;
  const int H = c.hidden, kvdim = c.n_kv_heads * c.head_dim;
  const int featK = c.n_target_layers * c.target_hidden;
  for (int64_t c0 = 0; c0 < rows_upper_bound; c0 += h->inject_chunk) {
    const int rows = (int)std::min<int64_t>(h->inject_chunk, rows_upper_bound - c0);
    // The true row count is on the device (row tiles past it exit at once).  A
    // small bound is the per-step case, where usually only the first row tile is
    // live: size the K split for that tile rather than for the bound.
    const int plan_rows = rows <= 1024 ? std::min(rows, 64) : rows;
    // fc over the concatenated target layers
    GemmArgs ga = gemm_a1(nullptr, 0, rows, H, featK);
    for (int l = 0; l < c.n_target_layers; ++l) {
      ga.a_ptr[l] = target_hidden[l];
      ga.a_ld[l] = row_stride;
    }
    ga.a_nseg = c.n_target_layers;
    ga.a_segk = c.target_hidden;
    ga.a_rows = h->a_rows + c0;
    ga.a_wide = 1;  // the caller's hidden-state buffers may exceed 4 GiB
    ga.m_valid = h->req_off + n_req;
    ga.m_valid_base = (int)c0;
    set_b(ga, {{h->fc, H}}, featK);
    EpiStore<float>::Params pf{h->y, H};
    {
      Phase ph(h, s, DFLASH_PH_INJECT_FC);
      GemmPlan fp = plan_gemm(h->op_fc, plan_rows, H, featK, h->num_cus, false, true);
      if (plan_rows <= 64) fp.splits = std::max(fp.splits, FC_STEP_SPLITS);
      launch_gemm(h->op_fc, EPI_STORE_F32, ga, &pf, fp, h->partials, h->partials_elems, s);
    }
    {
      Phase ph(h, s, DFLASH_PH_INJECT_NORM);
      launch_rmsnorm(dt, rows, H, h->y, 0, 1, 1, h->hidden_norm, h->g, c.rms_eps, s, h->req_off + n_req, (int)c0);
    }
    // per-layer K|V of the fused feature, up to 8 layers per product
    for (int l0 = 0; l0 < c.n_layers; l0 += MAX_BSEG / 2) {
      const int nl = std::min(MAX_BSEG / 2, c.n_layers - l0);
      GemmArgs gk = gemm_a1(h->g, H, rows, 2 * kvdim * nl, H);
      gk.out_scale = h->s_qkv;
      gk.m_valid = h->req_off + n_req;
      gk.m_valid_base = (int)c0;
      for (int i = 0; i < nl; ++i) {
        gk.b_ptr[2 * i] = h->mats[l0 + i].k;
        gk.b_ptr[2 * i + 1] = h->mats[l0 + i].v;
        gk.b_begin[2 * i] = 2 * i * kvdim;
        gk.b_begin[2 * i + 1] = (2 * i + 1) * kvdim;
      }
      gk.b_begin[2 * nl] = 2 * nl * kvdim;
      gk.b_nseg = 2 * nl;
      gk.b_ld = H;
      EpiKVInject<f16_t>::Params pk;
      pk.cache_k = (f16_t*)h->cache_k;
      pk.cache_v = (f16_t*)h->cache_v;
      pk.row_slot = h->row_slot + c0;
      pk.row_pos = h->row_pos + c0;
      pk.k_gain = (const bf16_t* const*)(h->d_k_gains + l0);
      pk.rope = h->rope;
      pk.n_kv = c.n_kv_heads;
      pk.d = c.head_dim;
      pk.kv_dim = kvdim;
      pk.max_batch = c.max_batch + 1;  // cache slot dimension (one spare slot)
      pk.ctx_alloc = h->ctx_alloc;
      pk.eps = c.rms_eps;
      pk.layer0 = l0;
      pk.pages = h->pages();
      pk.err = h->err;
      // the parameter block has the same layout for fp32 (pointers only differ in type)
      GemmPlan kp = plan_gemm(h->op, plan_rows, gk.N, H, h->num_cus, false, true);
      if (plan_rows <= 64) kp.splits = std::max(kp.splits, KV_STEP_SPLITS);
      Phase ph(h, s, DFLASH_PH_INJECT_KV);
      launch_gemm(h->op, EPI_KVINJECT, gk, &pk, kp, h->partials, h->partials_elems, s);
    }
  }
  return hipGetLastError() == hipSuccess ? DFLASH_OK : DFLASH_E_HIP;
}

}  // namespace

extern "C" {

int dflash_inject_context(dflash_handle* h, void* stream, int32_t n_req, const int32_t* slots,
                          const int32_t* row_start, const int32_t* row_count, int64_t rows_upper_bound,
                          const void* const* target_hidden, int64_t row_stride) {
  if (!h || n_req < 0 || rows_upper_bound < 0) return DFLASH_E_INVALID;
  if (n_req == 0 || rows_upper_bound == 0) return DFLASH_OK;
  if (!row_start) return DFLASH_E_INVALID;
  int rc = validate_inject(h, n_req, slots, row_count, rows_upper_bound, target_hidden, row_stride);
  if (rc) return rc;
  const dflash_config& c = h->cfg;
  hipStream_t s = S(stream);
  {
    Phase ph(h, s, DFLASH_PH_INJECT_PREP);
    launch_inject_scan(n_req, slots, row_start, row_count, h->ctx_len, c.max_ctx, c.max_batch, rows_upper_bound,
                       h->req_off, h->req_pos, h->err, s);
    // source rows are int32 indices into the caller's buffers
    launch_inject_fill(n_req, rows_upper_bound, slots, row_start, nullptr, 0, 0, h->req_off, h->req_pos,
                       (int64_t)INT32_MAX, h->a_rows, h->row_slot, h->row_pos, h->err, s);
  }
  return inject_rows(h, s, n_req, rows_upper_bound, target_hidden, row_stride);
}

int dflash_inject_tree_path(dflash_handle* h, void* stream, int32_t n_req, const int32_t* slots,
                            const int32_t* path_nodes, const int32_t* path_len, int32_t max_path,
                            int32_t tree_stride, int64_t rows_upper_bound, const void* const* target_hidden,
                            int64_t row_stride) {
  if (!h || n_req < 0 || rows_upper_bound < 0 || max_path < 1 || tree_stride < 1) return DFLASH_E_INVALID;
  if (n_req == 0 || rows_upper_bound == 0) return DFLASH_OK;
  if (!path_nodes) return DFLASH_E_INVALID;
  int rc = validate_inject(h, n_req, slots, path_len, rows_upper_bound, target_hidden, row_stride);
  if (rc) return rc;
  if ((int64_t)n_req * tree_stride > (int64_t)INT32_MAX) return DFLASH_E_UNSUPPORTED;
  const dflash_config& c = h->cfg;
  hipStream_t s = S(stream);
  {
    Phase ph(h, s, DFLASH_PH_INJECT_PREP);
    launch_inject_scan(n_req, slots, nullptr, path_len, h->ctx_len, c.max_ctx, c.max_batch, rows_upper_bound,
                       h->req_off, h->req_pos, h->err, s);
    launch_inject_fill(n_req, rows_upper_bound, slots, nullptr, path_nodes, max_path, tree_stride, h->req_off,
                       h->req_pos, (int64_t)INT32_MAX, h->a_rows, h->row_slot, h->row_pos, h->err, s);
  }
  return inject_rows(h, s, n_req, rows_upper_bound, target_hidden, row_stride);
}

}  // extern "C"

namespace {

// DFlash 2 [P2 §3.2.3]: hbuf2 = dynamic conv of the block rows of the sub-layer
// input x = X * rs * gain held in hbuf (rs from the norm pass that wrote hbuf);
// the per-row kernel corrections come from one product with the layer's proj.
// A split product leaves its partial tiles to the convolution, which sums them
// in split order (as the reduction pass would) and applies the weight scale.
void conv_stage(dflash_handle* h, hipStream_t s, int M, int R, const void* proj, float proj_scale, const void* base,
                const void* gain) {
  const dflash_config& c = h->cfg;
  const int H = c.hidden, nc = 2 * (H / c.conv_group);
  Phase ph(h, s, DFLASH_PH_CONV);
  GemmArgs ga = gemm_a1(h->hbuf, H, M, nc, H);
  ga.out_scale = proj_scale;
  set_b(ga, {{proj, nc}}, H);
  ga.keep_partials = 1;
  EpiStore<float>::Params pc{h->cbuf, nc};
  const GemmShape gs = launch_gemm(h->op, EPI_STORE_F32, ga, &pc, plan_gemm(h->op, M, nc, H, h->num_cus), h->partials,
                                   h->partials_elems, s);
  if (gs.splits > 1)
    launch_dyn_conv(c.dtype, M, R, H, c.conv_group, h->X, h->rsbuf, gain, h->partials, gs.Npad, gs.splits,
                    (int64_t)gs.Mpad * gs.Npad, proj_scale, base, h->hbuf2, s);
  else
    launch_dyn_conv(c.dtype, M, R, H, c.conv_group, h->X, h->rsbuf, gain, h->cbuf, nc, 1, 0, 1.f, base, h->hbuf2, s);
}

// Output projection of a sub-layer (A [M, Kd] times B^T [H, Kd]): added to the
// residual stream; or, when an after-sub-layer convolution follows (post_pw =
// its P . W [2H/G, Kd]), the output goes to obuf and its kernel corrections,
// from the same product's extra columns, to cbuf -- norm_stage applies them.
// keep_partials (no convolution): a K-split product leaves its partials for the
// next norm pass to add (launch_partials_add_norm) instead of reducing them here.
GemmShape sublayer_out(dflash_handle* h, hipStream_t s, int M, const void* a, int Kd, const void* b, float b_scale,
                       const void* post_pw, int phase, bool keep_partials = false, bool balance = false) {
  const dflash_config& c = h->cfg;
  const int H = c.hidden;
  const int nc = post_pw ? 2 * (H / c.conv_group) : 0;
  GemmArgs ga = gemm_a1(a, Kd, M, H + nc, Kd);
  ga.out_scale = b_scale;
  Phase ph(h, s, phase);
  if (!post_pw) {
    set_b(ga, {{b, H}}, Kd);
    ga.keep_partials = keep_partials ? 1 : 0;
    EpiResidualAdd::Params pr{h->X, H};
    GemmPlan gp = plan_gemm(h->op, M, H, Kd, h->num_cus);
    if (keep_partials && balance && gp.splits == 1) {
      // one round of whole tiles that leaves some CUs one work-group more than
      // the rest: split K in two (the norm pass adds the partials anyway)
      const long tiles = (long)((M + gp.bm - 1) / gp.bm) * ((H + gp.bn - 1) / gp.bn);
      if (tiles < 2L * h->num_cus && tiles % h->num_cus != 0 && Kd / 64 >= 32) gp.splits = 2;
    }
    return launch_gemm(h->op, EPI_RESADD, ga, &pr, gp, h->partials, h->partials_elems, s);
  }
  set_b(ga, {{b, H}, {post_pw, nc}}, Kd);
  StoreSplitParams pd{h->obuf, H, h->cbuf, nc, H};
  launch_gemm(h->op, EPI_STORE_SPLIT, ga, &pd, plan_gemm(h->op, M, H + nc, Kd, h->num_cus), h->partials,
              h->partials_elems, s);
  return GemmShape{1, 0, 0};
}

// RMSNorm of the rows (map_mask: the mask rows only) into hbuf, after applying
// the pending after-sub-layer convolution with base post_base (or none); with
// DFlash 2 convolutions the rows' RMS scales go to rsbuf for the next one.
// pend: a product whose split partials still have to be added to X (scale
// pend_scale) -- added here, fused with the norm.
void norm_stage(dflash_handle* h, hipStream_t s, int rows, int map_mask, int K, int R, const void* gain,
                const void* post_base, const GemmShape* pend = nullptr, float pend_scale = 1.f) {
  const dflash_config& c = h->cfg;
  float* rs = c.conv_group > 0 ? h->rsbuf : nullptr;
  if (pend && pend->splits > 1) {
    Phase ph(h, s, DFLASH_PH_NORM);
    launch_partials_add_norm(c.dtype, rows, c.hidden, h->X, map_mask, K, R, h->partials, pend->Npad, pend->splits,
                             (int64_t)pend->Mpad * pend->Npad, pend_scale, gain, h->hbuf, c.rms_eps, s);
    return;
  }
  if (post_base) {
    Phase ph(h, s, DFLASH_PH_CONV);
    launch_conv_post_norm(c.dtype, rows, c.hidden, c.conv_group, h->X, map_mask, K, R, h->obuf, h->cbuf, post_base,
                          gain, h->hbuf, c.rms_eps, rs, s);
  } else {
    Phase ph(h, s, DFLASH_PH_NORM);
    launch_rmsnorm(c.dtype, rows, c.hidden, h->X, map_mask, K, R, gain, h->hbuf, c.rms_eps, s, nullptr, 0, rs);
  }
}

// DFlash 2 path selector [P2 §3.1.2-3.1.3] over rows n_req*K whose logits and
// final-normalised hidden rows (operand type, [rows, H]) are given; row
// statistics (row_max / row_lse) must be current.
void selector_stage(dflash_handle* h, hipStream_t s, int n_req, int K, const int32_t* slots, const int32_t* anchors,
                    const float* logits, const void* hidden, float T, uint64_t seed, uint64_t step, int32_t* draft_ids,
                    int32_t* cand_ids, float* cand_probs) {
  const dflash_config& c = h->cfg;
  const int rows = n_req * K, H = c.hidden, C = c.sel_cands, r = c.sel_rank;
  Phase ph(h, s, DFLASH_PH_SELECTOR);
  launch_topk(rows, c.vocab, C, logits, h->tmax, h->n_vtiles, h->lm_tile, T > 0.f ? 1.0f / T : 1.0f, h->row_max,
              h->row_lse, h->sel_cand, h->sel_cprob, s);
  GemmArgs ga = gemm_a1(hidden, H, rows, r, H);
  ga.out_scale = h->s_selh;
  set_b(ga, {{h->sel_h, r}}, H);
  EpiStore<float>::Params pg{h->sel_gate, r};
  launch_gemm(h->op, EPI_STORE_F32, ga, &pg, plan_gemm(h->op, rows, r, H, h->num_cus), h->partials,
              h->partials_elems, s);
  launch_sel_walk(c.dtype, n_req, K, C, r, c.vocab, slots, anchors, logits, h->sel_cand, h->sel_gate, h->sel_pred,
                  h->sel_succ, T, seed, step, h->sel_table, draft_ids, cand_ids ? cand_ids : h->sel_ids_ws,
                  cand_probs ? cand_probs : h->sel_probs_ws, h->err, s);
}

int validate_draft(dflash_handle* h, int n_req, const dflash_draft_params* p, const dflash_draft_outputs* o) {
  const dflash_config& c = h->cfg;
  if (!p || !o || n_req < 0) return DFLASH_E_INVALID;
  if (n_req > c.max_batch) return DFLASH_E_CAPACITY;
  if (c.page_size > 0 && !h->page_table) return DFLASH_E_INVALID;
  if (p->K < 1 || p->K > c.max_k) return DFLASH_E_CAPACITY;
  if (p->top_k < 0 || p->top_k > c.max_top_k || p->top_k > c.vocab) return DFLASH_E_CAPACITY;
  if (p->tree_budget < 0 || p->tree_budget > c.max_tree) return DFLASH_E_CAPACITY;
  if (!(p->temperature >= 0.f)) return DFLASH_E_INVALID;
  if (!o->draft_ids) return DFLASH_E_INVALID;
  if (p->top_k > 0 && (!o->topk_ids || !o->topk_probs)) return DFLASH_E_INVALID;
  if (p->tree_budget > 0 && (!o->tree_tokens || !o->tree_parents || !o->tree_depth)) return DFLASH_E_INVALID;
  return DFLASH_OK;
}

// LM-head statistics are ready; finish rows: stats, draft ids, top-k, tree.
void select_stage(dflash_handle* h, hipStream_t s, int n_req, const int32_t* slots, const int32_t* anchors,
                  const float* logits, const dflash_draft_params* p, const dflash_draft_outputs* o) {
  const dflash_config& c = h->cfg;
  const int K = p->K, rows = n_req * K, V = c.vocab;
  const float T = p->temperature;
  const float inv_t = T > 0.f ? 1.0f / T : 1.0f;
  Phase ph(h, s, DFLASH_PH_SELECT);
  launch_row_finalize(rows, h->n_vtiles, h->tmax, h->tsum, h->targ, h->row_max, h->row_lse,
                      T > 0.f ? nullptr : o->draft_ids, o->row_max, o->row_lse, s);
  if (T > 0.f && h->trunc_k > 0) {   // symmetric truncation: draw from the truncated rows
    launch_topk(rows, V, h->trunc_k, logits, h->tmax, h->n_vtiles, h->lm_tile, inv_t, h->row_max, h->row_lse,
                h->tr_ids, h->tr_probs, s);
    launch_trunc_rows(rows, h->trunc_k, h->trunc_p, h->tr_ids, h->tr_probs, h->kp_ids, h->kp_probs, s);
    launch_sparse_sample(rows, K, h->trunc_k, slots, p->seed, p->step, h->kp_ids, h->kp_probs, o->draft_ids, s);
  } else if (T > 0.f && h->trunc_p < 1.f) {   // top-p over whole rows
    launch_nucleus(rows, V, logits, rows, rows, 0, h->row_max, 1, inv_t, h->trunc_p, h->nuc, s);
    launch_nucleus_sample(rows, K, V, slots, p->seed, p->step, inv_t, logits, h->row_max, h->nuc, o->draft_ids, s);
  } else if (T > 0.f) {
    launch_sample(rows, K, slots, p->seed, p->step, inv_t, logits, V, h->n_vtiles, h->lm_tile, h->tmax, h->tsum,
                  h->row_max, o->draft_ids, s);
  }
  const int B = p->tree_budget;
  const int kc = B > 0 ? std::min(B, V) : 0;
  if (p->top_k > 0)
    launch_topk(rows, V, p->top_k, logits, h->tmax, h->n_vtiles, h->lm_tile, inv_t, h->row_max, h->row_lse,
                o->topk_ids, o->topk_probs, s);
  if (B > 0) {
    const int32_t* ids = o->topk_ids;
    const float* probs = o->topk_probs;
    int stride = p->top_k;
    if (p->top_k < kc) {
      launch_topk(rows, V, kc, logits, h->tmax, h->n_vtiles, h->lm_tile, inv_t, h->row_max, h->row_lse, h->tk_ids,
                  h->tk_probs, s);
      ids = h->tk_ids;
      probs = h->tk_probs;
      stride = kc;
    }
    launch_tree(n_req, K, kc, stride, B, probs, ids, anchors, o->tree_tokens, o->tree_parents, o->tree_depth,
                o->tree_mask, s);
  }
}

}  // namespace

extern "C" {

int dflash_draft_block(dflash_handle* h, void* stream, int32_t n_req, const int32_t* slots_in,
                       const int32_t* anchor_ids, const dflash_draft_params* p, const dflash_draft_outputs* o) {
  if (!h) return DFLASH_E_INVALID;
  int rc = validate_draft(h, n_req, p, o);
  if (rc) return rc;
  if (n_req == 0) return DFLASH_OK;
  if (!slots_in || !anchor_ids) return DFLASH_E_INVALID;
  const dflash_config& c = h->cfg;
  hipStream_t s = S(stream);
  // every later kernel addresses the cache through validated slot ids
  launch_sanitize_slots(n_req, slots_in, h->dslots, c.max_batch, h->err, s);
  const int32_t* slots = h->dslots;
  const int dt = c.dtype;
  const int K = p->K, R = K + 1, M = n_req * R;
  const int H = c.hidden, d = c.head_dim, nkv = c.n_kv_heads, g = c.n_q_heads / nkv;
  const int qdim = c.n_q_heads * d, kvdim = nkv * d, F = c.ffn, V = c.vocab;
  const int splits = h->attn_splits, gps = g / splits;
  const int rows_split = gps * R;
  const int qrt = (rows_split + 15) / 16;

  {
    Phase ph(h, s, DFLASH_PH_EMBED);
    launch_embed_norm(dt, M, R, anchor_ids, c.mask_token_id, V, h->embed, h->mask_emb, c.input_embedding_scale, H, h->X,
                      h->layers[0].in_norm, h->hbuf, c.rms_eps, h->err, s, c.conv_group > 0 ? h->rsbuf : nullptr);
  }
  {
    Phase ph(h, s, DFLASH_PH_ATTN_PLAN);
    if (h->attn_waves)   // equal ranges, no snapping to chunk starts
      launch_attn_plan(slots, h->ctx_len, n_req, nkv, splits, h->attn_wg, kAttnMinGroupsWave, 1, 1 << 30, h->plan,
                       h->seg_start, h->chunk_base, h->seg_desc, h->wg_range, s);
    else
      launch_attn_plan(slots, h->ctx_len, n_req, nkv, splits, h->attn_wg, kAttnMinGroups, kAttnChunkMin,
                       kAttnChunkMax, h->plan, h->seg_start, h->chunk_base, h->seg_desc, h->wg_range, s);
    launch_page_check(n_req, slots, h->ctx_len, c.max_batch, h->pages(), h->err, s);
  }
  const int64_t layer_cache = (int64_t)(c.max_batch + 1) * nkv * h->ctx_alloc * d * h->esize;
  const void* post_m = nullptr;   // the last MLP's pending after-sub-layer convolution
  GemmShape down{1, 0, 0};        // the last down product's pending split partials (splits > 1)
  float down_scale = 1.f;
  for (int l = 0; l < c.n_layers; ++l) {
    const dflash_layer_weights& L = h->layers[l];
    const dflash_handle::Mats& W = h->mats[l];
    // DFlash 2: dynamic convolution of the attention sub-layer's input
    const void* attn_in = h->hbuf;
    if (c.conv_group > 0) {
      conv_stage(h, s, M, R, W.conv_a, W.s_ca, L.attn_conv_base, L.in_norm);
      attn_in = h->hbuf2;
    }
    // q | k | v with head norm + RoPE into the attention layouts
    {
      GemmArgs ga = gemm_a1(attn_in, H, M, qdim + 2 * kvdim, H);
      ga.out_scale = h->s_qkv;
      set_b(ga, {{W.q, qdim}, {W.k, kvdim}, {W.v, kvdim}}, H);
      EpiQKV<f16_t>::Params pq;
      pq.qb = (f16_t*)h->qb;
      pq.kb = (f16_t*)h->kb;
      pq.vb = (f16_t*)h->vb;
      pq.slots = slots;
      pq.ctx_len = h->ctx_len;
      pq.q_gain = (const bf16_t*)L.q_norm;
      pq.k_gain = (const bf16_t*)L.k_norm;
      pq.rope = h->rope;
      pq.R = R;
      pq.group = g;
      pq.n_kv = nkv;
      pq.d = d;
      pq.q_dim = qdim;
      pq.kv_dim = kvdim;
      pq.QRpad = h->QRpad;
      pq.Rpad = h->Rpad;
      pq.eps = c.rms_eps;
      pq.err = h->err;
      Phase ph(h, s, DFLASH_PH_QKV);
      launch_gemm(h->op, EPI_QKV, ga, &pq, plan_gemm(h->op, M, ga.N, H, h->num_cus), h->partials, h->partials_elems,
                  s);
    }
    // attention over [context ; block]
    {
      AttnArgs a;
      a.qb = h->qb;
      // contiguous: the layer's region; paged: the layer's part of page 0
      const int64_t lofs = c.page_size > 0 ? (int64_t)l * nkv * c.page_size * d * h->esize : l * layer_cache;
      a.cache_k = (const char*)h->cache_k + lofs;
      a.cache_v = (const char*)h->cache_v + lofs;
      a.page_table = h->pages().table;
      a.pages_per_slot = h->pages_per_slot;
      a.gpp = c.page_size / 32;
      a.n_pages = c.num_pages;
      a.table_rows = c.max_batch;
      a.page_elems = h->page_elems;
      a.kb = h->kb;
      a.vb = h->vb;
      a.slots = slots;
      a.ctx_len = h->ctx_len;
      a.plan = h->plan;
      a.seg_start = h->seg_start;
      a.chunk_base = h->chunk_base;
      a.seg_desc = h->seg_desc;
      a.wg_range = h->wg_range;
      a.n_seg = n_req * nkv * splits;
      a.chunk_min = kAttnChunkMin;
      a.chunk_max = kAttnChunkMax;
      a.o_part = h->o_part;
      a.m_part = h->m_part;
      a.l_part = h->l_part;
      a.n_kv = nkv;
      a.R = R;
      a.Rpad = h->Rpad;
      a.QRpad = h->QRpad;
      a.rows_per_split = rows_split;
      a.splits = splits;
      a.ctx_alloc = h->ctx_alloc;
      a.scale_log2 = 1.4426950408889634f / sqrtf((float)d);
      a.causal = c.causal_block ? 1 : 0;
      {
        Phase ph(h, s, DFLASH_PH_ATTN);
        if (h->attn_waves) launch_attn_waves(d, qrt, a, h->attn_wg, s);
        else launch_attn(d, qrt, a, h->attn_wg, s);
      }
      AttnCombineArgs cb;
      cb.o_part = h->o_part;
      cb.m_part = h->m_part;
      cb.l_part = h->l_part;
      cb.seg_start = h->seg_start;
      cb.chunk_base = h->chunk_base;
      cb.out = h->attn_out;
      cb.n_kv = nkv;
      cb.group = g;
      cb.R = R;
      cb.rows_per_split = rows_split;
      cb.splits = splits;
      cb.QRT16 = 16 * qrt;
      cb.q_dim = qdim;
      cb.D = d;
      cb.chunk_min = kAttnChunkMin;
      cb.chunk_max = kAttnChunkMax;
      cb.wave_plan = h->attn_waves ? h->plan : nullptr;
      Phase ph(h, s, DFLASH_PH_ATTN_COMBINE);
      launch_attn_combine(dt, d, cb, dim3(n_req, nkv * splits, (rows_split + 15) / 16), s);
    }
    // output projection + residual (with a DFlash 2 convolution: applied in the norm pass)
    const void* post_a = c.conv_group > 0 ? L.attn_conv_post_base : nullptr;
    // without DFlash 2 convolutions a K-split output product leaves its partials
    // to the post-attention norm pass, which adds them to X and normalises in one pass
    const bool keep_o = !post_a && H <= 8192;
    const GemmShape og = sublayer_out(h, s, M, h->attn_out, qdim, W.o, W.s_o, post_a ? W.conv_ap : nullptr,
                                      DFLASH_PH_O, keep_o, /*balance=*/true);
    const GemmShape o_pend = keep_o ? og : GemmShape{1, 0, 0};
    norm_stage(h, s, M, 0, K, R, L.post_norm, post_a, &o_pend, W.s_o);
    // DFlash 2: dynamic convolution of the MLP sub-layer's input
    const void* mlp_in = h->hbuf;
    if (c.conv_group > 0) {
      conv_stage(h, s, M, R, W.conv_m, W.s_cm, L.mlp_conv_base, L.post_norm);
      mlp_in = h->hbuf2;
    }
    // SwiGLU MLP
    {
      GemmArgs ga = gemm_a1(mlp_in, H, M, 2 * F, H);
      ga.out_scale = W.s_gu;
      ga.b_ptr[0] = W.gate;
      ga.b_ptr[1] = W.up;
      ga.b_interleave = 1;
      ga.b_ld = H;
      EpiSwiGLU<f16_t>::Params ps{(f16_t*)h->act, F, F, h->err};
      {
        Phase ph(h, s, DFLASH_PH_GATE_UP);
        launch_gemm(h->op, EPI_SWIGLU, ga, &ps, plan_gemm(h->op, M, 2 * F, H, h->num_cus), h->partials,
                    h->partials_elems, s);
      }
      post_m = c.conv_group > 0 ? L.mlp_conv_post_base : nullptr;
      // without DFlash 2 convolutions a K-split down product leaves its partials
      // to the next norm pass, which adds them to X and normalises in one pass
      const bool keep = c.conv_group == 0 && H <= 8192;
      const GemmShape gs = sublayer_out(h, s, M, h->act, F, W.down, W.s_down, post_m ? W.conv_mp : nullptr,
                                        DFLASH_PH_DOWN, keep);
      down = keep ? gs : GemmShape{1, 0, 0};   // pending only when the partials were kept
      down_scale = W.s_down;
    }
    if (l + 1 < c.n_layers) norm_stage(h, s, M, 0, K, R, h->layers[l + 1].in_norm, post_m, &down, down_scale);
  }
  // final norm on the K mask rows, LM head with streaming statistics
  const int rows = n_req * K;
  norm_stage(h, s, rows, 1, K, R, h->final_norm, post_m, &down, down_scale);
  const float T = p->temperature;
  const bool need_logits = o->logits || T > 0.f || p->top_k > 0 || p->tree_budget > 0 || c.sel_rank > 0;
  float* logits = o->logits ? o->logits : (need_logits ? h->logits_ws : nullptr);
  {
    GemmArgs ga = gemm_a1(h->hbuf, H, rows, V, H);
    ga.out_scale = h->s_lm;
    set_b(ga, {{h->lm, V}}, H);
    EpiLMHead::Params pl;
    pl.logits = logits;
    pl.ld = V;
    pl.tile_max = h->tmax;
    pl.tile_sum = h->tsum;
    pl.tile_arg = h->targ;
    pl.n_tiles = h->n_vtiles;
    pl.inv_temp = T > 0.f ? 1.0f / T : 1.0f;
    pl.out_mult = c.output_multiplier;
    pl.softcap = c.logit_softcap;
    GemmPlan gp = plan_gemm(h->op, rows, V, H, h->num_cus, /*wide=*/true, /*big_ok=*/true);
    gp.splits = 1;   // the vocabulary gives plenty of tiles; statistics are per output tile
    Phase ph(h, s, DFLASH_PH_LM_HEAD);
    launch_gemm(h->op, EPI_LMHEAD, ga, &pl, gp, h->partials, h->partials_elems, s);
  }
  select_stage(h, s, n_req, slots, anchor_ids, logits, p, o);
  if (c.sel_rank > 0)
    selector_stage(h, s, n_req, K, slots, anchor_ids, logits, h->hbuf, T, p->seed, p->step, o->draft_ids, o->cand_ids,
                   o->cand_probs);
  if (o->hidden) launch_to_f32(c.dtype, (int64_t)rows * H, h->hbuf, o->hidden, s);
  return hipGetLastError() == hipSuccess ? DFLASH_OK : DFLASH_E_HIP;
}

__global__ void lm_stats_from_logits_kernel(int V, int n_tiles, int tile_w, const float* logits, float inv_temp,
                                            float* tmax, float* tsum, int32_t* targ) {
  // one wave per (row, tile_w-column tile): the same statistics the LM-head epilogue produces
  const int m = blockIdx.y, t = blockIdx.x, lane = threadIdx.x;
  const int per = tile_w / 64;
  float best = -INFINITY;
  int arg = 0x7fffffff;
  float s[4];
  for (int q = 0; q < per; ++q) {
    const int n = t * tile_w + lane + 64 * q;
    s[q] = -INFINITY;
    if (n < V) {
      s[q] = logits[(int64_t)m * V + n] * inv_temp;
      if (s[q] > best) { best = s[q]; arg = n; }
    }
  }
  const float mx = wave_max(best);
  int cand = best == mx ? arg : 0x7fffffff;
  for (int o = 32; o > 0; o >>= 1) cand = min(cand, __shfl_xor(cand, o, 64));
  float e = 0.f;
  for (int q = 0; q < per; ++q)
    if (t * tile_w + lane + 64 * q < V) e += expf(s[q] - mx);
  e = wave_sum(e);
  if (lane == 0) {
    tmax[(int64_t)m * n_tiles + t] = mx;
    tsum[(int64_t)m * n_tiles + t] = e;
    targ[(int64_t)m * n_tiles + t] = cand;
  }
}

int dflash_select_from_logits(dflash_handle* h, void* stream, int32_t n_req, const int32_t* slots,
                              const int32_t* anchor_ids, const float* logits, const dflash_draft_params* p,
                              const dflash_draft_outputs* o) {
  if (!h) return DFLASH_E_INVALID;
  int rc = validate_draft(h, n_req, p, o);
  if (rc) return rc;
  if (n_req == 0) return DFLASH_OK;
  if (!slots || !logits) return DFLASH_E_INVALID;
  hipStream_t s = S(stream);
  const float T = p->temperature;
  const int rows = n_req * p->K;
  dim3 grid(h->n_vtiles, rows);
  {
    Phase ph(h, s, DFLASH_PH_SELECT);
    lm_stats_from_logits_kernel<<<grid, 64, 0, s>>>(h->cfg.vocab, h->n_vtiles, h->lm_tile, logits,
                                                     T > 0.f ? 1.0f / T : 1.0f, h->tmax, h->tsum, h->targ);
  }
  select_stage(h, s, n_req, slots, anchor_ids, logits, p, o);
  return hipGetLastError() == hipSuccess ? DFLASH_OK : DFLASH_E_HIP;
}

}  // extern "C"

namespace {
// Truncated rows of `rows` logits rows (scratch rows [row0, row0 + rows)): statistics,
// top-k, then top-p; kept ids / probabilities land in kp_ids / kp_probs at row0.
void truncate_rows(dflash_handle* h, hipStream_t s, int row0, int rows, const float* logits, float T) {
  const int V = h->cfg.vocab, nt = h->n_vtiles;
  const float inv_t = 1.0f / T;
  const int64_t o = (int64_t)row0 * nt;
  // one pass: row max / log-sum and the 128-id tile maxima (the LM head's tile width)
  launch_row_stats(rows, V, logits, inv_t, h->vt_max + o, nt, h->vrow_max + row0, h->vrow_lse + row0, 1, 1 << 30,
                   1 << 30, 0, 1, s);
  launch_topk(rows, V, h->trunc_k, logits, h->vt_max + o, nt, h->lm_tile, inv_t, h->vrow_max + row0,
              h->vrow_lse + row0, h->tr_ids + (int64_t)row0 * h->trunc_k, h->tr_probs + (int64_t)row0 * h->trunc_k, s);
  launch_trunc_rows(rows, h->trunc_k, h->trunc_p, h->tr_ids + (int64_t)row0 * h->trunc_k,
                    h->tr_probs + (int64_t)row0 * h->trunc_k, h->kp_ids + (int64_t)row0 * h->trunc_k,
                    h->kp_probs + (int64_t)row0 * h->trunc_k, s);
}
}  // namespace

extern "C" {

int dflash_set_page_table(dflash_handle* h, const int32_t* table) {
  if (!h) return DFLASH_E_INVALID;
  if (h->cfg.page_size == 0) return DFLASH_E_UNSUPPORTED;
  h->page_table = table;
  return DFLASH_OK;
}

int dflash_set_sampling(dflash_handle* h, int32_t top_k, float top_p) {
  if (!h) return DFLASH_E_INVALID;
  if (top_k < 0 || top_k > 64 || !(top_p > 0.f && top_p <= 1.f)) return DFLASH_E_INVALID;
  if (top_k == 0 && top_p < 1.f && !draw_vocab_ok(h->cfg.vocab)) return DFLASH_E_CAPACITY;
  if (top_k > h->cfg.vocab) return DFLASH_E_CAPACITY;
  h->trunc_k = top_k;
  h->trunc_p = top_p;
  return DFLASH_OK;
}

int dflash_verify(dflash_handle* h, void* stream, int32_t n_req, int32_t K, const int32_t* slots,
                  const int32_t* draft_ids, const float* draft_logits, const float* target_logits, float temperature,
                  uint64_t seed, uint64_t step, int32_t* out_tokens, int32_t* out_len, int32_t* accept_len,
                  int32_t* next_anchor) {
  if (!h || n_req < 0) return DFLASH_E_INVALID;
  if (n_req == 0) return DFLASH_OK;
  const dflash_config& c = h->cfg;
  if (n_req > c.max_batch || K < 1 || K > c.max_k) return DFLASH_E_CAPACITY;
  if (!draft_ids || !target_logits || !out_tokens || !out_len || !accept_len) return DFLASH_E_INVALID;
  if (!(temperature >= 0.f)) return DFLASH_E_INVALID;
  if (temperature > 0.f && (!draft_logits || !slots)) return DFLASH_E_INVALID;
  if (temperature > 0.f && !draw_vocab_ok(c.vocab)) return DFLASH_E_CAPACITY;
  hipStream_t s = S(stream);
  Phase ph(h, s, DFLASH_PH_VERIFY);
  if (temperature == 0.f) {
    launch_verify_greedy(n_req, K, c.vocab, draft_ids, target_logits, h->post, out_tokens, out_len, accept_len,
                         next_anchor, s);
  } else if (h->trunc_k > 0) {
    // target rows [0, n(K+1)) and draft rows after them, each truncated
    const int nt = n_req * (K + 1), nd = n_req * K;
    truncate_rows(h, s, 0, nt, target_logits, temperature);
    truncate_rows(h, s, nt, nd, draft_logits, temperature);
    const int tk = h->trunc_k;
    launch_verify_sparse(n_req, K, tk, tk, slots, draft_ids, h->kp_ids, h->kp_probs, h->kp_ids + (int64_t)nt * tk,
                         h->kp_probs + (int64_t)nt * tk, seed, step, out_tokens, out_len, accept_len, next_anchor,
                         h->err, s);
  } else {
    launch_verify_rejection(n_req, K, c.vocab, slots, draft_ids, draft_logits, target_logits, 1.0f / temperature,
                            seed, step, h->vstats, h->vacc, h->vchunks, out_tokens, out_len, accept_len,
                            next_anchor, h->err, s, h->trunc_p < 1.f ? h->nuc : nullptr, h->trunc_p);
  }
  return hipGetLastError() == hipSuccess ? DFLASH_OK : DFLASH_E_HIP;
}

int dflash_verify_tree(dflash_handle* h, void* stream, int32_t n_req, int32_t K, int32_t n_nodes,
                       const int32_t* slots, const int32_t* tree_tokens, const int32_t* tree_parents,
                       const float* target_logits, float temperature, uint64_t seed, uint64_t step,
                       int32_t* out_tokens, int32_t* out_len, int32_t* accept_len, int32_t* next_anchor,
                       int32_t* path_nodes) {
  if (!h || n_req < 0) return DFLASH_E_INVALID;
  if (n_req == 0) return DFLASH_OK;
  const dflash_config& c = h->cfg;
  if (n_req > c.max_batch || K < 1 || K > c.max_k || n_nodes < 1 || n_nodes > c.max_tree + 1)
    return DFLASH_E_CAPACITY;
  if (!tree_tokens || !tree_parents || !target_logits || !out_tokens || !out_len || !accept_len)
    return DFLASH_E_INVALID;
  if (!(temperature >= 0.f)) return DFLASH_E_INVALID;
  if (temperature > 0.f && !slots) return DFLASH_E_INVALID;
  if (temperature > 0.f && (int64_t)tree_walk_segments(c.vocab) * 8 > 65536) return DFLASH_E_CAPACITY;
  hipStream_t s = S(stream);
  Phase ph(h, s, DFLASH_PH_VERIFY);
  launch_verify_tree(n_req, n_nodes, K + 1, c.vocab, slots, tree_tokens, tree_parents, target_logits, temperature,
                     seed, step, out_tokens, out_len, accept_len, next_anchor, path_nodes, h->err, s);
  return hipGetLastError() == hipSuccess ? DFLASH_OK : DFLASH_E_HIP;
}

int dflash_select_path(dflash_handle* h, void* stream, int32_t n_req, int32_t K, const int32_t* slots,
                       const int32_t* anchor_ids, const float* logits, const float* hidden, float temperature,
                       uint64_t seed, uint64_t step, int32_t* draft_ids, int32_t* cand_ids, float* cand_probs) {
  if (!h || n_req < 0) return DFLASH_E_INVALID;
  const dflash_config& c = h->cfg;
  if (c.sel_rank <= 0) return DFLASH_E_INVALID;
  if (n_req == 0) return DFLASH_OK;
  if (n_req > c.max_batch || K < 1 || K > c.max_k) return DFLASH_E_CAPACITY;
  if (!slots || !anchor_ids || !logits || !hidden || !draft_ids || !cand_ids || !cand_probs) return DFLASH_E_INVALID;
  if (!(temperature >= 0.f)) return DFLASH_E_INVALID;
  hipStream_t s = S(stream);
  const int rows = n_req * K;
  dflash_draft_params p{};
  p.K = K;
  p.temperature = temperature;
  p.seed = seed;
  p.step = step;
  dflash_draft_outputs o{};
  o.draft_ids = draft_ids;
  {
    Phase ph(h, s, DFLASH_PH_SELECT);
    lm_stats_from_logits_kernel<<<dim3(h->n_vtiles, rows), 64, 0, s>>>(c.vocab, h->n_vtiles, h->lm_tile, logits,
                                                                        temperature > 0.f ? 1.0f / temperature : 1.0f,
                                                                        h->tmax, h->tsum, h->targ);
  }
  select_stage(h, s, n_req, slots, anchor_ids, logits, &p, &o);
  launch_from_f32(c.dtype, (int64_t)rows * c.hidden, hidden, h->sel_hin, s);
  selector_stage(h, s, n_req, K, slots, anchor_ids, logits, h->sel_hin, temperature, seed, step, draft_ids, cand_ids,
                 cand_probs);
  return hipGetLastError() == hipSuccess ? DFLASH_OK : DFLASH_E_HIP;
}

int dflash_verify_subset(dflash_handle* h, void* stream, int32_t n_req, int32_t K, int32_t C, const int32_t* slots,
                         const int32_t* draft_ids, const int32_t* cand_ids, const float* cand_probs,
                         const float* target_logits, float temperature, uint64_t seed, uint64_t step,
                         int32_t* out_tokens, int32_t* out_len, int32_t* accept_len, int32_t* next_anchor) {
  if (!h || n_req < 0) return DFLASH_E_INVALID;
  if (n_req == 0) return DFLASH_OK;
  const dflash_config& c = h->cfg;
  if (n_req > c.max_batch || K < 1 || K > c.max_k) return DFLASH_E_CAPACITY;
  if (C < 1 || C > 64) return DFLASH_E_CAPACITY;
  if (!draft_ids || !target_logits || !out_tokens || !out_len || !accept_len) return DFLASH_E_INVALID;
  if (!(temperature >= 0.f)) return DFLASH_E_INVALID;
  hipStream_t s = S(stream);
  Phase ph(h, s, DFLASH_PH_VERIFY);
  if (temperature == 0.f) {
    launch_verify_greedy(n_req, K, c.vocab, draft_ids, target_logits, h->post, out_tokens, out_len, accept_len,
                         next_anchor, s);
  } else {
    if (!slots || !cand_ids || !cand_probs) return DFLASH_E_INVALID;
    if (!draw_vocab_ok(c.vocab)) return DFLASH_E_CAPACITY;
    if (h->trunc_k > 0) {   // the target's p truncated; q is the selector's own subset law
      truncate_rows(h, s, 0, n_req * (K + 1), target_logits, temperature);
      launch_verify_sparse(n_req, K, h->trunc_k, C, slots, draft_ids, h->kp_ids, h->kp_probs, cand_ids, cand_probs,
                           seed, step, out_tokens, out_len, accept_len, next_anchor, h->err, s);
      return hipGetLastError() == hipSuccess ? DFLASH_OK : DFLASH_E_HIP;
    }
    launch_verify_subset(n_req, K, C, c.vocab, slots, draft_ids, cand_ids, cand_probs, target_logits,
                         1.0f / temperature, seed, step, h->vstats, h->vacc, h->vchunks, out_tokens, out_len,
                         accept_len, next_anchor, h->err, s, h->trunc_p < 1.f ? h->nuc : nullptr, h->trunc_p);
  }
  return hipGetLastError() == hipSuccess ? DFLASH_OK : DFLASH_E_HIP;
}

int dflash_profile(dflash_handle* h, int32_t enable) {
  if (!h) return DFLASH_E_INVALID;
  h->prof = enable != 0;
  return DFLASH_OK;
}

int dflash_profile_read(dflash_handle* h, int32_t n, double* ms, int32_t* launches) {
  if (!h || n < 0) return DFLASH_E_INVALID;
  std::vector<double> acc(DFLASH_PH_COUNT, 0.0);
  std::vector<int32_t> cnt(DFLASH_PH_COUNT, 0);
  int rc = DFLASH_OK;
  for (auto& m : h->marks) {
    float t = 0.f;
    if (hipEventSynchronize(m.b) != hipSuccess || hipEventElapsedTime(&t, m.a, m.b) != hipSuccess) rc = DFLASH_E_HIP;
    acc[m.phase] += t;
    cnt[m.phase] += 1;
    h->event_pool.push_back(m.a);
    h->event_pool.push_back(m.b);
  }
  h->marks.clear();
  for (int i = 0; i < n && i < DFLASH_PH_COUNT; ++i) {
    if (ms) ms[i] = acc[i];
    if (launches) launches[i] = cnt[i];
  }
  return rc;
}

int dflash_get_error(dflash_handle* h, void* stream, int32_t* code) {
  if (!h || !code) return DFLASH_E_INVALID;
  if (hipStreamSynchronize(S(stream)) != hipSuccess) return DFLASH_E_HIP;
  int32_t v = 0;
  if (hipMemcpy(&v, h->err, 4, hipMemcpyDeviceToHost) != hipSuccess) return DFLASH_E_HIP;
  if (hipMemset(h->err, 0, 4) != hipSuccess) return DFLASH_E_HIP;
  *code = v;
  return DFLASH_OK;
}

int dflash_ctx_lens(dflash_handle* h, void* stream, int32_t* out_dev) {
  if (!h || !out_dev) return DFLASH_E_INVALID;
  return hipMemcpyAsync(out_dev, h->ctx_len, 4 * h->cfg.max_batch, hipMemcpyDeviceToDevice, S(stream)) == hipSuccess
             ? DFLASH_OK
             : DFLASH_E_HIP;
}

int dflash_copy_cache(dflash_handle* h, void* stream, int32_t layer, int32_t slot, int32_t start, int32_t n,
                      void* k_out, void* v_out) {
  if (!h || !k_out || !v_out) return DFLASH_E_INVALID;
  const dflash_config& c = h->cfg;
  if (layer < 0 || layer >= c.n_layers || slot < 0 || slot >= c.max_batch || start < 0 || n < 0 ||
      start + n > c.max_ctx)
    return DFLASH_E_INVALID;
  if (c.page_size > 0 && !h->page_table) return DFLASH_E_INVALID;
  launch_copy_cache(c.dtype, h->cache_k, h->cache_v, layer, slot, start, n, c.max_batch + 1, c.n_kv_heads, c.head_dim,
                    h->ctx_alloc, h->pages(), k_out, v_out, S(stream));
  return hipGetLastError() == hipSuccess ? DFLASH_OK : DFLASH_E_HIP;
}

int dflash_synth_target_logits(void* stream, int32_t n_req, int32_t K, int32_t vocab, const float* draft_logits,
                               float sigma, uint64_t seed, uint64_t step, float* out) {
  if (n_req < 0 || K < 1 || vocab < 1 || !draft_logits || !out) return DFLASH_E_INVALID;
  if (n_req == 0) return DFLASH_OK;
  launch_synth_target(n_req, K, vocab, draft_logits, sigma, seed, step, out, S(stream));
  return hipGetLastError() == hipSuccess ? DFLASH_OK : DFLASH_E_HIP;
}

int dflash_philox_uniforms(void* stream, int32_t n, uint64_t seed, uint32_t slot, uint64_t step, uint32_t purpose,
                           float* out) {
  if (n < 0 || (n > 0 && !out)) return DFLASH_E_INVALID;
  launch_philox_fill(n, seed, slot, step, purpose, out, S(stream));
  return hipGetLastError() == hipSuccess ? DFLASH_OK : DFLASH_E_HIP;
}

}  // extern "C"
