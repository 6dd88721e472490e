// GEMM epilogues.  Each receives a slab of ROWS rows of the output tile staged
// in LDS (fp32, row stride `ld`) and finishes the fused step that follows the
// product.
#pragma once
#include "common.h"
#include "kv_layout.h"

namespace dfl {

__device__ __forceinline__ float silu_f(float x) { return x / (1.0f + expf(-x)); }

// ---- plain store (fp32 or T) ----
template <typename OutT>
struct EpiStore {
  struct Params { OutT* out; int64_t ld; };
  template <int BN, int ROWS>
  __device__ static void apply(const Params& p, const float* st, int ld, int m0, int n0, int M, int N, int, int tid) {
    for (int idx = tid; idx < ROWS * BN; idx += 256) {
      const int r = idx / BN, c = idx % BN;
      const int m = m0 + r, n = n0 + c;
      if (m < M && n < N) p.out[(int64_t)m * p.ld + n] = from_f32<OutT>(st[r * ld + c]);
    }
  }
};

// ---- fp32 store split at a column: columns [0, split) to out, the rest to out2 ----
struct StoreSplitParams { float* out; int64_t ld; float* out2; int64_t ld2; int split; };
struct EpiStoreSplit {
  typedef StoreSplitParams Params;
  template <int BN, int ROWS>
  __device__ static void apply(const Params& p, const float* st, int ld, int m0, int n0, int M, int N, int, int tid) {
    for (int idx = tid; idx < ROWS * BN; idx += 256) {
      const int r = idx / BN, c = idx % BN;
      const int m = m0 + r, n = n0 + c;
      if (m < M && n < N) {
        if (n < p.split) p.out[(int64_t)m * p.ld + n] = st[r * ld + c];
        else p.out2[(int64_t)m * p.ld2 + (n - p.split)] = st[r * ld + c];
      }
    }
  }
};

// ---- residual add into the fp32 stream ----
// Four columns per thread and item; every item's X load is issued before the
// first add, so the loads' latencies overlap (the stores into X would otherwise
// order each load after the previous item's store).  N and ld are multiples of 4.
struct EpiResidualAdd {
  struct Params { float* x; int64_t ld; };
  // The X values of one ROWS-row slab, loadable ahead of the stage (a product
  // may load them before its main loop: X is written only by this epilogue,
  // each element by one thread).
  template <int BN, int ROWS>
  struct Pre {
    static constexpr int C4 = BN / 4, NV = ROWS * C4 / 256;
    static_assert(ROWS * C4 % 256 == 0, "whole items per thread");
    float4 xv[NV];
  };
  template <int BN, int ROWS>
  __device__ static void load(const Params& p, int m0, int n0, int M, int N, int tid, Pre<BN, ROWS>& pre) {
    constexpr int C4 = Pre<BN, ROWS>::C4;
#pragma unroll
    for (int j = 0; j < Pre<BN, ROWS>::NV; ++j) {
      const int idx = tid + j * 256, r = idx / C4, c = 4 * (idx % C4);
      const int m = m0 + r, n = n0 + c;
      pre.xv[j] = m < M && n < N ? *(const float4*)(p.x + (int64_t)m * p.ld + n) : make_float4(0.f, 0.f, 0.f, 0.f);
    }
  }
  template <int BN, int ROWS>
  __device__ static void add(const Params& p, const float* st, int ld, int m0, int n0, int M, int N, int tid,
                             const Pre<BN, ROWS>& pre) {
    constexpr int C4 = Pre<BN, ROWS>::C4;
#pragma unroll
    for (int j = 0; j < Pre<BN, ROWS>::NV; ++j) {
      const int idx = tid + j * 256, r = idx / C4, c = 4 * (idx % C4);
      const int m = m0 + r, n = n0 + c;
      if (m < M && n < N) {
        const float* sr = st + r * ld + c;
        *(float4*)(p.x + (int64_t)m * p.ld + n) =
            make_float4(pre.xv[j].x + sr[0], pre.xv[j].y + sr[1], pre.xv[j].z + sr[2], pre.xv[j].w + sr[3]);
      }
    }
  }
  template <int BN, int ROWS>
  __device__ static void apply(const Params& p, const float* st, int ld, int m0, int n0, int M, int N, int, int tid) {
    Pre<BN, ROWS> pre;
    load<BN, ROWS>(p, m0, n0, M, N, tid, pre);
    add<BN, ROWS>(p, st, ld, m0, n0, M, N, tid, pre);
  }
};

// ---- SwiGLU: tile columns [0, BN/2) are gate, [BN/2, BN) the matching up columns ----
template <typename OutT>
struct EpiSwiGLU {
  struct Params { OutT* out; int64_t ld; int F; int32_t* err; };
  template <int BN, int ROWS>
  __device__ static void apply(const Params& p, const float* st, int ld, int m0, int n0, int M, int, int, int tid) {
    constexpr int H = BN / 2;
    bool bad = false;
    for (int idx = tid; idx < ROWS * H; idx += 256) {
      const int r = idx / H, c = idx % H;
      const int m = m0 + r, f = n0 / 2 + c;
      if (m < M && f < p.F) {
        const float gt = st[r * ld + c], up = st[r * ld + H + c];
        p.out[(int64_t)m * p.ld + f] = store_cvt<OutT>(silu_f(gt) * up, bad);
      }
    }
    report_nonfinite(p.err, bad, tid);
  }
};

// Per-head RMSNorm + rotate-half RoPE of one head held in a staged row.
// Lanes [0, d/2) of a lane group handle the pairs (i, i + d/2).  G: gain storage type.
template <typename G>
__device__ __forceinline__ void norm_rope_pair(float& x1, float& x2, int i, int d, const G* gain, float eps,
                                               const float2* rope_row) {
  const float ss = group_sum(x1 * x1 + x2 * x2, d / 2);
  const float rs = rsqrtf(ss / (float)d + eps);
  x1 = x1 * rs * to_f32(gain[i]);
  x2 = x2 * rs * to_f32(gain[i + d / 2]);
  const float2 cs = rope_row[i];  // (cos, sin)
  const float y1 = x1 * cs.x - x2 * cs.y;
  const float y2 = x2 * cs.x + x1 * cs.y;
  x1 = y1;
  x2 = y2;
}

// ---- draft block: q | k | v projections -> head norm + RoPE -> attention layouts ----
// q rows go to qb[r][kv][i*R + j][d] (q head kv*g + i, block row j), k rows to
// kb[r][kv][Rpad * d] and v rows to vb[r][kv][Rpad * d], in the 32-key block
// order of the cache (kv_layout.h).
template <typename T>
struct EpiQKV {
  typedef typename WeightOf<T>::type W;
  struct Params {
    T* qb; T* kb; T* vb;
    const int32_t* slots; const int32_t* ctx_len;
    const W* q_gain; const W* k_gain;
    const float2* rope;      // [pos][d/2] (cos, sin)
    int R, group, n_kv, d, q_dim, kv_dim, QRpad, Rpad;
    float eps;
    int32_t* err;            // device error word (out-of-range 16-bit stores)
  };
  template <int BN, int ROWS>
  __device__ static void apply(const Params& p, const float* st, int ld, int m0, int n0, int M, int, int, int tid) {
    if (p.d == 128) run<128, BN, ROWS>(p, st, ld, m0, n0, M, tid);
    else run<64, BN, ROWS>(p, st, ld, m0, n0, M, tid);
  }
  // The items (row, head) of a wave are fixed at compile time, so every global
  // load they need -- slot, context length, RoPE pair -- is issued for all of
  // them before the first one is used.
  template <int D, int BN, int ROWS>
  __device__ static void run(const Params& p, const float* st, int ld, int m0, int n0, int M, int tid) {
    constexpr int HALF = D / 2, PER = 64 / HALF, HEADS = BN / D, ITEMS = ROWS * HEADS;
    constexpr int NIT = ITEMS / (4 * PER);
    static_assert(BN % D == 0 && ITEMS % (4 * PER) == 0, "whole items per wave");
    const int lane = tid & 63, wave = tid >> 6;
    const int sub = lane / HALF, i = lane % HALF;
    int m_[NIT], j_[NIT], req_[NIT], nb_[NIT];
    int pos_[NIT];
    float2 cs_[NIT];
#pragma unroll
    for (int k = 0; k < NIT; ++k) {
      const int it = (k * 4 + wave) * PER + sub;
      const int r = it / HEADS, hh = it % HEADS;
      m_[k] = m0 + r;
      req_[k] = m_[k] / p.R;
      j_[k] = m_[k] % p.R;
      nb_[k] = n0 + hh * D;
    }
    // rows past M load request 0's values (never used)
#pragma unroll
    for (int k = 0; k < NIT; ++k) pos_[k] = p.slots[m_[k] < M ? req_[k] : 0];
#pragma unroll
    for (int k = 0; k < NIT; ++k) pos_[k] = p.ctx_len[pos_[k]] + j_[k];
#pragma unroll
    for (int k = 0; k < NIT; ++k) cs_[k] = p.rope[(int64_t)pos_[k] * HALF + i];
    const float qg1 = to_f32(p.q_gain[i]), qg2 = to_f32(p.q_gain[i + HALF]);
    const float kg1 = to_f32(p.k_gain[i]), kg2 = to_f32(p.k_gain[i + HALF]);
    bool bad = false;
#pragma unroll
    for (int k = 0; k < NIT; ++k) {
      const int it = (k * 4 + wave) * PER + sub;
      const int r = it / HEADS, hh = it % HEADS;
      const int m = m_[k], req = req_[k], j = j_[k], nb = nb_[k];
      float x1 = st[r * ld + hh * D + i], x2 = st[r * ld + hh * D + i + HALF];
      if (nb < p.q_dim + p.kv_dim) {   // q or k head: RMSNorm + RoPE (every lane of the group reduces)
        const bool isq = nb < p.q_dim;
        const float ss = group_sum(x1 * x1 + x2 * x2, HALF);
        const float rs = rsqrtf(ss / (float)D + p.eps);
        x1 *= rs * (isq ? qg1 : kg1);
        x2 *= rs * (isq ? qg2 : kg2);
        const float2 cs = cs_[k];
        const float y1 = x1 * cs.x - x2 * cs.y, y2 = x2 * cs.x + x1 * cs.y;
        x1 = y1;
        x2 = y2;
        if (m >= M) continue;
        if (isq) {
          const int qh = nb / D, kv = qh / p.group, gi = qh % p.group;
          T* dst = p.qb + ((int64_t)(req * p.n_kv + kv) * p.QRpad + gi * p.R + j) * D;
          dst[i] = store_cvt<T>(x1, bad);
          dst[i + HALF] = store_cvt<T>(x2, bad);
        } else {
          const int kh = (nb - p.q_dim) / D;
          T* dst = p.kb + (int64_t)(req * p.n_kv + kh) * p.Rpad * D;
          dst[k_off(j, i, D)] = store_cvt<T>(x1, bad);
          dst[k_off(j, i + HALF, D)] = store_cvt<T>(x2, bad);
        }
      } else {
        if (m >= M) continue;
        const int vh = (nb - p.q_dim - p.kv_dim) / D;
        T* dst = p.vb + (int64_t)(req * p.n_kv + vh) * p.Rpad * D;
        dst[v_off(j, i, D)] = store_cvt<T>(x1, bad);
        dst[v_off(j, i + HALF, D)] = store_cvt<T>(x2, bad);
      }
    }
    report_nonfinite(p.err, bad, tid);
  }
};

// ---- context injection: per-layer k|v of the fused feature -> k-norm + RoPE -> cache ----
// Cache: K and V [layer][slot][kv][ctx_alloc * d], positions in 32-key blocks (kv_layout.h).
template <typename T>
struct EpiKVInject {
  typedef typename WeightOf<T>::type W;
  struct Params {
    T* cache_k; T* cache_v;
    const int32_t* row_slot; const int32_t* row_pos;   // per GEMM row (global row index)
    const W* const* k_gain;                              // device array [n_layers] of gains
    const float2* rope;
    int n_kv, d, kv_dim, max_batch;
    int64_t ctx_alloc;
    float eps;
    int layer0;                                          // first layer of this product
    KvPages pages;                                       // paged storage (table null: contiguous)
    int32_t* err;                                        // device error word (unmapped pages)
  };
  template <int BN, int ROWS>
  __device__ static void apply(const Params& p, const float* st, int ld, int m0, int n0, int M, int, int, int tid) {
    if (p.d == 128) run<128, BN, ROWS>(p, st, ld, m0, n0, M, tid);
    else run<64, BN, ROWS>(p, st, ld, m0, n0, M, tid);
  }
  // Lane r < ROWS first loads row r's slot and position; every wave then takes
  // its (row, head) K items, fixed at compile time, CH at a time, reading the
  // row's slot and position from that lane and issuing the chunk's remaining
  // global loads (cache location, RoPE pair, gains) before the first is used (a
  // loop over rows would wait for each row's loads in turn; CH bounds the
  // registers a chunk holds beside the accumulators).  V heads: lanes walk rows
  // (consecutive positions -> coalesced stores), waves walk columns.
  template <int D, int BN, int ROWS>
  __device__ static void run(const Params& p, const float* st, int ld, int m0, int n0, int M, int tid) {
    constexpr int HALF = D / 2, PER = 64 / HALF, HEADS = BN / D, ITEMS = ROWS * HEADS;
    constexpr int NIT = ITEMS / (4 * PER), CH = NIT < 2 ? NIT : 2;
    static_assert(BN % D == 0 && ITEMS % (4 * PER) == 0 && NIT % CH == 0 && ROWS <= 64, "whole items per wave");
    const int lane = tid & 63, wave = tid >> 6;
    const int sub = lane / HALF, i = lane % HALF;
    bool bad = false;
    const int mrow = m0 + lane;
    const int lslot = lane < ROWS && mrow < M ? p.row_slot[mrow] : -1;
    const int lpos = lslot >= 0 ? p.row_pos[mrow] : 0;
    auto head_of = [&](int hh, int& layer, bool& isv, int& head) {
      const int nb = n0 + hh * D;
      layer = nb / (2 * p.kv_dim);
      const int within = nb % (2 * p.kv_dim);
      isv = within >= p.kv_dim;
      head = (within % p.kv_dim) / D;
    };
#pragma unroll 1
    for (int k0 = 0; k0 < NIT; k0 += CH) {
      int r_[CH], hh_[CH], slot_[CH], pos_[CH], pin_[CH];
      int64_t hb_[CH];
      float2 cs_[CH];
      float g1_[CH], g2_[CH];
#pragma unroll
      for (int k = 0; k < CH; ++k) {
        const int it = ((k0 + k) * 4 + wave) * PER + sub;
        r_[k] = it / HEADS;
        hh_[k] = it % HEADS;
        int layer, head;
        bool isv;
        head_of(hh_[k], layer, isv, head);
        slot_[k] = __shfl(lslot, r_[k], 64);
        pos_[k] = __shfl(lpos, r_[k], 64);
        if (isv) slot_[k] = -1;
      }
#pragma unroll
      for (int k = 0; k < CH; ++k) {
        int layer, head;
        bool isv;
        head_of(hh_[k], layer, isv, head);
        hb_[k] = 0;
        pin_[k] = 0;
        if (slot_[k] >= 0 &&
            !kv_locate(p.pages, p.ctx_alloc * D, p.max_batch, p.n_kv, D, p.layer0 + layer, slot_[k], head, pos_[k],
                       &hb_[k], &pin_[k])) {
          if (i == 0) raise_error(p.err, ERR_PAGE);
          slot_[k] = -1;
        }
        cs_[k] = p.rope[(int64_t)pos_[k] * HALF + i];
        const W* gain = p.k_gain[layer];
        g1_[k] = to_f32(gain[i]);
        g2_[k] = to_f32(gain[i + HALF]);
      }
#pragma unroll
      for (int k = 0; k < CH; ++k) {
        int layer, head;
        bool isv;
        head_of(hh_[k], layer, isv, head);
        if (!isv) {
          // every lane of the row's group reduces, valid row or not
          float x1 = st[r_[k] * ld + hh_[k] * D + i], x2 = st[r_[k] * ld + hh_[k] * D + i + HALF];
          const float ss = group_sum(x1 * x1 + x2 * x2, HALF);
          const float rs = rsqrtf(ss / (float)D + p.eps);
          x1 *= rs * g1_[k];
          x2 *= rs * g2_[k];
          const float2 cs = cs_[k];
          const float y1 = x1 * cs.x - x2 * cs.y, y2 = x2 * cs.x + x1 * cs.y;
          if (slot_[k] >= 0) {
            T* dst = p.cache_k + hb_[k];
            dst[k_off(pin_[k], i, D)] = store_cvt<T>(y1, bad);
            dst[k_off(pin_[k], i + HALF, D)] = store_cvt<T>(y2, bad);
          }
        }
      }
    }
    // V heads
    constexpr int RPL = 64 / ROWS;   // columns handled at once by one wave
    const int r = lane % ROWS;
    const int vslot = __shfl(lslot, r, 64), vpos = __shfl(lpos, r, 64);
#pragma unroll
    for (int hh = 0; hh < HEADS; ++hh) {
      int layer, head;
      bool isv;
      head_of(hh, layer, isv, head);
      if (!isv || vslot < 0) continue;
      int64_t hb = 0;
      int pin = 0;
      if (!kv_locate(p.pages, p.ctx_alloc * D, p.max_batch, p.n_kv, D, p.layer0 + layer, vslot, head, vpos, &hb, &pin))
        continue;   // unmapped: flagged by the K half
      T* base = p.cache_v + hb;
      for (int c = wave * RPL + lane / ROWS; c < D; c += 4 * RPL)
        base[v_off(pin, c, D)] = store_cvt<T>(st[r * ld + hh * D + c], bad);
    }
    report_nonfinite(p.err, bad, tid);
  }
};

// ---- LM head: logits (optional store) + per-(row, 128-column tile) max / sum-exp / argmax ----
// The statistics tile is 128 columns whatever the GEMM tile: a BN-wide GEMM tile
// tn writes statistics tiles tn * BN/128 .. +BN/128-1.
constexpr int LM_STAT_TILE = 128;
struct EpiLMHead {
  struct Params {
    float* logits;           // [M][ld] or null
    int64_t ld;
    float* tile_max;         // [M][n_tiles]   (of z / T)
    float* tile_sum;         // [M][n_tiles]   sum exp(z/T - tile_max)
    int32_t* tile_arg;       // [M][n_tiles]
    int n_tiles;
    float inv_temp, out_mult, softcap;
  };
  template <int BN, int ROWS>
  __device__ static void apply(const Params& p, const float* st, int ld, int m0, int n0, int M, int N, int tn,
                               int tid) {
    static_assert(BN % LM_STAT_TILE == 0, "GEMM tile of whole statistics tiles");
    const int lane = tid & 63, wave = tid >> 6;
    for (int it = wave; it < ROWS * (BN / LM_STAT_TILE); it += 4) {
      const int r = it % ROWS, hs = it / ROWS;   // row, statistics tile inside the GEMM tile
      const int m = m0 + r;
      if (m >= M) continue;
      float best = -INFINITY;
      int arg = 0x7fffffff;
      float zz[LM_STAT_TILE / 64];
#pragma unroll
      for (int q = 0; q < LM_STAT_TILE / 64; ++q) {
        const int c = hs * LM_STAT_TILE + lane + 64 * q, n = n0 + c;
        float z = st[r * ld + c] * p.out_mult;
        if (p.softcap > 0.f) z = p.softcap * tanhf(z / p.softcap);
        zz[q] = z;
        if (n < N) {
          if (p.logits) p.logits[(int64_t)m * p.ld + n] = z;
          const float s = z * p.inv_temp;
          if (s > best) { best = s; arg = n; }
        }
      }
      const float mx = wave_max(best);
      int cand = (best == mx) ? arg : 0x7fffffff;
#pragma unroll
      for (int o = 32; o > 0; o >>= 1) cand = min(cand, __shfl_xor(cand, o, 64));
      float e = 0.f;
#pragma unroll
      for (int q = 0; q < LM_STAT_TILE / 64; ++q) {
        const int n = n0 + hs * LM_STAT_TILE + lane + 64 * q;
        if (n < N) e += expf(zz[q] * p.inv_temp - mx);
      }
      e = wave_sum(e);
      const int t = tn * (BN / LM_STAT_TILE) + hs;
      if (lane == 0 && t < p.n_tiles) {
        const int64_t o = (int64_t)m * p.n_tiles + t;
        p.tile_max[o] = mx;
        p.tile_sum[o] = e;
        p.tile_arg[o] = cand;
      }
    }
  }
};

}  // namespace dfl
