// Row-wise and selection kernels of the drafter hot path: RoPE table, block
// embedding, RMSNorm, injection row tables, LM-head row statistics, sampling,
// top-k, prefix tree, verification.
#include <algorithm>

#include "ops.h"

namespace dfl {

// ---- block reductions (256 threads) ----
__device__ __forceinline__ float block_sum(float v, float* red) {
  v = wave_sum(v);
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  __syncthreads();
  if (lane == 0) red[w] = v;
  __syncthreads();
  float t = 0.f;
  for (int i = 0; i < (int)(blockDim.x >> 6); ++i) t += red[i];
  return t;
}

// ---------------------------------------------------------------------------
// RoPE table: (cos, sin) of pos * theta^(-2i/d), angle formed and reduced in fp64.
// ---------------------------------------------------------------------------
__global__ void rope_table_kernel(float2* table, int n_pos, int d, double theta) {
  const int half = d / 2;
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= (int64_t)n_pos * half) return;
  const int p = (int)(idx / half), i = (int)(idx % half);
  const double inv = pow(theta, -2.0 * (double)i / (double)d);
  double ang = fmod((double)p * inv, 6.283185307179586476925286766559);
  table[idx] = make_float2((float)cos(ang), (float)sin(ang));
}

// Four values of one row, gain-scaled and stored as one 8- or 16-byte write.
__device__ __forceinline__ void store4(float* p, float a, float b, float c, float d) {
  *(float4*)p = make_float4(a, b, c, d);
}
__device__ __forceinline__ void store4(bf16_t* p, float a, float b, float c, float d) {
  bf16_t v[4] = {(bf16_t)a, (bf16_t)b, (bf16_t)c, (bf16_t)d};
  *(uint2*)p = *(const uint2*)v;
}
__device__ __forceinline__ void store4(f16_t* p, float a, float b, float c, float d) {
  f16_t v[4] = {(f16_t)a, (f16_t)b, (f16_t)c, (f16_t)d};
  *(uint2*)p = *(const uint2*)v;
}
__device__ __forceinline__ float4 load4f(const float* p) { return *(const float4*)p; }
__device__ __forceinline__ float4 load4f(const bf16_t* p) {
  const uint2 u = *(const uint2*)p;
  const bf16_t* v = (const bf16_t*)&u;
  return make_float4((float)v[0], (float)v[1], (float)v[2], (float)v[3]);
}

// ---------------------------------------------------------------------------
// Block embedding [P2 §2.2; P4 §4]: row r*R + j holds the anchor (j = 0) or the
// mask token (j >= 1), embedded and scaled; then the first layer's RMSNorm.
// ---------------------------------------------------------------------------
template <typename C>
__global__ __launch_bounds__(256) void embed_norm_kernel(int R, const int32_t* anchors, int mask_id, int vocab,
                                                          const typename WeightOf<C>::type* embed,
                                                          const typename WeightOf<C>::type* mask_emb, float scale, int H,
                                                          float* X, const typename WeightOf<C>::type* gain, C* h_out,
                                                          float eps, int32_t* err, float* rs_out) {
  __shared__ float red[4];
  const int m = blockIdx.x;
  const int r = m / R, j = m % R;
  int id = j == 0 ? anchors[r] : mask_id;
  if (id < 0 || id >= vocab) {
    if (threadIdx.x == 0) raise_error(err, ERR_BAD_TOKEN);
    id = 0;
  }
  const auto* e = (j > 0 && mask_emb) ? mask_emb : embed + (int64_t)id * H;
  float* xr = X + (int64_t)m * H;
  C* hr = h_out + (int64_t)m * H;
  // four elements per access when the caller's rows allow it (H is a multiple of 128)
  constexpr uintptr_t A4 = 4 * sizeof(*e) - 1;
  const bool vec = (((uintptr_t)e | (uintptr_t)gain) & A4) == 0;
  float ss = 0.f;
  if (vec) {
    for (int c = threadIdx.x * 4; c < H; c += 1024) {
      const float4 v = load4f(e + c);
      const float4 x = make_float4(v.x * scale, v.y * scale, v.z * scale, v.w * scale);
      *(float4*)(xr + c) = x;
      ss += x.x * x.x + x.y * x.y + x.z * x.z + x.w * x.w;
    }
  } else {
    for (int c = threadIdx.x; c < H; c += 256) {
      const float v = to_f32(e[c]) * scale;
      xr[c] = v;
      ss += v * v;
    }
  }
  ss = block_sum(ss, red);
  const float rs = rsqrtf(ss / (float)H + eps);
  if (rs_out && threadIdx.x == 0) rs_out[m] = rs;
  if (vec) {
    for (int c = threadIdx.x * 4; c < H; c += 1024) {
      const float4 x = *(const float4*)(xr + c), g = load4f(gain + c);
      store4(hr + c, x.x * rs * g.x, x.y * rs * g.y, x.z * rs * g.z, x.w * rs * g.w);
    }
  } else {
    for (int c = threadIdx.x; c < H; c += 256) hr[c] = from_f32<C>(xr[c] * rs * to_f32(gain[c]));
  }
}


// RMSNorm of fp32 rows, one 256-thread work-group per row (H a multiple of 4):
// out[o] = x * rsqrt(mean(x^2) + eps) * gain, x = X row (map_mask ? (o / K) * R + 1 + o % K : o).
// Rows at or past (*n_valid - valid_base) are skipped when n_valid is given.
// rs_out (or null) receives each row's rsqrt(mean(x^2) + eps).
template <typename C>
__global__ __launch_bounds__(256) void rmsnorm_kernel(int n_rows, int H, const float* X, int map_mask, int K, int R,
                                                        const typename WeightOf<C>::type* gain, C* h_out, float eps,
                                                        const int32_t* n_valid, int valid_base, float* rs_out) {
  __shared__ float red[4];
  const int o = blockIdx.x;
  if (o >= n_rows) return;
  if (n_valid && o >= *n_valid - valid_base) return;   // uniform over the work-group
  const int src = map_mask ? (o / K) * R + 1 + (o % K) : o;
  const float* x = X + (int64_t)src * H;
  float ss = 0.f;
  for (int c = threadIdx.x * 4; c < H; c += 1024) {
    const float4 v = load4f(x + c);
    ss += v.x * v.x + v.y * v.y + v.z * v.z + v.w * v.w;
  }
  ss = block_sum(ss, red);
  const float rs = rsqrtf(ss / (float)H + eps);
  if (rs_out && threadIdx.x == 0) rs_out[o] = rs;
  C* y = h_out + (int64_t)o * H;
  for (int c = threadIdx.x * 4; c < H; c += 1024) {
    const float4 v = load4f(x + c), gn = load4f(gain + c);
    store4(y + c, v.x * rs * gn.x, v.y * rs * gn.y, v.z * rs * gn.z, v.w * rs * gn.w);
  }
}

// The residual add of a product whose K split left its partials in place (fp32
// [splits][.][ld], summed in split order and scaled, as the split-K reduction
// does), fused with the RMSNorm that follows it: the row of X is updated and
// normalised as in rmsnorm_kernel (same row mapping; only the mapped rows of X
// are updated).  One 256-thread work-group per row; H <= 8192.
template <typename C>
__global__ __launch_bounds__(256) void partials_add_norm_kernel(int n_rows, int H, float* X, int map_mask, int K, int R,
                                                                  const float* P, int ld, int splits,
                                                                  int64_t split_stride, float scale,
                                                                  const typename WeightOf<C>::type* gain, C* h_out,
                                                                  float eps) {
  __shared__ float red[4];
  constexpr int MAXV = 8;
  const int out = blockIdx.x;
  if (out >= n_rows) return;
  const int m = map_mask ? (out / K) * R + 1 + (out % K) : out;
  float* x = X + (int64_t)m * H;
  const float* p = P + (int64_t)m * ld;
  float4 v[MAXV];
  float ss = 0.f;
#pragma unroll
  for (int i = 0; i < MAXV; ++i) {
    const int c = threadIdx.x * 4 + i * 1024;
    if (c < H) {
      float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
      for (int sp = 0; sp < splits; ++sp) {
        const float4 q = load4f(p + sp * split_stride + c);
        acc.x += q.x;
        acc.y += q.y;
        acc.z += q.z;
        acc.w += q.w;
      }
      const float4 a = load4f(x + c);
      v[i] = make_float4(a.x + acc.x * scale, a.y + acc.y * scale, a.z + acc.z * scale, a.w + acc.w * scale);
      *(float4*)(x + c) = v[i];
      ss += v[i].x * v[i].x + v[i].y * v[i].y + v[i].z * v[i].z + v[i].w * v[i].w;
    }
  }
  ss = block_sum(ss, red);
  const float rs = rsqrtf(ss / (float)H + eps);
  C* y = h_out + (int64_t)out * H;
#pragma unroll
  for (int i = 0; i < MAXV; ++i) {
    const int c = threadIdx.x * 4 + i * 1024;
    if (c < H) {
      const float4 gn = load4f(gain + c);
      store4(y + c, v[i].x * rs * gn.x, v[i].y * rs * gn.y, v[i].z * rs * gn.z, v[i].w * rs * gn.w);
    }
  }
}

// DFlash 2 [P2 §3.2.3], convolution after a sub-layer, fused with the RMSNorm
// that follows it: the sub-layer output o (fp32 [M, H], before the residual add)
// is convolved over the block rows, y_m = (base0 + c0_m) * o_m + (base1 + c1_m) *
// o_{m-1} (o_{m-1} = 0 on a block's first row, corrections corr [M, 2H/G] shared
// by groups of G channels), added to X, and the updated row normalised as in
// rmsnorm_kernel (same row mapping; only the mapped rows of X are updated).
template <typename C>
__global__ __launch_bounds__(256) void conv_post_norm_kernel(int n_rows, int H, int G, float* X, int map_mask, int K,
                                                               int R, const float* o, const float* corr,
                                                               const typename WeightOf<C>::type* base,
                                                               const typename WeightOf<C>::type* gain, C* h_out,
                                                               float eps, float* rs_out) {
  __shared__ float red[4];
  const int out = blockIdx.x;   // one 256-thread work-group per row
  if (out >= n_rows) return;
  const int m = map_mask ? (out / K) * R + 1 + (out % K) : out;
  const bool first = m % R == 0;
  const int ng = H / G;
  float* x = X + (int64_t)m * H;
  const float* om = o + (int64_t)m * H;
  const float* cr = corr + (int64_t)m * 2 * ng;
  float ss = 0.f;
  for (int c = threadIdx.x * 4; c < H; c += 1024) {   // G is a multiple of 4: the four channels share a group
    float4 v = load4f(x + c);
    const float4 a = load4f(om + c), b0 = load4f(base + c), b1 = load4f(base + H + c);
    const float4 u = first ? make_float4(0.f, 0.f, 0.f, 0.f) : load4f(om - H + c);
    const float c0 = cr[c / G], c1 = cr[ng + c / G];
    v.x += (b0.x + c0) * a.x + (b1.x + c1) * u.x;
    v.y += (b0.y + c0) * a.y + (b1.y + c1) * u.y;
    v.z += (b0.z + c0) * a.z + (b1.z + c1) * u.z;
    v.w += (b0.w + c0) * a.w + (b1.w + c1) * u.w;
    *(float4*)(x + c) = v;
    ss += v.x * v.x + v.y * v.y + v.z * v.z + v.w * v.w;
  }
  ss = block_sum(ss, red);
  const float rs = rsqrtf(ss / (float)H + eps);
  if (rs_out && threadIdx.x == 0) rs_out[out] = rs;
  C* y = h_out + (int64_t)out * H;
  for (int c = threadIdx.x * 4; c < H; c += 1024) {   // this thread's own stores above
    const float4 v = *(const float4*)(x + c), gn = load4f(gain + c);
    store4(y + c, v.x * rs * gn.x, v.y * rs * gn.y, v.z * rs * gn.z, v.w * rs * gn.w);
  }
}

// ---------------------------------------------------------------------------
// Injection row tables.  Requests are appended in call order; a request whose
// rows do not fit its slot, or whose slot is invalid, is skipped and flagged.
// ---------------------------------------------------------------------------
__global__ void inject_scan_kernel(int n_req, const int32_t* slots, const int32_t* row_count, int32_t* ctx_len,
                                   int max_ctx, int max_batch, int64_t rows_upper, int32_t* req_off,
                                   int32_t* req_pos, int32_t* err) {
  if (threadIdx.x != 0) return;
  int64_t off = 0;
  for (int r = 0; r < n_req; ++r) {
    const int slot = slots[r];
    int cnt = row_count[r];
    req_off[r] = (int32_t)off;
    if (slot < 0 || slot >= max_batch) {
      raise_error(err, ERR_BAD_SLOT);
      req_pos[r] = 0;
      continue;
    }
    if (cnt < 0) {
      raise_error(err, ERR_ROWS);
      cnt = 0;
    }
    const int c0 = ctx_len[slot];
    if ((int64_t)c0 + cnt > max_ctx) {
      raise_error(err, ERR_CAPACITY);
      cnt = 0;
    }
    if (off + cnt > rows_upper) {
      raise_error(err, ERR_ROWS);
      cnt = 0;
    }
    req_pos[r] = c0;
    ctx_len[slot] = c0 + cnt;
    off += cnt;
  }
  req_off[n_req] = (int32_t)off;
}

// Source row of new row i of request r: row_start[r] + i, or, for a tree path,
// r * tree_stride + path_nodes[r * max_path + i] (a node index of that request's
// block of tree_stride rows; a node outside [0, tree_stride) is skipped and flagged).
__global__ void inject_fill_kernel(int n_req, int64_t rows_upper, const int32_t* slots, const int32_t* row_start,
                                   const int32_t* path_nodes, int max_path, int tree_stride,
                                   const int32_t* req_off, const int32_t* req_pos, int64_t max_row, int32_t* a_rows,
                                   int32_t* row_slot, int32_t* row_pos, int32_t* err) {
  const int64_t m = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (m >= rows_upper) return;
  if (m >= req_off[n_req]) {
    a_rows[m] = -1;
    row_slot[m] = -1;
    row_pos[m] = 0;
    return;
  }
  int lo = 0, hi = n_req - 1;  // last r with req_off[r] <= m
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (req_off[mid] <= m) lo = mid;
    else hi = mid - 1;
  }
  // skip empty requests that share the same offset
  while (lo + 1 <= n_req - 1 && req_off[lo + 1] <= m) ++lo;
  const int i = (int)(m - req_off[lo]);
  int64_t src;
  if (path_nodes) {
    const int node = i < max_path ? path_nodes[(int64_t)lo * max_path + i] : -1;
    src = node >= 0 && node < tree_stride ? (int64_t)lo * tree_stride + node : -1;
  } else {
    src = (int64_t)row_start[lo] + i;
  }
  if (src < 0 || src >= max_row) {  // not addressable: skip the row (its slot is left as it was)
    raise_error(err, ERR_ROWS);
    a_rows[m] = -1;
    row_slot[m] = -1;
    row_pos[m] = 0;
    return;
  }
  a_rows[m] = (int32_t)src;
  row_slot[m] = slots[lo];
  row_pos[m] = req_pos[lo] + i;
}

// ---------------------------------------------------------------------------
// LM-head rows: merge tile statistics (fixed tile order).
// row_max = max z/T, row_lse = log sum exp(z/T - row_max), argmax (lowest id on ties).
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(64) void row_finalize_kernel(int n_tiles, const float* tmax, const float* tsum,
                                                           const int32_t* targ, float* row_max, float* row_lse,
                                                           int32_t* argmax_out, float* out_row_max,
                                                           float* out_row_lse) {
  const int m = blockIdx.x, lane = threadIdx.x;
  const float* tm = tmax + (int64_t)m * n_tiles;
  const float* ts = tsum + (int64_t)m * n_tiles;
  const int32_t* ta = targ + (int64_t)m * n_tiles;
  float best = -INFINITY;
  int arg = 0x7fffffff;
  for (int t = lane; t < n_tiles; t += 64) {
    const float v = tm[t];
    if (v > best) { best = v; arg = ta[t]; }   // ascending tiles: first max per lane has the lowest id
  }
  const float M = wave_max(best);
  int cand = best == M ? arg : 0x7fffffff;
  for (int o = 32; o > 0; o >>= 1) cand = min(cand, __shfl_xor(cand, o, 64));
  // fixed-order sum: each lane a contiguous range, then a tree over lanes
  const int per = (n_tiles + 63) / 64;
  float s = 0.f;
  for (int t = lane * per; t < min(n_tiles, (lane + 1) * per); ++t) s += ts[t] * expf(tm[t] - M);
  s = wave_sum(s);
  if (lane == 0) {
    const float lse = logf(s);
    row_max[m] = M;
    row_lse[m] = lse;
    if (argmax_out) argmax_out[m] = cand;
    if (out_row_max) out_row_max[m] = M;
    if (out_row_lse) out_row_lse[m] = lse;
  }
}

// ---------------------------------------------------------------------------
// Inverse-CDF draft sampling [P2 §2.2]: the smallest id c
// with sum_{id<=c} exp(z_id/T - M) > u * S, with u = Philox(seed; j+1, slot,
// step, 0).  The sum runs over the LM-head tile sums (ascending tiles), then
// inside the selected tile (ascending ids).
// ---------------------------------------------------------------------------
__device__ __forceinline__ float block_incl_scan(float v, float* sh) {
  // inclusive scan over 256 threads in thread order
  const int t = threadIdx.x, lane = t & 63, w = t >> 6;
  float x = v;
  for (int o = 1; o < 64; o <<= 1) {
    const float y = __shfl_up(x, o, 64);
    if (lane >= o) x += y;
  }
  __syncthreads();
  if (lane == 63) sh[w] = x;
  __syncthreads();
  float add = 0.f;
  for (int i = 0; i < w; ++i) add += sh[i];
  return x + add;
}

__global__ __launch_bounds__(256) void sample_kernel(int K, const int32_t* slots, uint64_t seed, uint64_t step,
                                                      float inv_temp, const float* logits, int V, int n_tiles,
                                                      int tile_w, const float* tmax, const float* tsum, const float* row_max,
                                                      int32_t* draft_ids) {
  __shared__ float sh[8];
  __shared__ int s_thread;
  __shared__ int s_tile;
  __shared__ float s_before;
  const int m = blockIdx.x;
  const int r = m / K, j = m % K;
  const float M = row_max[m];
  const float u = philox_uniform(seed, (uint32_t)slots[r], step, (uint32_t)(j + 1), PURPOSE_DRAFT);
  const int per = (n_tiles + 255) / 256;
  const int t0 = threadIdx.x * per, t1 = min(n_tiles, t0 + per);
  const float* tm = tmax + (int64_t)m * n_tiles;
  const float* ts = tsum + (int64_t)m * n_tiles;
  float w = 0.f;
  for (int t = t0; t < t1; ++t) w += ts[t] * expf(tm[t] - M);
  const float incl = block_incl_scan(w, sh);
  __shared__ float s_total;
  if (threadIdx.x == 255) s_total = incl;
  if (threadIdx.x == 0) s_thread = -1;
  __syncthreads();
  const float target = u * s_total;
  const float excl = incl - w;
  if (excl <= target && target < incl) s_thread = threadIdx.x;  // exactly one thread (ranges are disjoint)
  __syncthreads();
  if (threadIdx.x == 0 && s_thread < 0) {
    // rounding put the target on/after the total: take the last tile with mass
    int th = 255;
    s_thread = th;
  }
  __syncthreads();
  if ((int)threadIdx.x == s_thread) {
    float acc = excl;
    int tile = -1;
    float before = excl;
    int last_nz = -1;
    float last_before = excl;
    for (int t = t0; t < t1; ++t) {
      const float wt = ts[t] * expf(tm[t] - M);
      if (wt > 0.f) { last_nz = t; last_before = acc; }
      if (target < acc + wt && tile < 0) { tile = t; before = acc; }
      acc += wt;
    }
    if (tile < 0) {   // fall back to the last tile with mass (at or before this range)
      int t = last_nz;
      before = last_before;
      if (t < 0) {    // scan backwards over all tiles
        float a2 = 0.f;
        for (int q = 0; q < n_tiles; ++q) {
          const float wt = ts[q] * expf(tm[q] - M);
          if (wt > 0.f) { t = q; before = a2; }
          a2 += wt;
        }
      }
      tile = t;
    }
    s_tile = tile;
    s_before = before;
  }
  __syncthreads();
  if (threadIdx.x < 64) {
    // inside the chosen tile: lane l owns ids [tile*tile_w + l*epl, +epl), scanned in id order
    const int lane = threadIdx.x;
    const int tile = s_tile;
    const int epl = tile_w / 64;
    const float* z = logits + (int64_t)m * V;
    const int c0 = tile * tile_w + lane * epl;
    float e[4];
    float lsum = 0.f;
    for (int q = 0; q < epl; ++q) {
      const int c = c0 + q;
      e[q] = c < V ? expf(z[c] * inv_temp - M) : 0.f;
      lsum += e[q];
    }
    float x = lsum;
    for (int o = 1; o < 64; o <<= 1) {
      const float y = __shfl_up(x, o, 64);
      if (lane >= o) x += y;
    }
    float acc = s_before + (x - lsum);
    const float tgt = target;
    int pick = 0x7fffffff, lastp = -1;
    for (int q = 0; q < epl; ++q) {
      if (e[q] > 0.f) {
        if (pick == 0x7fffffff && tgt < acc + e[q]) pick = c0 + q;
        lastp = c0 + q;
      }
      acc += e[q];
    }
    for (int o = 32; o > 0; o >>= 1) pick = min(pick, __shfl_xor(pick, o, 64));
    if (pick == 0x7fffffff) {   // rounding: last id of the tile with weight
      for (int o = 32; o > 0; o >>= 1) lastp = max(lastp, __shfl_xor(lastp, o, 64));
      pick = lastp < 0 ? tile * tile_w : lastp;
    }
    if (lane == 0) draft_ids[m] = pick;
  }
}

// ---------------------------------------------------------------------------
// Top-k per row [P5 §3.2: softmax over the vocabulary, then top-k]: order by
// logit descending, ties by lower id.  Candidates are pruned with the LM-head
// tile maxima (the k largest tile maxima bound the k-th largest logit), then a
// radix select on 64-bit keys (orderable logit bits, inverted id) finds the
// exact k-th key; the selected k are sorted with a bitonic network.
// ---------------------------------------------------------------------------
__device__ __forceinline__ uint32_t f2key(float f) {
  const uint32_t b = __float_as_uint(f);
  return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
}
__device__ __forceinline__ uint64_t ckey(float f, int idx) {
  return ((uint64_t)f2key(f) << 32) | (uint64_t)(0xFFFFFFFFu - (uint32_t)idx);
}

static constexpr int TOPK_CAP = 4096;
static constexpr int TOPK_TILE_CAP = 512;   // listed candidate tiles (more: scan all tiles)

// k-th largest (1-based) composite key among n items provided by get(i).
template <class Get>
__device__ uint64_t radix_kth(int n, int k, Get get, uint32_t* hist, uint64_t* sh_prefix, int* sh_k) {
  uint64_t prefix = 0;
  int krem = k;
  for (int pass = 7; pass >= 0; --pass) {
    const int shift = pass * 8;
    for (int b = threadIdx.x; b < 256; b += blockDim.x) hist[b] = 0;
    __syncthreads();
    const uint64_t hmask = pass == 7 ? 0ull : (~0ull << (shift + 8));
    for (int i = threadIdx.x; i < n; i += blockDim.x) {
      const uint64_t key = get(i);
      if ((key & hmask) == (prefix & hmask)) atomicAdd(&hist[(key >> shift) & 255], 1u);
    }
    __syncthreads();
    if (threadIdx.x == 0) {
      int cum = 0, b = 255;
      for (; b > 0; --b) {
        if (cum + (int)hist[b] >= krem) break;
        cum += hist[b];
      }
      *sh_prefix = prefix | ((uint64_t)b << shift);
      *sh_k = krem - cum;
    }
    __syncthreads();
    prefix = *sh_prefix;
    krem = *sh_k;
    __syncthreads();
  }
  return prefix;
}

__global__ __launch_bounds__(256) void topk_kernel(int V, int k, const float* logits, const float* tmax, int n_tiles,
                                                    int tile_w, float inv_temp, const float* row_max, const float* row_lse,
                                                    int32_t* ids_out, float* probs_out) {
  __shared__ uint32_t hist[256];
  __shared__ uint64_t sh_prefix;
  __shared__ int sh_k;
  __shared__ uint64_t cand[TOPK_CAP];
  __shared__ int s_n;
  __shared__ uint64_t sel[512];
  const int m = blockIdx.x;
  const float* z = logits + (int64_t)m * V;
  const float* tm = tmax + (int64_t)m * n_tiles;
  const int kk = min(k, V);
  // threshold from the tile maxima (tile max is in z/T units: compare via the same scaling).
  // With fewer tiles than k the maxima bound nothing: every element is a candidate.
  uint32_t thr = 0;
  if (kk <= n_tiles) {
    const uint64_t tkey = radix_kth(n_tiles, kk, [&](int i) { return ckey(tm[i], i); }, hist, &sh_prefix, &sh_k);
    thr = (uint32_t)(tkey >> 32);
  }
  // tiles whose maximum reaches the threshold, listed in parallel (ascending order is not needed:
  // the selection below is by key), then their elements scanned one tile per pass
  __shared__ int tiles[TOPK_TILE_CAP];
  __shared__ int s_nt;
  if (threadIdx.x == 0) { s_n = 0; s_nt = 0; }
  __syncthreads();
  for (int t = threadIdx.x; t < n_tiles; t += 256)
    if (f2key(tm[t]) >= thr) {
      const int q = atomicAdd(&s_nt, 1);
      if (q < TOPK_TILE_CAP) tiles[q] = t;
    }
  __syncthreads();
  const int nt = s_nt;
  for (int q = 0; q < (nt <= TOPK_TILE_CAP ? nt : n_tiles); ++q) {
    const int t = nt <= TOPK_TILE_CAP ? tiles[q] : q;
    if (nt > TOPK_TILE_CAP && f2key(tm[t]) < thr) continue;
    const int c = t * tile_w + threadIdx.x;
    if ((int)threadIdx.x < tile_w && c < V) {
      const float v = z[c] * inv_temp;
      if (f2key(v) >= thr) {
        const int slot = atomicAdd(&s_n, 1);
        if (slot < TOPK_CAP) cand[slot] = ckey(v, c);
      }
    }
  }
  __syncthreads();
  const int n = s_n;
  uint64_t kth;
  if (n <= TOPK_CAP) {
    kth = radix_kth(n, kk, [&](int i) { return cand[i]; }, hist, &sh_prefix, &sh_k);
  } else {
    kth = radix_kth(V, kk, [&](int i) { return ckey(z[i] * inv_temp, i); }, hist, &sh_prefix, &sh_k);
  }
  // gather the k selected keys
  if (threadIdx.x == 0) s_n = 0;
  __syncthreads();
  int P = 1;
  while (P < kk) P <<= 1;
  if (n <= TOPK_CAP) {
    for (int i = threadIdx.x; i < n; i += 256)
      if (cand[i] >= kth) sel[atomicAdd(&s_n, 1)] = cand[i];
  } else {
    for (int i = threadIdx.x; i < V; i += 256) {
      const uint64_t key = ckey(z[i] * inv_temp, i);
      if (key >= kth) sel[atomicAdd(&s_n, 1)] = key;
    }
  }
  __syncthreads();
  for (int i = kk + threadIdx.x; i < P; i += 256) sel[i] = 0;
  __syncthreads();
  // bitonic sort, descending
  for (int size = 2; size <= P; size <<= 1) {
    for (int stride = size >> 1; stride > 0; stride >>= 1) {
      for (int i = threadIdx.x; i < P; i += 256) {
        const int jx = i ^ stride;
        if (jx > i) {
          const bool desc = (i & size) == 0;
          const uint64_t a = sel[i], b = sel[jx];
          if (desc ? (a < b) : (a > b)) {
            sel[i] = b;
            sel[jx] = a;
          }
        }
      }
      __syncthreads();
    }
  }
  const float M = row_max[m], L = row_lse[m];
  for (int i = threadIdx.x; i < kk; i += 256) {
    const int id = (int)(0xFFFFFFFFu - (uint32_t)(sel[i] & 0xFFFFFFFFull));
    ids_out[(int64_t)m * k + i] = id;
    probs_out[(int64_t)m * k + i] = expf(z[id] * inv_temp - M - L);
  }
}

// Small k (<= 64).  The k-th largest tile maximum (a radix select over the
// maxima's order keys) bounds the k-th largest logit from below, so the top k
// lie among the logits at or above it in the tiles whose maximum reaches it;
// those are gathered into LDS (at least k of them, usually a few more) and each
// is placed by its rank among them (the keys are distinct: they carry the id).
// More than TOPK_RANK_CAP gathered (heavy ties) falls back to k rounds of
// block maxima over the same tiles.  Same keys, order and probabilities as
// topk_kernel.
__device__ __forceinline__ uint64_t block_max_u64(uint64_t v, uint64_t* sh) {
  for (int o = 32; o > 0; o >>= 1) {
    const uint32_t lo = __shfl_xor((uint32_t)v, o, 64), hi = __shfl_xor((uint32_t)(v >> 32), o, 64);
    const uint64_t y = ((uint64_t)hi << 32) | lo;
    v = y > v ? y : v;
  }
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  __syncthreads();
  if (lane == 0) sh[w] = v;
  __syncthreads();
  uint64_t m = sh[0];
  for (int i = 1; i < (int)(blockDim.x >> 6); ++i) m = sh[i] > m ? sh[i] : m;
  return m;
}

// k-th largest of n 32-bit keys (1 <= k <= n): four 8-bit digit passes, each a
// shared histogram of the keys that match the digits found so far, searched by
// one wave from the top bucket down (four buckets per lane, integer scan).
template <class Get>
__device__ uint32_t radix_kth32(int n, int k, Get get, uint32_t* hist, uint32_t* sh_prefix, int* sh_k) {
  uint32_t prefix = 0;
  int krem = k;
  const int lane = threadIdx.x & 63;
  for (int pass = 3; pass >= 0; --pass) {
    const int shift = pass * 8;
    for (int b = threadIdx.x; b < 256; b += blockDim.x) hist[b] = 0;
    __syncthreads();
    const uint32_t hmask = pass == 3 ? 0u : (~0u << (shift + 8));
    for (int i = threadIdx.x; i < n; i += blockDim.x) {
      const uint32_t key = get(i);
      if ((key & hmask) == (prefix & hmask)) atomicAdd(&hist[(key >> shift) & 255], 1u);
    }
    __syncthreads();
    if (threadIdx.x < 64) {
      const int b0 = 255 - 4 * lane;   // buckets b0, b0-1, b0-2, b0-3 (descending)
      int c[4], ls = 0;
#pragma unroll
      for (int q = 0; q < 4; ++q) { c[q] = (int)hist[b0 - q]; ls += c[q]; }
      int incl = ls;
      for (int o = 1; o < 64; o <<= 1) {
        const int y = __shfl_up(incl, o, 64);
        if (lane >= o) incl += y;
      }
      const int excl = incl - ls;
      if (excl < krem && krem <= incl) {
        int cum = excl, q = 0;
        for (; q < 3; ++q) {
          if (cum + c[q] >= krem) break;
          cum += c[q];
        }
        *sh_prefix = prefix | ((uint32_t)(b0 - q) << shift);
        *sh_k = krem - cum;
      }
    }
    __syncthreads();
    prefix = *sh_prefix;
    krem = *sh_k;
    __syncthreads();
  }
  return prefix;
}

constexpr int TOPK_SMALL_K = 64, TOPK_SMALL_TILES = 2048, TOPK_RANK_CAP = 1024;

__global__ __launch_bounds__(256) void topk_small_kernel(int V, int k, const float* logits, const float* tmax,
                                                          int n_tiles, int tile_w, float inv_temp,
                                                          const float* row_max, const float* row_lse,
                                                          int32_t* ids_out, float* probs_out) {
  __shared__ uint64_t red[4];
  __shared__ uint32_t hist[256];
  __shared__ uint32_t s_pref;
  __shared__ int s_kr;
  __shared__ int tiles[TOPK_SMALL_TILES];
  __shared__ int s_nt, s_nc;
  __shared__ uint64_t cand[TOPK_RANK_CAP];
  __shared__ uint64_t sel[TOPK_SMALL_K];
  const int m = blockIdx.x, tid = threadIdx.x;
  const float* z = logits + (int64_t)m * V;
  const float* tm = tmax + (int64_t)m * n_tiles;
  const int kk = min(k, V);
  // the kk-th largest tile maximum (no bound when there are no more tiles than kk)
  uint32_t thr = 0;
  if (kk < n_tiles) thr = radix_kth32(n_tiles, kk, [&](int i) { return f2key(tm[i]); }, hist, &s_pref, &s_kr);
  if (tid == 0) { s_nt = 0; s_nc = 0; }
  __syncthreads();
  for (int t = tid; t < n_tiles; t += 256)
    if (f2key(tm[t]) >= thr) tiles[atomicAdd(&s_nt, 1)] = t;
  __syncthreads();
  const int ne = s_nt * tile_w;
  for (int e = tid; e < ne; e += 256) {
    const int c = tiles[e / tile_w] * tile_w + e % tile_w;
    if (c < V) {
      const float v = z[c] * inv_temp;
      if (f2key(v) >= thr) {
        const int q = atomicAdd(&s_nc, 1);
        if (q < TOPK_RANK_CAP) cand[q] = ckey(v, c);
      }
    }
  }
  __syncthreads();
  const int nc = s_nc;
  if (nc <= TOPK_RANK_CAP) {
    for (int i = tid; i < nc; i += 256) {
      const uint64_t key = cand[i];
      int rank = 0;
      for (int j = 0; j < nc; ++j) rank += cand[j] > key ? 1 : 0;
      if (rank < kk) sel[rank] = key;
    }
  } else {
    uint64_t prev = ~0ull;
    for (int i = 0; i < kk; ++i) {
      uint64_t best = 0;
      for (int e = tid; e < ne; e += 256) {
        const int c = tiles[e / tile_w] * tile_w + e % tile_w;
        if (c < V) {
          const uint64_t key = ckey(z[c] * inv_temp, c);
          if (key < prev && key > best) best = key;
        }
      }
      prev = block_max_u64(best, red);
      if (tid == 0) sel[i] = prev;
    }
  }
  __syncthreads();
  const float M = row_max[m], L = row_lse[m];
  for (int i = tid; i < kk; i += 256) {
    const int id = (int)(0xFFFFFFFFu - (uint32_t)(sel[i] & 0xFFFFFFFFull));
    ids_out[(int64_t)m * k + i] = id;
    probs_out[(int64_t)m * k + i] = expf(z[id] * inv_temp - M - L);
  }
}

// ---------------------------------------------------------------------------
// Best-first top-B prefix tree [P5 §2.3] per request (one wave): the frontier
// (at most 2B + 1 rank tuples) sits in LDS; each pop is a wave-parallel
// arg-best under the order (larger fp32 prefix probability, then shallower,
// then lexicographically smaller rank tuple).  Node 0 is the root (anchor).
// Mask [P5 §3.3]: node i sees itself, its ancestors and the root.
// ---------------------------------------------------------------------------
static constexpr int TREE_MAXB = 256;
static constexpr int TREE_MAXF = 2 * TREE_MAXB + 2;

__global__ __launch_bounds__(64) void tree_kernel(int L, int Kc, int stride, int B, const float* probs, const int32_t* ids,
                                                   const int32_t* anchors, int32_t* tokens, int32_t* parents,
                                                   int32_t* depth_out, uint64_t* mask) {
  __shared__ float f_p[TREE_MAXF];
  __shared__ int f_parent[TREE_MAXF], f_rank[TREE_MAXF], f_depth[TREE_MAXF];
  __shared__ int f_alive[TREE_MAXF];
  __shared__ int n_parent[TREE_MAXB + 1], n_rank[TREE_MAXB + 1], n_depth[TREE_MAXB + 1];
  __shared__ float n_p[TREE_MAXB + 1];
  __shared__ int s_nf;
  const int r = blockIdx.x, lane = threadIdx.x;
  const float* pr = probs + (int64_t)r * L * stride;   // position i's candidates at pr[i * stride ..]
  const int32_t* id = ids + (int64_t)r * L * stride;
  const int words = (B + 1 + 63) / 64;

  // rank-tuple comparison for exact ties: walk both parent chains (equal depth)
  auto lex_less = [&](int pa, int ra, int pb, int rb) -> bool {
    // tuples are (chain(pa), ra) and (chain(pb), rb); compare from the root down
    int ca[64], cb[64];
    int da = 0, db = 0;
    for (int x = pa; x > 0; x = n_parent[x]) ca[da++] = n_rank[x];
    for (int x = pb; x > 0; x = n_parent[x]) cb[db++] = n_rank[x];
    for (int i = 1; i <= da; ++i) {
      const int a = ca[da - i], b = cb[db - i];
      if (a != b) return a < b;
    }
    return ra < rb;
  };
  auto better = [&](int a, int b) -> bool {   // frontier entries
    if (f_p[a] != f_p[b]) return f_p[a] > f_p[b];
    if (f_depth[a] != f_depth[b]) return f_depth[a] < f_depth[b];
    return lex_less(f_parent[a], f_rank[a], f_parent[b], f_rank[b]);
  };

  if (lane == 0) {
    n_parent[0] = -1; n_rank[0] = 0; n_depth[0] = 0; n_p[0] = 1.f;
    f_p[0] = pr[0]; f_parent[0] = 0; f_rank[0] = 1; f_depth[0] = 1; f_alive[0] = 1;
    s_nf = 1;
  }
  __syncthreads();
  int nodes = 0;
  for (int step = 0; step < B; ++step) {
    const int nf = s_nf;
    int best = -1;
    for (int i = lane; i < nf; i += 64)
      if (f_alive[i] && (best < 0 || better(i, best))) best = i;
    for (int o = 32; o > 0; o >>= 1) {
      const int other = __shfl_xor(best, o, 64);
      if (other >= 0 && (best < 0 || better(other, best))) best = other;
    }
    if (best < 0) break;
    if (lane == 0) {
      const int idx = nodes + 1;
      const int d = f_depth[best], par = f_parent[best], rk = f_rank[best];
      f_alive[best] = 0;
      n_parent[idx] = par; n_rank[idx] = rk; n_depth[idx] = d; n_p[idx] = f_p[best];
      int nf2 = nf;
      if (rk < Kc) {   // sibling
        const float pp = d == 1 ? pr[rk] : n_p[par] * pr[(d - 1) * stride + rk];
        f_p[nf2] = pp; f_parent[nf2] = par; f_rank[nf2] = rk + 1; f_depth[nf2] = d; f_alive[nf2] = 1; ++nf2;
      }
      if (d < L) {     // child
        f_p[nf2] = f_p[best] * pr[d * stride]; f_parent[nf2] = idx; f_rank[nf2] = 1; f_depth[nf2] = d + 1;
        f_alive[nf2] = 1; ++nf2;
      }
      s_nf = nf2;
    }
    ++nodes;
    __syncthreads();
  }
  // outputs
  const int64_t base = (int64_t)r * (B + 1);
  for (int i = lane; i <= B; i += 64) {
    if (i == 0) {
      tokens[base] = anchors ? anchors[r] : -1;
      parents[base] = -1;
      depth_out[base] = 0;
    } else if (i <= nodes) {
      const int d = n_depth[i];
      tokens[base + i] = id[(d - 1) * stride + n_rank[i] - 1];
      parents[base + i] = n_parent[i];
      depth_out[base + i] = d;
    } else {
      tokens[base + i] = -1;
      parents[base + i] = -1;
      depth_out[base + i] = -1;
    }
  }
  if (mask) {
    // row i = row(parent) | bit(i); rows built in node order by lane 0 (parents precede children)
    if (lane == 0) {
      uint64_t* mrow0 = mask + base * words;
      for (int w = 0; w < words; ++w) mrow0[w] = 0;
      mrow0[0] = 1ull;
      for (int i = 1; i <= B; ++i) {
        uint64_t* mr = mask + (base + i) * words;
        if (i <= nodes) {
          const uint64_t* mp = mask + (base + n_parent[i]) * words;
          for (int w = 0; w < words; ++w) mr[w] = mp[w];
          mr[i / 64] |= 1ull << (i % 64);
        } else {
          for (int w = 0; w < words; ++w) mr[w] = 0;
        }
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Verification.
// Greedy [P2 §2.3]: a = sum_i prod_{k<=i} [d_k == argmax t_{k-1}]; emit d_1..d_a, argmax t_a.
// Rejection [P2 §2.3, §4.2]: accept d_i iff u_i * q_i(d_i) < p_{i-1}(d_i); at the
// first rejection draw from max(0, p - q) (or p when that mass is below
// RESIDUAL_EPS); after K acceptances draw the bonus from p_K.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void argmax_rows_kernel(int V, const float* x, int32_t* out) {
  __shared__ float sv[4];
  __shared__ int si[4];
  const int64_t m = blockIdx.x;
  const float* row = x + m * V;
  float best = -INFINITY;
  int arg = 0x7fffffff;
  if ((V & 3) == 0) {   // 16-byte loads, 8 in flight per thread; ids increase along each thread's walk
    const float4* r4 = (const float4*)row;
    const int V4 = V >> 2;
    int c = threadIdx.x;
    for (; c + 1792 < V4; c += 2048) {
      float4 q[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) q[u] = r4[c + 256 * u];
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int b = 4 * (c + 256 * u);
        if (q[u].x > best) { best = q[u].x; arg = b; }
        if (q[u].y > best) { best = q[u].y; arg = b + 1; }
        if (q[u].z > best) { best = q[u].z; arg = b + 2; }
        if (q[u].w > best) { best = q[u].w; arg = b + 3; }
      }
    }
    for (; c < V4; c += 256) {
      const float4 q = r4[c];
      const int b = 4 * c;
      if (q.x > best) { best = q.x; arg = b; }
      if (q.y > best) { best = q.y; arg = b + 1; }
      if (q.z > best) { best = q.z; arg = b + 2; }
      if (q.w > best) { best = q.w; arg = b + 3; }
    }
  } else {
    for (int c = threadIdx.x; c < V; c += 256) {
      const float v = row[c];
      if (v > best) { best = v; arg = c; }
    }
  }
  const float M = wave_max(best);
  int cand = best == M ? arg : 0x7fffffff;
  for (int o = 32; o > 0; o >>= 1) cand = min(cand, __shfl_xor(cand, o, 64));
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  if (lane == 0) { sv[w] = M; si[w] = cand; }
  __syncthreads();
  if (threadIdx.x == 0) {
    float b = sv[0];
    int a = si[0];
    for (int i = 1; i < 4; ++i)
      if (sv[i] > b || (sv[i] == b && si[i] < a)) { b = sv[i]; a = si[i]; }
    out[m] = a;
  }
}

__global__ void greedy_finish_kernel(int n_req, int K, const int32_t* draft_ids, const int32_t* post,
                                     int32_t* out_tokens, int32_t* out_len, int32_t* accept_len,
                                     int32_t* next_anchor) {
  const int r = blockIdx.x * blockDim.x + threadIdx.x;
  if (r >= n_req) return;
  const int32_t* d = draft_ids + (int64_t)r * K;
  const int32_t* p = post + (int64_t)r * (K + 1);
  int a = 0;
  while (a < K && d[a] == p[a]) ++a;
  int32_t* o = out_tokens + (int64_t)r * (K + 1);
  for (int i = 0; i < a; ++i) o[i] = d[i];
  o[a] = p[a];
  for (int i = a + 1; i <= K; ++i) o[i] = -1;
  out_len[r] = a + 1;
  accept_len[r] = a;
  if (next_anchor) next_anchor[r] = p[a];
}

// ---------------------------------------------------------------------------
// Row statistics of fp32 logits rows for verification and truncation, one
// 256-thread block per row in one coalesced pass: M = max z/T and S = sum
// exp(z/T - M) (online, per lane, then combined), and optionally the maximum of
// z/T over each 128-id tile (the pruning bound of the top-k kernels).  Lane l
// of a wave reads ids 4l..4l+3 of a 256-id unit (one 16-byte load when `vec`),
// so lanes 0-31 cover one tile and lanes 32-63 the next.  Row m's results go to
// o = (m / per) * group + off + m % per: out_max[o * os] and out_b[o * os]
// (S, or log S with want_log).
// ---------------------------------------------------------------------------
constexpr int RS_TILE = 128;

// e^x as 2^(x log2 e) on the hardware's base-2 exponential (v_exp_f32): a few
// ulp for the x <= 0 the sums here take (larger relative error only where the
// result is far below the terms that dominate a sum); 0 for x = -inf.
__device__ __forceinline__ float exp_sum_term(float x) { return __builtin_amdgcn_exp2f(x * 1.44269504088896341f); }

__device__ __forceinline__ void load4_row(const float* row, int c0, int V, bool vec, float x[4]) {
  if (vec && c0 + 3 < V) {
    const float4 v = *(const float4*)(row + c0);
    x[0] = v.x; x[1] = v.y; x[2] = v.z; x[3] = v.w;
  } else {
#pragma unroll
    for (int q = 0; q < 4; ++q) x[q] = c0 + q < V ? row[c0 + q] : -INFINITY;
  }
}

template <bool TILES, bool VEC>
__global__ __launch_bounds__(256) void row_stats_kernel(int V, const float* x, float inv_temp, float* tmax, int n_tiles,
                                                        float* out_max, float* out_b, int os, int per, int group,
                                                        int off, int want_log) {
  __shared__ float sm[4], ss[4];
  const int64_t m = blockIdx.x;
  const float* row = x + m * V;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int units = (V + 255) / 256;
  float lm = -INFINITY, ls = 0.f;
  // four units per wave and pass: their loads are issued together (bytes in flight)
  for (int u0 = w; u0 < units; u0 += 16) {
    float v[4][4];
    if (VEC && (u0 + 13) * 256 <= V) {   // the pass lies inside the row: plain 16-byte loads
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const float4 q = *(const float4*)(row + (u0 + 4 * j) * 256 + 4 * lane);
        v[j][0] = q.x; v[j][1] = q.y; v[j][2] = q.z; v[j][3] = q.w;
      }
    } else {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int c0 = (u0 + 4 * j) * 256 + 4 * lane;
#pragma unroll
        for (int q = 0; q < 4; ++q) v[j][q] = c0 + q < V ? row[c0 + q] : -INFINITY;
      }
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int u = u0 + 4 * j;
      float mx = -INFINITY;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        v[j][q] *= inv_temp;   // -inf (past the row) stays -inf
        mx = fmaxf(mx, v[j][q]);
      }
      if (TILES) {
        float tm = mx;
#pragma unroll
        for (int o = 16; o > 0; o >>= 1) tm = fmaxf(tm, __shfl_xor(tm, o, 64));
        const int t = 2 * u + (lane >> 5);
        if ((lane & 31) == 0 && t < n_tiles) tmax[m * n_tiles + t] = tm;
      }
      if (mx > -INFINITY) {
        const float nm = fmaxf(lm, mx);
        float acc = ls * exp_sum_term(lm - nm);     // lm = -inf with ls = 0 gives 0
#pragma unroll
        for (int q = 0; q < 4; ++q) acc += exp_sum_term(v[j][q] - nm);
        lm = nm;
        ls = acc;
      }
    }
  }
  const float wm = wave_max(lm);
  const float wsum = wave_sum(wm > -INFINITY && lm > -INFINITY ? ls * exp_sum_term(lm - wm) : 0.f);
  if (lane == 0) { sm[w] = wm; ss[w] = wsum; }
  __syncthreads();
  if (threadIdx.x == 0) {
    const float M = fmaxf(fmaxf(sm[0], sm[1]), fmaxf(sm[2], sm[3]));
    float S = 0.f;
    for (int i = 0; i < 4; ++i) S += sm[i] > -INFINITY ? ss[i] * expf(sm[i] - M) : 0.f;
    const int64_t o = (m / per) * group + off + m % per;
    out_max[o * os] = M;
    out_b[o * os] = want_log ? logf(S) : S;
  }
}

// ---------------------------------------------------------------------------
// Inverse-CDF draw over ids [0, V) in ascending order by one 256-thread block,
// for weights given four ids at a time: wf(c0, e) fills e[0..3] with the
// weights of ids c0..c0+3 (0 beyond V).  Sums of 256-id chunks (coalesced, one
// wave per chunk) go to LDS; one wave scans them in lane-contiguous ranges to
// the chunk where the cumulative mass first exceeds u * total, then scans that
// chunk's ids.  Neighbouring ranges share their end points, so exactly one
// range holds the target; should rounding leave it past the last weight, the
// last id with weight in the chosen range is taken.
// ---------------------------------------------------------------------------
constexpr int DRAW_CHUNK = 256;

template <class WF>
__device__ __forceinline__ void chunk_sums(int V, WF wf, float* csum) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int nch = (V + DRAW_CHUNK - 1) / DRAW_CHUNK;
  // four chunks per wave and pass, their loads issued together
  for (int c0 = w; c0 < nch; c0 += 16) {
    float e[4][4];
#pragma unroll
    for (int j = 0; j < 4; ++j) wf((c0 + 4 * j) * DRAW_CHUNK + 4 * lane, e[j]);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const float t = wave_sum((e[j][0] + e[j][1]) + (e[j][2] + e[j][3]));
      if (lane == 0 && c0 + 4 * j < nch) csum[c0 + 4 * j] = t;
    }
  }
}

// total of the chunk sums (wave 0 computes, every thread gets it)
__device__ __forceinline__ float chunk_total(int V, const float* csum, float* sh) {
  const int nch = (V + DRAW_CHUNK - 1) / DRAW_CHUNK;
  if (threadIdx.x < 64) {
    float t = 0.f;
    for (int c = threadIdx.x; c < nch; c += 64) t += csum[c];
    t = wave_sum(t);
    if (threadIdx.x == 0) sh[0] = t;
  }
  __syncthreads();
  const float t = sh[0];
  __syncthreads();
  return t;
}

__device__ __forceinline__ float wave_incl_scan_f(float v, int lane) {
  for (int o = 1; o < 64; o <<= 1) {
    const float y = __shfl_up(v, o, 64);
    if (lane >= o) v += y;
  }
  return v;
}

template <class WF>
__device__ int chunk_draw(int V, float u, WF wf, const float* csum, float* sh, int* si) {
  const int nch = (V + DRAW_CHUNK - 1) / DRAW_CHUNK;
  const int lane = threadIdx.x & 63;
  if (threadIdx.x < 64) {
    // level 1: the chunk
    const int per = (nch + 63) / 64;
    const int c0 = lane * per, c1 = min(nch, c0 + per);
    float ls = 0.f;
    for (int c = c0; c < c1; ++c) ls += csum[c];
    const float incl = wave_incl_scan_f(ls, lane);
    float excl = __shfl_up(incl, 1, 64);
    if (lane == 0) excl = 0.f;
    const float target = u * __shfl(incl, 63, 64);
    const unsigned long long hit = __ballot(ls > 0.f && excl <= target && target < incl);
    const unsigned long long nz = __ballot(ls > 0.f);
    const int owner = hit ? __ffsll((long long)hit) - 1 : (nz ? 63 - __clzll((long long)nz) : -1);
    if (lane == owner) {
      float acc = excl, before = excl, lastb = excl;
      int ch = -1, last = -1;
      for (int c = c0; c < c1; ++c) {
        const float wc = csum[c];
        if (wc > 0.f) {
          last = c;
          lastb = acc;
          if (hit && ch < 0 && target < acc + wc) { ch = c; before = acc; }
        }
        acc += wc;
      }
      if (ch < 0) { ch = last; before = lastb; }
      si[0] = ch;
      sh[0] = before;
      sh[1] = target;
    }
    if (owner < 0 && lane == 0) si[0] = -1;
  }
  __syncthreads();
  const int ch = si[0];
  const float before = sh[0], target = sh[1];
  __syncthreads();
  if (ch < 0) return 0;   // no weight anywhere
  if (threadIdx.x < 64) {
    // level 2: the id inside the chunk (lane l holds ids 4l..4l+3, ascending with l)
    const int c0 = ch * DRAW_CHUNK + 4 * lane;
    float e[4];
    wf(c0, e);
    const float ls = ((e[0] + e[1]) + e[2]) + e[3];
    const float incl = before + wave_incl_scan_f(ls, lane);
    float excl = __shfl_up(incl, 1, 64);
    if (lane == 0) excl = before;
    const unsigned long long hit = __ballot(ls > 0.f && excl <= target && target < incl);
    const unsigned long long nz = __ballot(ls > 0.f);
    const int owner = hit ? __ffsll((long long)hit) - 1 : (nz ? 63 - __clzll((long long)nz) : -1);
    if (lane == owner) {
      float acc = excl;
      int pick = -1, last = -1;
      for (int q = 0; q < 4; ++q) {
        if (e[q] > 0.f) {
          last = c0 + q;
          if (hit && pick < 0 && target < acc + e[q]) pick = c0 + q;
        }
        acc += e[q];
      }
      si[1] = pick >= 0 ? pick : last;
    }
    if (owner < 0 && lane == 0) si[1] = ch * DRAW_CHUNK;
  }
  __syncthreads();
  const int pick = si[1];
  __syncthreads();
  return pick;
}

// ---------------------------------------------------------------------------
// Top-p over whole rows [P2 §3.3, with no top-k cut]: the set of ids in
// probability-descending order (ties: ascending id) up to the one whose
// cumulative probability reaches top_p.  Probabilities are compared through an
// order-preserving uint32 key of s = z / T; the threshold key is found by a
// radix select from the most significant byte, each pass a histogram of the
// probability mass (exp(s - row max)) of the ids that still match the prefix.
// Ids at the threshold key have equal probability; the set takes the fewest of
// them, lowest ids first, that reach top_p.
// ---------------------------------------------------------------------------
__device__ __forceinline__ uint32_t order_key(float s) {
  const uint32_t u = __float_as_uint(s);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
__device__ __forceinline__ float key_value(uint32_t k) {
  return __uint_as_float((k & 0x80000000u) ? (k & 0x7fffffffu) : ~k);
}
__device__ __forceinline__ bool in_nucleus(float s, int id, const Nucleus& n) {
  const uint32_t k = order_key(s);
  return k > n.key || (k == n.key && id <= n.cut);
}

// The probability law of one row as the rejection kernels use it: exp(s - m) * inv,
// zero outside the row's top-p set when one is given.
struct RowLaw {
  float m, inv;
  const Nucleus* n;
  __device__ __forceinline__ float operator()(float s, int id) const {
    if (n && !in_nucleus(s, id, *n)) return 0.f;
    return exp_sum_term(s - m) * inv;
  }
};
__device__ __forceinline__ RowLaw row_law(const float* st, const Nucleus* nuc, int j) {
  RowLaw L;
  L.m = st[2 * j];
  L.n = nuc ? nuc + j : nullptr;
  L.inv = 1.0f / (nuc ? nuc[j].mass : st[2 * j + 1]);
  return L;
}

// one 512-thread work-group per row; each wave fills its own histogram with LDS
// atomics and the waves' histograms are summed in a fixed order
constexpr int NUC_THREADS = 512, NUC_WAVES = NUC_THREADS / 64;
__global__ __launch_bounds__(NUC_THREADS) void nucleus_kernel(int V, const float* logits, int per, int nrow, int off,
                                                               const float* st_max, int st_stride, float inv_temp,
                                                               float top_p, int vec, Nucleus* out) {
  __shared__ float hm[NUC_WAVES][256];
  __shared__ int hc[NUC_WAVES][256];
  __shared__ uint32_t s_prefix, s_mask;
  __shared__ float s_above, s_target;
  __shared__ int s_cnt, s_cut;
  __shared__ int scan[NUC_WAVES];
  const int i = blockIdx.x;
  const int j = (i / per) * nrow + off + i % per;
  const float* z = logits + (int64_t)i * V;
  const float mx = st_max[(int64_t)j * st_stride];
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const bool vv = vec != 0;
  if (tid == 0) {
    s_prefix = 0;
    s_mask = 0;
    s_above = 0.f;
  }
  for (int pass = 0; pass < 4; ++pass) {
    const int shift = 24 - 8 * pass;
    for (int b = lane; b < 256; b += 64) {
      hm[w][b] = 0.f;
      hc[w][b] = 0;
    }
    __syncthreads();
    const uint32_t prefix = s_prefix, mask = s_mask;
    for (int c = tid * 4; c < V; c += 4 * NUC_THREADS) {
      float x[4];
      load4_row(z, c, V, vv, x);
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const float sv = x[q] * inv_temp;
        const uint32_t k = order_key(sv);
        if (c + q < V && (k & mask) == prefix) {
          const int b = (int)((k >> shift) & 255u);
          atomicAdd(&hm[w][b], exp_sum_term(sv - mx));
          atomicAdd(&hc[w][b], 1);
        }
      }
    }
    __syncthreads();
    if (tid < 256) {   // 256 buckets, one per thread; waves summed in a fixed order
      const int b = tid;
      float sm = hm[0][b];
      int sc = hc[0][b];
      for (int q = 1; q < NUC_WAVES; ++q) {
        sm += hm[q][b];
        sc += hc[q][b];
      }
      hm[0][b] = sm;
      hc[0][b] = sc;
    }
    __syncthreads();
    if (tid == 0) {
      if (pass == 0) {   // the row's total, in the same terms as the members' mass
        float t = 0.f;
        for (int b = 255; b >= 0; --b) t += hm[0][b];
        s_target = top_p * t;
      }
      const float above = s_above, target = s_target;
      float cum = 0.f, cum_low = 0.f;
      int sel = -1, low = -1;
      for (int b = 255; b >= 0; --b) {
        if (hc[0][b] == 0) continue;
        if (above + cum + hm[0][b] >= target) {
          sel = b;
          break;
        }
        low = b;
        cum_low = cum;
        cum += hm[0][b];
      }
      if (sel < 0) {   // rounding left the target past the total: every remaining id
        sel = low < 0 ? 0 : low;
        cum = cum_low;
      }
      s_above = above + cum;
      s_prefix = prefix | ((uint32_t)sel << shift);
      s_mask = mask | (255u << shift);
      s_cnt = hc[0][sel];
    }
    __syncthreads();
  }
  const uint32_t key = s_prefix;
  const float above = s_above;
  const int cnt = s_cnt;
  const float wk = exp_sum_term(key_value(key) - mx);
  int kk = cnt;
  if (wk > 0.f) {
    const float need = (s_target - above) / wk;
    kk = need <= 1.f ? 1 : min(cnt, (int)ceilf(need));
  }
  if (kk >= cnt) {
    if (tid == 0) s_cut = 0x7fffffff;   // all ids at the threshold
  } else {
    // the kk-th lowest id at the threshold key: ascending 1024-id chunks
    if (tid == 0) s_cut = -1;
    int before = 0;
    for (int c0 = 0; c0 < V; c0 += 4 * NUC_THREADS) {
      const int c = c0 + tid * 4;
      float x[4];
      load4_row(z, c, V, vv, x);
      int n = 0;
#pragma unroll
      for (int q = 0; q < 4; ++q) n += (c + q < V && order_key(x[q] * inv_temp) == key) ? 1 : 0;
      // inclusive scan of n over the 256 threads
      int incl = n;
      for (int o = 1; o < 64; o <<= 1) {
        const int y = __shfl_up(incl, o, 64);
        if (lane >= o) incl += y;
      }
      __syncthreads();
      if (lane == 63) scan[w] = incl;
      __syncthreads();
      int add = before, chunk_total = 0;
      for (int q = 0; q < NUC_WAVES; ++q) {
        if (q < w) add += scan[q];
        chunk_total += scan[q];
      }
      const int ex = add + incl - n;   // ids at the key before this thread's four
      if (n > 0 && ex < kk && kk <= ex + n) {
        int seen = ex;
        for (int q = 0; q < 4; ++q)
          if (c + q < V && order_key(x[q] * inv_temp) == key && ++seen == kk) s_cut = c + q;
      }
      before += chunk_total;
      __syncthreads();
      if (before >= kk) break;
    }
  }
  __syncthreads();
  if (tid == 0) {
    Nucleus nu;
    nu.key = key;
    nu.cut = s_cut;
    nu.mass = above + (float)kk * wk;
    nu.pad = 0.f;
    out[j] = nu;
  }
}

// draft draw from the top-p set of each row: one 256-thread work-group per row,
// inverse CDF in ascending id order (Philox(seed; j+1, slot, step, 0))
__global__ __launch_bounds__(256) void nucleus_sample_kernel(int K, int V, const int32_t* slots, uint64_t seed,
                                                              uint64_t step, float inv_temp, const float* logits,
                                                              const float* row_max, const Nucleus* nuc, int vec,
                                                              int32_t* draft_ids) {
  extern __shared__ float csum[];
  __shared__ float sh[4];
  __shared__ int si[2];
  const int m = blockIdx.x;
  const int r = m / K, j = m % K;
  const float* z = logits + (int64_t)m * V;
  const float mx = row_max[m];
  const Nucleus nu = nuc[m];
  const bool vv = vec != 0;
  auto wf = [&](int c0, float* e) {
    float x[4];
    load4_row(z, c0, V, vv, x);
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const float sv = x[q] * inv_temp;
      e[q] = c0 + q < V && in_nucleus(sv, c0 + q, nu) ? exp_sum_term(sv - mx) : 0.f;
    }
  };
  chunk_sums(V, wf, csum);
  __syncthreads();
  const float u = philox_uniform(seed, (uint32_t)slots[r], step, (uint32_t)(j + 1), PURPOSE_DRAFT);
  const int pick = chunk_draw(V, u, wf, csum, sh, si);
  if (threadIdx.x == 0) draft_ids[m] = pick;
}

static constexpr float RESIDUAL_EPS = 9.5367431640625e-07f;  // 2^-20

// Rejection verification at temperature T > 0 [P2 §2.3, §4.2; P1 "验证"], in
// three steps so that the residual's pass over the vocabulary spreads over the
// GPU instead of one work-group per request:
//  1. verify_accept_kernel, one wave per request: lane i tests draft position
//     i+1 (accept iff u * q(d_i) < p(d_i), Philox(seed; i+1, slot, step, 1));
//     the first failure (or K) is the number accepted, a.
//  2. resid_chunks_kernel, a grid of work-groups per request: sums of p and of
//     the residual max(0, p - q) over 256-id chunks of row a (p alone after K
//     acceptances).
//  3. verify_draw_kernel, one work-group per request: the inverse-CDF draw
//     (Philox(seed; a+1, slot, step, 2)) from the residual, from p when its mass
//     is below RESIDUAL_EPS, or from the bonus row p_K.
// Two forms of q: dense (the drafter's logits: q = softmax(z / T)) and subset
// [P2 §3.1.3]: the selector's C candidates with a distribution over them,
// q_full(v) = the summed probability of the candidates with id v (0 outside);
// there the residual is p away from the candidates and p - min(p, q) at them,
// so the chunk sums of p are corrected at the few candidates, in id order.
// Statistics rows per request: K+1 target rows, then (dense) K draft rows.
// ---------------------------------------------------------------------------
constexpr int SUBSET_MAX_C = 64;

__global__ __launch_bounds__(64) void verify_accept_kernel(int K, int V, int subset, const int32_t* slots,
                                                            const int32_t* draft_ids, const float* draft_logits,
                                                            const float* target, float inv_temp,
                                                            const float* stats, int C, const int32_t* cand_ids,
                                                            const float* cand_probs, uint64_t seed, uint64_t step,
                                                            int32_t* acc_out, int32_t* err, const Nucleus* nuc) {
  const int r = blockIdx.x, lane = threadIdx.x;
  const int nrow = subset ? K + 1 : 2 * K + 1;
  const float* ts = stats + (int64_t)r * nrow * 2;
  bool fail = false, bad = false;
  if (lane < K) {
    const int tok = draft_ids[(int64_t)r * K + lane];
    bad = tok < 0 || tok >= V;
    if (bad) {
      fail = true;
    } else {
      const Nucleus* nr = nuc ? nuc + (int64_t)r * nrow : nullptr;
      const float p = nr ? row_law(ts, nr, lane)(target[((int64_t)r * (K + 1) + lane) * V + tok] * inv_temp, tok)
                         : expf(target[((int64_t)r * (K + 1) + lane) * V + tok] * inv_temp - ts[2 * lane]) /
                               ts[2 * lane + 1];
      float q = 0.f;
      if (subset) {
        const int64_t b = ((int64_t)r * K + lane) * C;
        for (int j = 0; j < C; ++j)
          if (cand_ids[b + j] == tok) q += cand_probs[b + j];
      } else {
        const int sr = K + 1 + lane;
        const float sq = draft_logits[((int64_t)r * K + lane) * V + tok] * inv_temp;
        q = nr ? row_law(ts, nr, sr)(sq, tok) : expf(sq - ts[2 * sr]) / ts[2 * sr + 1];
      }
      const float u = philox_uniform(seed, (uint32_t)slots[r], step, (uint32_t)(lane + 1), PURPOSE_ACCEPT);
      fail = !(u * q < p);
    }
  }
  const unsigned long long f = __ballot(fail);
  const int a = f ? __ffsll((long long)f) - 1 : K;
  if (lane == a && bad) raise_error(err, ERR_BAD_TOKEN);   // not a token: rejected here, flagged
  if (lane == 0) acc_out[r] = a;
}

// chunk sums of row a: csp = p, csr = max(0, p - q) (dense q, a < K); grid (G, n_req)
__global__ __launch_bounds__(256) void resid_chunks_kernel(int K, int V, int dense, const float* draft_logits,
                                                            const float* target, float inv_temp,
                                                            const float* stats, int vec, const int32_t* acc,
                                                            int per_wg, float* csp, float* csr, const Nucleus* nuc) {
  const int r = blockIdx.y, lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int nch = (V + DRAW_CHUNK - 1) / DRAW_CHUNK;
  const int a = acc[r];
  const bool resid = dense && a < K;
  const int nrow = dense ? 2 * K + 1 : K + 1;
  const float* ts = stats + (int64_t)r * nrow * 2;
  const float* t = target + ((int64_t)r * (K + 1) + a) * V;
  const float* z = draft_logits + ((int64_t)r * K + (resid ? a : 0)) * V;
  const Nucleus* nr = nuc ? nuc + (int64_t)r * nrow : nullptr;
  const RowLaw P = row_law(ts, nr, a);
  const RowLaw Q = resid ? row_law(ts, nr, K + 1 + a) : P;
  const bool vv = vec != 0;
  const int ch0 = blockIdx.x * per_wg, ch1 = min(nch, ch0 + per_wg);
  float* op = csp + (int64_t)r * nch;
  float* orr = csr + (int64_t)r * nch;
  for (int c0 = ch0 + w; c0 < ch1; c0 += 16) {
    float x[4][4], y[4][4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      load4_row(t, (c0 + 4 * j) * DRAW_CHUNK + 4 * lane, V, vv, x[j]);
      if (resid) load4_row(z, (c0 + 4 * j) * DRAW_CHUNK + 4 * lane, V, vv, y[j]);
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int cb = (c0 + 4 * j) * DRAW_CHUNK + 4 * lane;
      float sp = 0.f, sr = 0.f;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        if (cb + q < V) {
          const float pv = P(x[j][q] * inv_temp, cb + q);
          sp += pv;
          if (resid) sr += fmaxf(pv - Q(y[j][q] * inv_temp, cb + q), 0.f);
        }
      }
      sp = wave_sum(sp);
      if (resid) sr = wave_sum(sr);
      if (lane == 0 && c0 + 4 * j < ch1) {
        op[c0 + 4 * j] = sp;
        if (resid) orr[c0 + 4 * j] = sr;
      }
    }
  }
}

__global__ __launch_bounds__(256) void verify_draw_kernel(int K, int V, int subset, const int32_t* slots,
                                                           const int32_t* draft_ids, const float* draft_logits,
                                                           const float* target, float inv_temp,
                                                           const float* stats, int vec, int C,
                                                           const int32_t* cand_ids, const float* cand_probs,
                                                           const int32_t* acc, const float* csp, const float* csr,
                                                           uint64_t seed, uint64_t step, int32_t* out_tokens,
                                                           int32_t* out_len, int32_t* accept_len,
                                                           int32_t* next_anchor, const Nucleus* nuc) {
  extern __shared__ float csum[];
  __shared__ float sh[4];
  __shared__ int si[2];
  __shared__ int s_nc;
  __shared__ int sc_id[SUBSET_MAX_C];
  __shared__ float sc_q[SUBSET_MAX_C];
  const int r = blockIdx.x;
  const int nch = (V + DRAW_CHUNK - 1) / DRAW_CHUNK;
  const int a = acc[r];
  const bool bonus = a == K;
  const int nrow = subset ? K + 1 : 2 * K + 1;
  const float* ts = stats + (int64_t)r * nrow * 2;
  const float* t = target + ((int64_t)r * (K + 1) + a) * V;
  const float* z = draft_logits ? draft_logits + ((int64_t)r * K + (bonus ? 0 : a)) * V : nullptr;
  const Nucleus* nr = nuc ? nuc + (int64_t)r * nrow : nullptr;
  const RowLaw P = row_law(ts, nr, a);
  const RowLaw Q = !subset && !bonus ? row_law(ts, nr, K + 1 + a) : P;
  const bool vv = vec != 0;
  if (subset && threadIdx.x == 0) {
    // candidates of the rejected position, sorted by id, equal ids merged
    int n = 0;
    if (!bonus) {
      const int64_t b = ((int64_t)r * K + a) * C;
      for (int j = 0; j < C; ++j) {
        const int id = cand_ids[b + j];
        const float q = cand_probs[b + j];
        if (id < 0 || id >= V) continue;
        int pos = n;
        while (pos > 0 && sc_id[pos - 1] > id) --pos;
        if (pos > 0 && sc_id[pos - 1] == id) {
          sc_q[pos - 1] += q;
          continue;
        }
        for (int k = n; k > pos; --k) {
          sc_id[k] = sc_id[k - 1];
          sc_q[k] = sc_q[k - 1];
        }
        sc_id[pos] = id;
        sc_q[pos] = q;
        ++n;
      }
    }
    s_nc = n;
  }
  const float* src = !bonus && !subset ? csr : csp;
  for (int c = threadIdx.x; c < nch; c += 256) csum[c] = src[(int64_t)r * nch + c];
  __syncthreads();
  const int nc = subset ? s_nc : 0;
  auto wp = [&](int c0, float* e) {
    float x[4];
    load4_row(t, c0, V, vv, x);
#pragma unroll
    for (int q = 0; q < 4; ++q) e[q] = c0 + q < V ? P(x[q] * inv_temp, c0 + q) : 0.f;
  };
  auto wr = [&](int c0, float* e) {   // the residual of ids c0..c0+3
    wp(c0, e);
    if (subset) {
      for (int k = 0; k < nc; ++k) {
        const int j = sc_id[k] - c0;
#pragma unroll
        for (int q = 0; q < 4; ++q)
          if (j == q) e[q] = fmaxf(e[q] - sc_q[k], 0.f);
      }
    } else {
      float y[4];
      load4_row(z, c0, V, vv, y);
#pragma unroll
      for (int q = 0; q < 4; ++q)
        if (c0 + q < V) e[q] = fmaxf(e[q] - Q(y[q] * inv_temp, c0 + q), 0.f);
    }
  };
  bool use_resid = !bonus;
  if (use_resid) {
    if (subset && threadIdx.x == 0) {   // p - min(p, q) at each candidate, in id order
      for (int k = 0; k < nc; ++k) {
        const int id = sc_id[k];
        const float pv = P(t[id] * inv_temp, id);
        const int ch = id / DRAW_CHUNK;
        csum[ch] = fmaxf(csum[ch] - fminf(pv, sc_q[k]), 0.f);
      }
    }
    __syncthreads();
    if (chunk_total(V, csum, sh) < RESIDUAL_EPS) {   // exhausted / underflowed: draw from p
      use_resid = false;
      for (int c = threadIdx.x; c < nch; c += 256) csum[c] = csp[(int64_t)r * nch + c];
      __syncthreads();
    }
  }
  const float u2 = philox_uniform(seed, (uint32_t)slots[r], step, (uint32_t)(a + 1), PURPOSE_RESAMPLE);
  const int pick = use_resid ? chunk_draw(V, u2, wr, csum, sh, si) : chunk_draw(V, u2, wp, csum, sh, si);
  const int32_t* d = draft_ids + (int64_t)r * K;
  int32_t* o = out_tokens + (int64_t)r * (K + 1);
  for (int i = threadIdx.x; i <= K; i += 256) o[i] = i < a ? d[i] : (i == a ? pick : -1);
  if (threadIdx.x == 0) {
    out_len[r] = a + 1;
    accept_len[r] = a;
    if (next_anchor) next_anchor[r] = pick;
  }
}

// ---------------------------------------------------------------------------
// Symmetric top-k / top-p truncation [P2 §3.3]: a distribution is cut to its
// top-k ids (probability descending, id ascending), renormalised, cut again to
// the shortest prefix of that order whose cumulative probability reaches top_p
// (the crossing id kept), and renormalised.  Sets are at most 64 ids, one lane
// per id; ids out of the set are written -1 with probability 0.
// ---------------------------------------------------------------------------
constexpr int TRUNC_MAX_K = 64;

__device__ __forceinline__ float wave_incl_scan(float v, int lane) {
  for (int o = 1; o < 64; o <<= 1) {
    const float y = __shfl_up(v, o, 64);
    if (lane >= o) v += y;
  }
  return v;
}

// one wave per row: ids_in / probs_in [rows][k] in top-k order with full-vocabulary probabilities
__global__ __launch_bounds__(64) void trunc_rows_kernel(int k, float top_p, const int32_t* ids_in,
                                                         const float* probs_in, int32_t* ids_out, float* probs_out) {
  const int64_t m = blockIdx.x;
  const int lane = threadIdx.x;
  const bool on = lane < k;
  const int id = on ? ids_in[m * k + lane] : -1;
  const float p = on ? probs_in[m * k + lane] : 0.f;
  const float r = p / wave_sum(p);
  const float incl = wave_incl_scan(r, lane);
  float excl = __shfl_up(incl, 1, 64);
  if (lane == 0) excl = 0.f;
  const bool keep = on && (top_p >= 1.f || excl < top_p);
  const float z = wave_sum(keep ? r : 0.f);
  if (on) {
    ids_out[m * k + lane] = keep ? id : -1;
    probs_out[m * k + lane] = keep ? r / z : 0.f;
  }
}

// Inverse-CDF draw in ascending id order over a lane set (ids < 0 unused):
// every lane's rank by id places the set in id order in LDS, then a prefix scan
// in that order (neighbouring ranges share end points exactly).  Returns the id
// (wave-uniform); falls back to the last id with weight.
__device__ int sparse_draw(int id, float w, float u, int lane, float* sp, int* si) {
  const bool on = id >= 0;
  int rank = 0;
  for (int l = 0; l < 64; ++l) {
    const int o = __shfl(id, l, 64);
    rank += (o >= 0 && o < id) ? 1 : 0;
  }
  sp[lane] = 0.f;
  si[lane] = -1;
  __syncthreads();
  if (on) {
    sp[rank] = w;
    si[rank] = id;
  }
  __syncthreads();
  const float ws = sp[lane];
  const int is = si[lane];
  const float incl = wave_incl_scan(ws, lane);
  float excl = __shfl_up(incl, 1, 64);
  if (lane == 0) excl = 0.f;
  const float tm = u * __shfl(incl, 63, 64);
  const unsigned long long hit = __ballot(is >= 0 && ws > 0.f && excl <= tm && tm < incl);
  int pick;
  if (hit) {
    pick = __ffsll((long long)hit) - 1;
  } else {
    const unsigned long long nz = __ballot(is >= 0 && ws > 0.f);
    pick = nz ? 63 - __clzll((long long)nz) : 0;
  }
  const int out = __shfl(is, pick, 64);
  __syncthreads();
  return out < 0 ? 0 : out;
}

// drafts from truncated rows: row j of request r draws with Philox(seed; j+1, slot, step, 0)
__global__ __launch_bounds__(64) void sparse_sample_kernel(int K, int k, const int32_t* slots, uint64_t seed,
                                                            uint64_t step, const int32_t* ids, const float* probs,
                                                            int32_t* draft_ids) {
  __shared__ float sp[64];
  __shared__ int si[64];
  const int64_t m = blockIdx.x;
  const int r = (int)(m / K), j = (int)(m % K), lane = threadIdx.x;
  const int id = lane < k ? ids[m * k + lane] : -1;
  const float w = lane < k ? probs[m * k + lane] : 0.f;
  const float u = philox_uniform(seed, (uint32_t)slots[r], step, (uint32_t)(j + 1), PURPOSE_DRAFT);
  const int pick = sparse_draw(id, w, u, lane, sp, si);
  if (lane == 0) draft_ids[m] = pick;
}

// Rejection against sparse distributions, one wave per request: p rows (target,
// truncated) [n][K+1][kp], q rows (draft: truncated, or the selector's subset)
// [n][K][kq]; ids < 0 unused, equal ids in q summed.  Same test, residual,
// fallback and Philox uniforms as rejection_kernel.
__global__ __launch_bounds__(64) void rejection_sparse_kernel(int K, int kp, int kq, const int32_t* slots,
                                                               const int32_t* draft_ids, const int32_t* p_ids,
                                                               const float* p_probs, const int32_t* q_ids,
                                                               const float* q_probs, uint64_t seed, uint64_t step,
                                                               int32_t* out_tokens, int32_t* out_len,
                                                               int32_t* accept_len, int32_t* next_anchor,
                                                               int32_t* err) {
  __shared__ float sp[64];
  __shared__ int si[64];
  const int r = blockIdx.x, lane = threadIdx.x;
  const uint32_t slot = (uint32_t)slots[r];
  const int32_t* d = draft_ids + (int64_t)r * K;
  auto p_at = [&](int row, int tok) {   // p_row(tok), wave-uniform
    const int64_t b = ((int64_t)r * (K + 1) + row) * kp;
    const float v = (lane < kp && p_ids[b + lane] == tok) ? p_probs[b + lane] : 0.f;
    return wave_sum(v);
  };
  auto q_at = [&](int row, int tok) {
    const int64_t b = ((int64_t)r * K + row) * kq;
    const float v = (lane < kq && q_ids[b + lane] == tok) ? q_probs[b + lane] : 0.f;
    return wave_sum(v);
  };
  int a = 0;
  for (; a < K; ++a) {
    const int tok = d[a];
    if (tok < 0) {
      if (lane == 0) raise_error(err, ERR_BAD_TOKEN);
      break;
    }
    const float pt = p_at(a, tok), qt = q_at(a, tok);
    const float u = philox_uniform(seed, slot, step, (uint32_t)(a + 1), PURPOSE_ACCEPT);
    if (!(u * qt < pt)) break;
  }
  // draw at row a: the residual max(0, p - q) (p alone when it is exhausted), or the bonus from p_K
  const int64_t pb = ((int64_t)r * (K + 1) + a) * kp;
  const int id = lane < kp ? p_ids[pb + lane] : -1;
  const float pv = (lane < kp && id >= 0) ? p_probs[pb + lane] : 0.f;
  float w = pv;
  if (a < K) {
    float qv = 0.f;
    const int64_t qb = ((int64_t)r * K + a) * kq;
    for (int l = 0; l < kq; ++l) {
      const int qi = q_ids[qb + l];
      if (qi == id && id >= 0) qv += q_probs[qb + l];
    }
    w = fmaxf(pv - qv, 0.f);
    if (wave_sum(w) < RESIDUAL_EPS) w = pv;   // exhausted / underflowed: draw from p
  }
  const float u2 = philox_uniform(seed, slot, step, (uint32_t)(a + 1), PURPOSE_RESAMPLE);
  const int pick = sparse_draw(id, w, u2, lane, sp, si);
  int32_t* o = out_tokens + (int64_t)r * (K + 1);
  for (int i = lane; i <= K; i += 64) o[i] = i < a ? d[i] : (i == a ? pick : -1);
  if (lane == 0) {
    out_len[r] = a + 1;
    accept_len[r] = a;
    if (next_anchor) next_anchor[r] = pick;
  }
}

// ---------------------------------------------------------------------------
// DFlash 2 dynamic convolution [P2 §3.2.3]: y_t = k_{t,0} x_t + k_{t,1} x_{t-1}
// over the R rows of each request's block (x_{-1} = 0), per channel c with
// k_{t,j}[c] = base_j[c] + corr[t][j * H/G + c/G]; corr = x . proj^T comes from
// the GEMM before (on the operand-type copy of x).  x is the sub-layer's RMSNorm
// of the fp32 residual X, recomputed here in fp32 for rows t and t-1 so that y
// is rounded to the operand type once.  One work-group per row.
// ---------------------------------------------------------------------------
template <typename T>
__global__ __launch_bounds__(256) void dyn_conv_kernel(int M, int R, int H, int G, const float* X, const float* rs,
                                                        const typename WeightOf<T>::type* gain, const float* corr,
                                                        int corr_ld, int splits, int64_t split_stride, float scale,
                                                        const typename WeightOf<T>::type* base, T* y) {
  // elementwise: one thread per four channels of one row; x_m = X_m * rs_m * gain
  // with the row scales rs written by the RMSNorm pass that produced the
  // correction product's input; the corrections are scale times the sum, in
  // split order, of the product's split partials (one split: the product itself)
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int h4 = H / 4;
  if (i >= (int64_t)M * h4) return;
  const int m = (int)(i / h4), c = (int)(i % h4) * 4;
  const bool first = m % R == 0;
  const int ng = H / G;
  const float4 v = load4f(X + (int64_t)m * H + c), g = load4f(gain + c);
  const float4 b0 = load4f(base + c), b1 = load4f(base + H + c);
  const float4 u = first ? make_float4(0.f, 0.f, 0.f, 0.f) : load4f(X + (int64_t)(m - 1) * H + c);
  const float r0 = rs[m], r1 = first ? 0.f : rs[m - 1];
  const float* cp = corr + (int64_t)m * corr_ld + c / G;
  float c0 = 0.f, c1 = 0.f;
  for (int sp = 0; sp < splits; ++sp) {
    c0 += cp[sp * split_stride];
    c1 += cp[sp * split_stride + ng];
  }
  c0 *= scale;
  c1 *= scale;
  store4(y + (int64_t)m * H + c, (b0.x + c0) * v.x * r0 * g.x + (b1.x + c1) * u.x * r1 * g.x,
         (b0.y + c0) * v.y * r0 * g.y + (b1.y + c1) * u.y * r1 * g.y,
         (b0.z + c0) * v.z * r0 * g.z + (b1.z + c1) * u.z * r1 * g.z,
         (b0.w + c0) * v.w * r0 * g.w + (b1.w + c1) * u.w * r1 * g.w);
}

// ---------------------------------------------------------------------------
// DFlash 2 path selector [P2 §3.1.2-3.1.3].  Candidates of mask position t are
// the top-C ids of its logits (top-k order); candidate b following predecessor a
// scores S_t(a, b) = z_t(b) + sum_i A[a][i] * gate_t[i] * B[b][i], gate = H(h_t).
// As the pages lay it out, every pair score is computed first, in parallel, into
// a table -- predecessors of position 0: the anchor; of position t >= 1: the C
// candidates of t-1 -- and only the walk over the table is sequential.
// ---------------------------------------------------------------------------
constexpr int SEL_RC = 120;   // rank chunk staged in LDS per pass (C = 64: 2 x 64 x 121 x 4 B < 64 KB)
constexpr int SEL_LD = SEL_RC + 1;   // padded row stride: the C successor rows fall in distinct banks

// table[r][t][i][j] = S_t(pred_i, cand_tj); grid (K, n_req), 256 threads.
template <typename W>
__global__ __launch_bounds__(256) void sel_table_kernel(int K, int C, int rank, int V, const int32_t* anchors,
                                                         const float* logits, const int32_t* cand, const float* gate,
                                                         const W* A, const W* B, float* table, int32_t* err) {
  extern __shared__ float st_lds[];          // [C][SEL_LD] gated predecessor codes, [C][SEL_LD] successor codes
  float* ap = st_lds;
  float* bs = st_lds + C * SEL_LD;
  const int t = blockIdx.x, r = blockIdx.y, tid = threadIdx.x;
  const int64_t row = (int64_t)r * K + t;
  const int np = t == 0 ? 1 : C;             // predecessors
  const int pairs = np * C;
  constexpr int PPT = 16;                    // pairs per thread (C <= 64 -> at most 4096 pairs)
  float acc[PPT];
#pragma unroll
  for (int q = 0; q < PPT; ++q) acc[q] = 0.f;
  for (int k0 = 0; k0 < rank; k0 += SEL_RC) {
    const int kn = min(SEL_RC, rank - k0);
    __syncthreads();
    for (int e = tid; e < np * SEL_RC; e += 256) {
      const int i = e / SEL_RC, k = e % SEL_RC;
      float v = 0.f;
      if (k < kn) {
        int a;
        if (t == 0) {
          a = anchors[r];
          if (a < 0 || a >= V) a = 0;
        } else {
          a = cand[(row - 1) * C + i];
        }
        v = to_f32(A[(int64_t)a * rank + k0 + k]) * gate[row * rank + k0 + k];
      }
      ap[i * SEL_LD + k] = v;
    }
    for (int e = tid; e < C * SEL_RC; e += 256) {
      const int j = e / SEL_RC, k = e % SEL_RC;
      bs[j * SEL_LD + k] = k < kn ? to_f32(B[(int64_t)cand[row * C + j] * rank + k0 + k]) : 0.f;
    }
    __syncthreads();
#pragma unroll
    for (int q = 0; q < PPT; ++q) {
      const int pidx = tid + q * 256;
      if (pidx < pairs) {
        const float* x = ap + (pidx / C) * SEL_LD;
        const float* y = bs + (pidx % C) * SEL_LD;
        float sum = 0.f;
        for (int k = 0; k < kn; ++k) sum += x[k] * y[k];
        acc[q] += sum;
      }
    }
  }
  if (t == 0 && tid == 0 && (anchors[r] < 0 || anchors[r] >= V)) raise_error(err, ERR_BAD_TOKEN);
#pragma unroll
  for (int q = 0; q < PPT; ++q) {
    const int pidx = tid + q * 256;
    if (pidx < pairs) {
      const int j = pidx % C;
      table[(row * C + pidx / C) * C + j] = logits[row * V + cand[row * C + j]] + acc[q];
    }
  }
}

// The walk over the table, one wave per request, lane j <-> candidate j.  Greedy:
// the highest score, lowest id on ties.  T > 0: softmax(S / T) over the
// candidates and an inverse-CDF draw in candidate order with u = Philox(seed;
// t+1, slot, step, 0); neighbouring lanes' prefix ranges share end points exactly.
__global__ __launch_bounds__(64) void sel_walk_kernel(int K, int C, const int32_t* slots, const int32_t* cand,
                                                       const float* table, float inv_temp, uint64_t seed,
                                                       uint64_t step, int32_t* draft_ids, int32_t* cand_out,
                                                       float* probs_out) {
  const int r = blockIdx.x, lane = threadIdx.x;
  const bool on = lane < C;
  int pidx = 0;                              // index of the predecessor among its candidates (anchor: 0)
  for (int t = 0; t < K; ++t) {
    const int64_t row = (int64_t)r * K + t;
    const int id = on ? cand[row * C + lane] : 0x7fffffff;
    const float sc = on ? table[(row * C + pidx) * C + lane] : -INFINITY;
    int pick;
    float pr;
    if (inv_temp == 0.f) {
      const float mx = wave_max(sc);
      int best = (on && sc == mx) ? id : 0x7fffffff;
      for (int o = 32; o > 0; o >>= 1) best = min(best, __shfl_xor(best, o, 64));
      const unsigned long long hit = __ballot(on && id == best);
      pick = hit ? __ffsll((long long)hit) - 1 : 0;
      pr = lane == pick ? 1.f : 0.f;
    } else {
      const float mx = wave_max(sc);
      const float e = on ? expf((sc - mx) * inv_temp) : 0.f;
      float incl = e;
      for (int o = 1; o < 64; o <<= 1) {
        const float y = __shfl_up(incl, o, 64);
        if (lane >= o) incl += y;
      }
      float excl = __shfl_up(incl, 1, 64);
      if (lane == 0) excl = 0.f;
      const float tot = __shfl(incl, 63, 64);
      const float u = philox_uniform(seed, (uint32_t)slots[r], step, (uint32_t)(t + 1), PURPOSE_DRAFT);
      const float tm = u * tot;
      const unsigned long long hit = __ballot(on && e > 0.f && excl <= tm && tm < incl);
      if (hit) {
        pick = __ffsll((long long)hit) - 1;
      } else {   // rounding put u * S on the total: the last candidate with weight
        const unsigned long long nz = __ballot(on && e > 0.f);
        pick = nz ? 63 - __clzll((long long)nz) : 0;
      }
      pr = e / tot;
    }
    if (on) {
      probs_out[row * C + lane] = pr;
      cand_out[row * C + lane] = id;
    }
    const int tok = __shfl(id, pick, 64);
    if (lane == 0) draft_ids[row] = tok;
    pidx = pick;
  }
}

// ---------------------------------------------------------------------------
// Draft-tree verifier walk [P5 §3.5]: from the root (node 0) the target's own
// decoding rule picks a token from the target row of the current node; the walk
// moves to the child carrying that token, if any, and otherwise stops with the
// pick as the new bonus token.  Greedy picks the row argmax (lowest id on ties);
// T > 0 draws by inverse CDF in ascending id order with u = Philox(seed;
// depth + 1, slot, step, 4).  out_tokens / path rows hold max_out entries
// (unused -1); a walk that would pass max_out rows stops there and flags ERR_ROWS,
// which also bounds the walk on malformed (cyclic) parent arrays.
// ---------------------------------------------------------------------------
// One work-group of 1024 threads walks one request's tree and reads only the
// rows of the nodes it visits.  A row is swept in tiles of 4096 ids: thread t
// holds ids 4096 * tile + 4t .. 4t + 3, so wave w covers the 256-id segment
// (tile, w), and segments taken in (tile, wave) order run in ascending id order.
// Greedy keeps a running (max, lowest id) per thread.  Sampling stores per
// segment (its max m_s, sum of exp(x - m_s)) in LDS during the one sweep; the
// block then scans the segment masses rescaled to the row max, finds the
// segment where u * S falls, and one wave rescans those 256 ids for the id.
constexpr int WALK_THREADS = 1024, WALK_TILE = 4 * WALK_THREADS, WALK_WAVES = WALK_THREADS / 64;
constexpr int WALK_BATCH = 12;   // tiles whose loads are in flight together (192 KB per work-group)

__device__ __forceinline__ float4 walk_load(const float* row, int V, int base, bool vec) {
  if (vec && base + 3 < V) return *(const float4*)(row + base);
  float4 q;
  q.x = base < V ? row[base] : -INFINITY;
  q.y = base + 1 < V ? row[base + 1] : -INFINITY;
  q.z = base + 2 < V ? row[base + 2] : -INFINITY;
  q.w = base + 3 < V ? row[base + 3] : -INFINITY;
  return q;
}

template <bool SAMPLE>
__global__ __launch_bounds__(WALK_THREADS) void tree_walk_kernel(int n_nodes, int max_out, int V, const int32_t* slots,
                                                                 const int32_t* tokens, const int32_t* parents,
                                                                 const float* target, float inv_temp, uint64_t seed,
                                                                 uint64_t step, int32_t* out_tokens, int32_t* out_len,
                                                                 int32_t* accept_len, int32_t* next_anchor,
                                                                 int32_t* path_out, int32_t* err) {
  extern __shared__ float2 seg[];   // SAMPLE only: [n_tiles * 16] (segment max, segment sum)
  __shared__ float red_v[WALK_WAVES];
  __shared__ int red_i[WALK_WAVES];
  __shared__ float s_total, s_before;
  __shared__ int s_seg, s_pick, s_child;
  const int r = blockIdx.x, tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int32_t* tok = tokens + (int64_t)r * n_nodes;
  const int32_t* par = parents + (int64_t)r * n_nodes;
  int32_t* o = out_tokens + (int64_t)r * max_out;
  int32_t* pth = path_out ? path_out + (int64_t)r * max_out : nullptr;
  const uint32_t slot = SAMPLE ? (uint32_t)slots[r] : 0u;
  const bool vec = (V & 3) == 0;
  const int n_tiles = (V + WALK_TILE - 1) / WALK_TILE;
  const int n_seg = n_tiles * WALK_WAVES;
  int node = 0, a = 0;
  if (pth && tid == 0) pth[0] = 0;
  for (;;) {
    const float* row = target + ((int64_t)r * n_nodes + node) * V;
    float best = -INFINITY;
    int arg = 0x7fffffff;
    for (int t0 = 0; t0 < n_tiles; t0 += WALK_BATCH) {
      float4 q[WALK_BATCH];
#pragma unroll
      for (int u = 0; u < WALK_BATCH; ++u)
        q[u] = t0 + u < n_tiles ? walk_load(row, V, (t0 + u) * WALK_TILE + 4 * tid, vec)
                                : make_float4(-INFINITY, -INFINITY, -INFINITY, -INFINITY);
#pragma unroll
      for (int u = 0; u < WALK_BATCH; ++u) {
        if (t0 + u >= n_tiles) break;
        if (!SAMPLE) {
          const int b = (t0 + u) * WALK_TILE + 4 * tid;
          if (q[u].x > best) { best = q[u].x; arg = b; }
          if (q[u].y > best) { best = q[u].y; arg = b + 1; }
          if (q[u].z > best) { best = q[u].z; arg = b + 2; }
          if (q[u].w > best) { best = q[u].w; arg = b + 3; }
        } else {
          const float x0 = q[u].x * inv_temp, x1 = q[u].y * inv_temp, x2 = q[u].z * inv_temp, x3 = q[u].w * inv_temp;
          const float m = wave_max(fmaxf(fmaxf(x0, x1), fmaxf(x2, x3)));
          float e = 0.f;
          if (m > -INFINITY) e = expf(x0 - m) + expf(x1 - m) + expf(x2 - m) + expf(x3 - m);
          e = wave_sum(e);
          if (lane == 0) seg[(t0 + u) * WALK_WAVES + wv] = make_float2(m, e);
        }
      }
    }
    int pick;
    if (!SAMPLE) {
      const float wm = wave_max(best);
      int cand = best == wm ? arg : 0x7fffffff;
      for (int off = 32; off > 0; off >>= 1) cand = min(cand, __shfl_xor(cand, off, 64));
      if (lane == 0) { red_v[wv] = wm; red_i[wv] = cand; }
      __syncthreads();
      if (tid == 0) {
        float bv = red_v[0];
        int bi = red_i[0];
        for (int i = 1; i < WALK_WAVES; ++i)
          if (red_v[i] > bv || (red_v[i] == bv && red_i[i] < bi)) { bv = red_v[i]; bi = red_i[i]; }
        s_pick = bi < V ? bi : 0;   // a row of NaN / -inf only: id 0
        s_child = 0x7fffffff;
      }
      __syncthreads();
      pick = s_pick;
    } else {
      __syncthreads();   // segment table complete
      // row max, then each thread's consecutive segments' mass at that max, scanned in thread order
      const int per = (n_seg + WALK_THREADS - 1) / WALK_THREADS;
      const int g0 = tid * per, g1 = min(n_seg, g0 + per);
      float mx = -INFINITY;
      for (int g = g0; g < g1; ++g) mx = fmaxf(mx, seg[g].x);
      mx = wave_max(mx);
      if (lane == 0) red_v[wv] = mx;
      __syncthreads();
      float M = red_v[0];
      for (int i = 1; i < WALK_WAVES; ++i) M = fmaxf(M, red_v[i]);
      float w = 0.f;
      for (int g = g0; g < g1; ++g) {
        const float2 sg = seg[g];
        if (sg.x > -INFINITY) w += sg.y * expf(sg.x - M);
      }
      float x = w;
      for (int off = 1; off < 64; off <<= 1) {
        const float y = __shfl_up(x, off, 64);
        if (lane >= off) x += y;
      }
      float xp = __shfl_up(x, 1, 64);
      if (lane == 0) xp = 0.f;
      __syncthreads();   // red_v reads done
      if (lane == 63) red_v[wv] = x;
      if (tid == 0) s_seg = -1;
      __syncthreads();
      float off_w = 0.f;
      for (int i = 0; i < wv; ++i) off_w += red_v[i];
      // [excl, incl) of neighbouring threads share their end points exactly, so
      // at most one thread's range holds u * S
      const float incl = off_w + x, excl = off_w + xp;
      if (tid == WALK_THREADS - 1) s_total = incl;
      if (tid == 0) s_child = 0x7fffffff;
      __syncthreads();
      const float u = philox_uniform(seed, slot, step, (uint32_t)(a + 1), PURPOSE_TREE_WALK);
      const float tm = u * s_total;
      if (w > 0.f && excl <= tm && tm < incl) {
        float acc = excl;
        int gs = -1;
        for (int g = g0; g < g1; ++g) {
          const float2 sg = seg[g];
          const float wg = sg.x > -INFINITY ? sg.y * expf(sg.x - M) : 0.f;
          if (wg > 0.f) { gs = g; s_before = acc; if (tm < acc + wg) break; }
          acc += wg;
        }
        s_seg = gs;
      }
      __syncthreads();
      if (tid == 0 && s_seg < 0) {   // rounding put u * S at or past the total: the last segment with mass
        float acc = 0.f;
        for (int g = 0; g < n_seg; ++g) {
          const float2 sg = seg[g];
          const float wg = sg.x > -INFINITY ? sg.y * expf(sg.x - M) : 0.f;
          if (wg > 0.f) { s_seg = g; s_before = acc; }
          acc += wg;
        }
        if (s_seg < 0) s_seg = 0;
      }
      __syncthreads();
      if (wv == 0) {   // rescan the chosen 256-id segment in ascending id order
        const int gsel = s_seg;
        const int base = (gsel / WALK_WAVES) * WALK_TILE + (gsel % WALK_WAVES) * 256 + 4 * lane;
        const float4 q = walk_load(row, V, base, vec);
        const float e0 = expf(q.x * inv_temp - M), e1 = expf(q.y * inv_temp - M), e2 = expf(q.z * inv_temp - M),
                    e3 = expf(q.w * inv_temp - M);
        const float ws = e0 + e1 + e2 + e3;
        float li = ws;
        for (int off = 1; off < 64; off <<= 1) {
          const float y = __shfl_up(li, off, 64);
          if (lane >= off) li += y;
        }
        float lp = __shfl_up(li, 1, 64);
        if (lane == 0) lp = 0.f;
        const float before = s_before;
        int last = -1;   // this lane's last id with weight
        if (ws > 0.f) last = e3 > 0.f ? base + 3 : e2 > 0.f ? base + 2 : e1 > 0.f ? base + 1 : base;
        int found = -1;
        float acc = before + lp;
        if (ws > 0.f && acc <= tm && tm < before + li) {
          const float ev[4] = {e0, e1, e2, e3};
          found = last;   // rounding inside the lane: its last id with weight
          for (int k = 0; k < 4; ++k) {
            if (ev[k] > 0.f && tm < acc + ev[k]) { found = base + k; break; }
            acc += ev[k];
          }
        }
        // the lane whose range holds u * S; else the last id of the segment with weight
        int fmin = found < 0 ? 0x7fffffff : found;
        int lmax = last;
        for (int off = 32; off > 0; off >>= 1) {
          fmin = min(fmin, __shfl_xor(fmin, off, 64));
          lmax = max(lmax, __shfl_xor(lmax, off, 64));
        }
        if (lane == 0) s_pick = fmin != 0x7fffffff ? fmin : (lmax >= 0 ? lmax : 0);
      }
      __syncthreads();
      pick = s_pick;
    }
    // the child of `node` carrying `pick`, searched by all threads (siblings carry distinct tokens;
    // the lowest index wins should a malformed tree repeat one)
    for (int c = 1 + tid; c < n_nodes; c += WALK_THREADS)
      if (par[c] == node && tok[c] == pick) atomicMin(&s_child, c);
    if (tid == 0) o[a] = pick;
    __syncthreads();
    int nxt = s_child == 0x7fffffff ? -1 : s_child;
    if (nxt >= 0 && a + 1 >= max_out) {   // deeper than the output rows allow: stop here
      if (tid == 0) raise_error(err, ERR_ROWS);
      nxt = -1;
    }
    if (nxt < 0) break;
    node = nxt;
    ++a;
    if (pth && tid == 0) pth[a] = nxt;
  }
  if (tid == 0) {
    for (int i = a + 1; i < max_out; ++i) {
      o[i] = -1;
      if (pth) pth[i] = -1;
    }
    out_len[r] = a + 1;
    accept_len[r] = a;
    if (next_anchor) next_anchor[r] = o[a];
  }
}

// ---------------------------------------------------------------------------
// Synthetic target logits (benchmark stand-in for the target model):
// row j < K = draft row j + sigma * N(0,1); row K = sigma * N(0,1).
// ---------------------------------------------------------------------------
__global__ void synth_target_kernel(int K, int V, const float* draft, float sigma, uint64_t seed, uint64_t step,
                                    float* out) {
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t rows = (int64_t)gridDim.y;
  (void)rows;
  const int rr = blockIdx.y;            // request * (K+1) + j
  if (idx >= V) return;
  const int r = rr / (K + 1), j = rr % (K + 1);
  U4 c{(uint32_t)idx, (uint32_t)rr, (uint32_t)step, PURPOSE_NOISE};
  const U4 o = philox4x32_10(c, (uint32_t)seed, (uint32_t)(seed >> 32));
  const float u1 = ((float)(o.x >> 8) + 1.0f) * (1.0f / 16777216.0f);
  const float u2 = (float)(o.y >> 8) * (1.0f / 16777216.0f);
  const float n = sqrtf(-2.0f * logf(u1)) * cosf(6.283185307f * u2);
  const float base = j < K ? draft[((int64_t)r * K + j) * V + idx] : 0.f;
  out[(int64_t)rr * V + idx] = base + sigma * n;
}

template <typename T>
__global__ void copy_cache_kernel(const T* cache_k, const T* cache_v, int layer, int slot, int start, int n,
                                  int max_batch, int n_kv, int d, int64_t ctx_alloc, KvPages pages, T* k_out,
                                  T* v_out) {
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t total = (int64_t)n * n_kv * d;
  if (idx >= total) return;
  const int e = (int)(idx % d);
  const int h = (int)((idx / d) % n_kv);
  const int i = (int)(idx / ((int64_t)d * n_kv));
  int64_t base;
  int pin;
  if (!kv_locate(pages, ctx_alloc * d, max_batch, n_kv, d, layer, slot, h, start + i, &base, &pin)) {
    k_out[idx] = (T)0.f;   // unmapped page
    v_out[idx] = (T)0.f;
    return;
  }
  k_out[idx] = cache_k[base + k_off(pin, e, d)];
  v_out[idx] = cache_v[base + v_off(pin, e, d)];
}

// paged cache: every page a request's context occupies must be mapped
__global__ void page_check_kernel(int n_req, const int32_t* slots, const int32_t* ctx_len, int max_batch,
                                  KvPages pages, int32_t* err) {
  const int r = blockIdx.x;
  const int slot = slots[r];
  if (slot < 0 || slot >= max_batch || slot >= pages.table_rows) return;
  const int np = (ctx_len[slot] + pages.page_size - 1) / pages.page_size;
  for (int p = threadIdx.x; p < np && p < pages.per_slot; p += blockDim.x) {
    const int pg = pages.table[(int64_t)slot * pages.per_slot + p];
    if ((unsigned)pg >= (unsigned)pages.n_pages) raise_error(err, ERR_PAGE);
  }
}

__global__ void reset_slots_kernel(int n, const int32_t* slots, int32_t* ctx_len, int max_batch, int32_t* err) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= n) return;
  const int s = slots[i];
  if (s < 0 || s >= max_batch) {
    raise_error(err, ERR_BAD_SLOT);
    return;
  }
  ctx_len[s] = 0;
}

// ---------------------------------------------------------------------------
// Weight conversion of a bf16 drafter (once, at handle creation).  absmax: the
// largest |w| as its fp32 bit pattern (for non-negative floats the integer order
// is the numeric order; Inf / NaN patterns sort above every finite value).
// convert: w * 2^s rounded to fp16; a bf16 value has 8 significant bits, so the
// result is exact whenever w * 2^s lies in fp16's normal range.
// ---------------------------------------------------------------------------
__global__ void absmax_bf16_kernel(const bf16_t* w, int64_t n, uint32_t* out) {
  uint32_t best = 0;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x)
    best = max(best, __float_as_uint(fabsf((float)w[i])));
  for (int o = 32; o > 0; o >>= 1) best = max(best, (uint32_t)__shfl_xor((int)best, o, 64));
  if ((threadIdx.x & 63) == 0) atomicMax(out, best);
}

__global__ void convert_bf16_f16_kernel(const bf16_t* w, int64_t n, float scale, f16_t* out) {
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x)
    out[i] = (f16_t)((float)w[i] * scale);
}

__global__ void absmax_f32_kernel(const float* w, int64_t n, uint32_t* out) {
  uint32_t best = 0;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x)
    best = max(best, __float_as_uint(fabsf(w[i])));
  for (int o = 32; o > 0; o >>= 1) best = max(best, (uint32_t)__shfl_xor((int)best, o, 64));
  if ((threadIdx.x & 63) == 0) atomicMax(out, best);
}

__global__ void convert_f32_f16_kernel(const float* w, int64_t n, float scale, f16_t* out) {
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x)
    out[i] = (f16_t)(w[i] * scale);
}

// C[r][j] = sum_k A[r][k] * B[k][j] in fp32 (A [R, K] and B [K, J] row-major),
// for products of weight matrices made once at create time.  64 x 64 output
// tiles, 16-deep K chunks staged in LDS, 4 x 4 outputs per thread.
template <typename W>
__global__ __launch_bounds__(256) void matmul_nn_kernel(int Rn, int J, int Kn, const W* A, const W* B, float* Cm) {
  __shared__ float as[16][65], bs[16][64];
  const int tid = threadIdx.x, tr = tid / 16, tc = tid % 16;
  const int r0 = blockIdx.y * 64, j0 = blockIdx.x * 64;
  float acc[4][4] = {};
  for (int k0 = 0; k0 < Kn; k0 += 16) {
    for (int e = tid; e < 64 * 16; e += 256) {
      const int rr = e / 16, kk = e % 16;         // A tile: 64 rows x 16 k
      as[kk][rr] = (r0 + rr < Rn && k0 + kk < Kn) ? to_f32(A[(int64_t)(r0 + rr) * Kn + k0 + kk]) : 0.f;
      const int kb = e / 64, jj = e % 64;         // B tile: 16 k x 64 columns
      bs[kb][jj] = (k0 + kb < Kn && j0 + jj < J) ? to_f32(B[(int64_t)(k0 + kb) * J + j0 + jj]) : 0.f;
    }
    __syncthreads();
#pragma unroll
    for (int kk = 0; kk < 16; ++kk) {
      float a[4], b[4];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        a[q] = as[kk][tr * 4 + q];
        b[q] = bs[kk][tc * 4 + q];
      }
#pragma unroll
      for (int q = 0; q < 4; ++q)
#pragma unroll
        for (int t = 0; t < 4; ++t) acc[q][t] += a[q] * b[t];
    }
    __syncthreads();
  }
#pragma unroll
  for (int q = 0; q < 4; ++q)
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const int r = r0 + tr * 4 + q, j = j0 + tc * 4 + t;
      if (r < Rn && j < J) Cm[(int64_t)r * J + j] = acc[q][t];
    }
}

__global__ void philox_fill_kernel(int n, uint64_t seed, uint32_t slot, uint64_t step, uint32_t purpose, float* out) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) out[i] = philox_uniform(seed, slot, step, (uint32_t)i, purpose);
}

// ===========================================================================
// launchers
// ===========================================================================
static inline unsigned cdiv(int64_t a, int64_t b) { return (unsigned)((a + b - 1) / b); }

void launch_rope_table(float2* table, int n_pos, int d, double theta, hipStream_t s) {
  const int64_t n = (int64_t)n_pos * (d / 2);
  rope_table_kernel<<<cdiv(n, 256), 256, 0, s>>>(table, n_pos, d, theta);
}

void launch_embed_norm(int dtype, int n_rows, int R, const int32_t* anchors, int mask_id, int vocab, const void* embed,
                       const void* mask_emb, float scale, int H, float* X, const void* gain, void* h_out, float eps,
                       int32_t* err, hipStream_t s, float* rs_out) {
  if (dtype == DT_BF16)
    embed_norm_kernel<f16_t><<<n_rows, 256, 0, s>>>(R, anchors, mask_id, vocab, (const bf16_t*)embed,
                                                     (const bf16_t*)mask_emb, scale, H, X, (const bf16_t*)gain,
                                                     (f16_t*)h_out, eps, err, rs_out);
  else
    embed_norm_kernel<float><<<n_rows, 256, 0, s>>>(R, anchors, mask_id, vocab, (const float*)embed,
                                                     (const float*)mask_emb, scale, H, X, (const float*)gain,
                                                     (float*)h_out, eps, err, rs_out);
}

void launch_rmsnorm(int dtype, int n_rows, int H, const float* X, int map_mask, int K, int R, const void* gain,
                    void* h_out, float eps, hipStream_t s, const int32_t* n_valid, int valid_base, float* rs_out) {
  if (n_rows <= 0) return;
  const int grid = n_rows;   // one 256-thread work-group per row
  if (dtype == DT_BF16)
    rmsnorm_kernel<f16_t><<<grid, 256, 0, s>>>(n_rows, H, X, map_mask, K, R, (const bf16_t*)gain, (f16_t*)h_out, eps,
                                                 n_valid, valid_base, rs_out);
  else
    rmsnorm_kernel<float><<<grid, 256, 0, s>>>(n_rows, H, X, map_mask, K, R, (const float*)gain, (float*)h_out, eps,
                                                 n_valid, valid_base, rs_out);
}

void launch_partials_add_norm(int dtype, int n_rows, int H, float* X, int map_mask, int K, int R, const float* P, int ld,
                              int splits, int64_t split_stride, float scale, const void* gain, void* h_out, float eps,
                              hipStream_t s) {
  if (n_rows <= 0) return;
  if (dtype == DT_BF16)
    partials_add_norm_kernel<f16_t><<<n_rows, 256, 0, s>>>(n_rows, H, X, map_mask, K, R, P, ld, splits, split_stride,
                                                            scale, (const bf16_t*)gain, (f16_t*)h_out, eps);
  else
    partials_add_norm_kernel<float><<<n_rows, 256, 0, s>>>(n_rows, H, X, map_mask, K, R, P, ld, splits, split_stride,
                                                            scale, (const float*)gain, (float*)h_out, eps);
}

void launch_conv_post_norm(int dtype, int n_rows, int H, int G, float* X, int map_mask, int K, int R, const float* o,
                           const float* corr, const void* base, const void* gain, void* h_out, float eps,
                           float* rs_out, hipStream_t s) {
  if (n_rows <= 0) return;
  if (dtype == DT_BF16)
    conv_post_norm_kernel<f16_t><<<n_rows, 256, 0, s>>>(n_rows, H, G, X, map_mask, K, R, o, corr,
                                                        (const bf16_t*)base, (const bf16_t*)gain, (f16_t*)h_out, eps,
                                                        rs_out);
  else
    conv_post_norm_kernel<float><<<n_rows, 256, 0, s>>>(n_rows, H, G, X, map_mask, K, R, o, corr,
                                                        (const float*)base, (const float*)gain, (float*)h_out, eps,
                                                        rs_out);
}

void launch_inject_scan(int n_req, const int32_t* slots, const int32_t* row_start, const int32_t* row_count,
                        int32_t* ctx_len, int max_ctx, int max_batch, int64_t rows_upper, int32_t* req_off,
                        int32_t* req_pos, int32_t* err, hipStream_t s) {
  (void)row_start;
  inject_scan_kernel<<<1, 64, 0, s>>>(n_req, slots, row_count, ctx_len, max_ctx, max_batch, rows_upper, req_off,
                                       req_pos, err);
}

void launch_inject_fill(int n_req, int64_t rows_upper, const int32_t* slots, const int32_t* row_start,
                        const int32_t* path_nodes, int max_path, int tree_stride, const int32_t* req_off,
                        const int32_t* req_pos, int64_t max_row, int32_t* a_rows, int32_t* row_slot,
                        int32_t* row_pos, int32_t* err, hipStream_t s) {
  if (rows_upper <= 0) return;
  inject_fill_kernel<<<cdiv(rows_upper, 256), 256, 0, s>>>(n_req, rows_upper, slots, row_start, path_nodes, max_path,
                                                           tree_stride, req_off, req_pos, max_row, a_rows, row_slot,
                                                           row_pos, err);
}

void launch_row_finalize(int n_rows, int n_tiles, const float* tmax, const float* tsum, const int32_t* targ,
                         float* row_max, float* row_lse, int32_t* argmax_out, float* out_row_max, float* out_row_lse,
                         hipStream_t s) {
  row_finalize_kernel<<<n_rows, 64, 0, s>>>(n_tiles, tmax, tsum, targ, row_max, row_lse, argmax_out, out_row_max,
                                             out_row_lse);
}

void launch_sample(int n_rows, int K, const int32_t* slots, uint64_t seed, uint64_t step, float inv_temp,
                   const float* logits, int V, int n_tiles, int tile_w, const float* tmax, const float* tsum,
                   const float* row_max, int32_t* draft_ids, hipStream_t s) {
  sample_kernel<<<n_rows, 256, 0, s>>>(K, slots, seed, step, inv_temp, logits, V, n_tiles, tile_w, tmax, tsum,
                                        row_max, draft_ids);
}

void launch_topk(int n_rows, int V, int k, const float* logits, const float* tmax, int n_tiles, int tile_w,
                 float inv_temp, const float* row_max, const float* row_lse, int32_t* ids_out, float* probs_out,
                 hipStream_t s) {
  if (k <= TOPK_SMALL_K && n_tiles <= TOPK_SMALL_TILES)
    topk_small_kernel<<<n_rows, 256, 0, s>>>(V, k, logits, tmax, n_tiles, tile_w, inv_temp, row_max, row_lse,
                                              ids_out, probs_out);
  else
    topk_kernel<<<n_rows, 256, 0, s>>>(V, k, logits, tmax, n_tiles, tile_w, inv_temp, row_max, row_lse, ids_out,
                                        probs_out);
}

void launch_tree(int n_req, int L, int Kc, int stride, int B, const float* probs, const int32_t* ids,
                 const int32_t* anchors, int32_t* tokens, int32_t* parents, int32_t* depth, uint64_t* mask,
                 hipStream_t s) {
  tree_kernel<<<n_req, 64, 0, s>>>(L, Kc, stride, B, probs, ids, anchors, tokens, parents, depth, mask);
}

void launch_verify_greedy(int n_req, int K, int V, const int32_t* draft_ids, const float* target, int32_t* post,
                          int32_t* out_tokens, int32_t* out_len, int32_t* accept_len, int32_t* next_anchor,
                          hipStream_t s) {
  argmax_rows_kernel<<<n_req * (K + 1), 256, 0, s>>>(V, target, post);
  greedy_finish_kernel<<<cdiv(n_req, 64), 64, 0, s>>>(n_req, K, draft_ids, post, out_tokens, out_len, accept_len,
                                                      next_anchor);
}

void launch_verify_tree(int n_req, int n_nodes, int max_out, int V, const int32_t* slots, const int32_t* tokens,
                        const int32_t* parents, const float* target, float temperature, uint64_t seed, uint64_t step,
                        int32_t* out_tokens, int32_t* out_len, int32_t* accept_len, int32_t* next_anchor,
                        int32_t* path_out, int32_t* err, hipStream_t s) {
  if (temperature == 0.f) {
    tree_walk_kernel<false><<<n_req, WALK_THREADS, 0, s>>>(n_nodes, max_out, V, slots, tokens, parents, target, 1.f,
                                                           seed, step, out_tokens, out_len, accept_len, next_anchor,
                                                           path_out, err);
  } else {
    const size_t lds = (size_t)tree_walk_segments(V) * sizeof(float2);
    tree_walk_kernel<true><<<n_req, WALK_THREADS, lds, s>>>(n_nodes, max_out, V, slots, tokens, parents, target,
                                                            1.0f / temperature, seed, step, out_tokens, out_len,
                                                            accept_len, next_anchor, path_out, err);
  }
}

int tree_walk_segments(int V) { return (V + WALK_TILE - 1) / WALK_TILE * WALK_WAVES; }

static inline int rows_vec_ok(int V, const float* p) { return (V & 3) == 0 && ((uintptr_t)p & 15) == 0; }
static inline size_t draw_lds_bytes(int V) { return (size_t)((V + DRAW_CHUNK - 1) / DRAW_CHUNK) * sizeof(float); }
int draw_vocab_ok(int V) { return draw_lds_bytes(V) <= 32768; }
int draw_chunks(int V) { return (V + DRAW_CHUNK - 1) / DRAW_CHUNK; }
static constexpr int RESID_CHUNKS_PER_WG = 32;

void launch_row_stats(int rows, int V, const float* x, float inv_temp, float* tmax, int n_tiles, float* out_max,
                      float* out_b, int os, int per, int group, int off, int want_log, hipStream_t s) {
  if (rows <= 0) return;
  const bool vec = rows_vec_ok(V, x);
  auto go = [&](auto kern) {
    kern<<<rows, 256, 0, s>>>(V, x, inv_temp, tmax, n_tiles, out_max, out_b, os, per, group, off, want_log);
  };
  if (tmax) {
    if (vec) go(row_stats_kernel<true, true>);
    else go(row_stats_kernel<true, false>);
  } else {
    if (vec) go(row_stats_kernel<false, true>);
    else go(row_stats_kernel<false, false>);
  }
}

void launch_verify_rejection(int n_req, int K, int V, const int32_t* slots, const int32_t* draft_ids,
                             const float* draft_logits, const float* target, float inv_temp, uint64_t seed,
                             uint64_t step, float* stats, int32_t* acc, float* chunks, int32_t* out_tokens,
                             int32_t* out_len, int32_t* accept_len, int32_t* next_anchor, int32_t* err,
                             hipStream_t s, Nucleus* nuc, float top_p) {
  // stats rows per request: K+1 target rows then K draft rows
  const int vec = rows_vec_ok(V, target) && rows_vec_ok(V, draft_logits);
  const int nch = (V + DRAW_CHUNK - 1) / DRAW_CHUNK;
  launch_row_stats(n_req * (K + 1), V, target, inv_temp, nullptr, 0, stats, stats + 1, 2, K + 1, 2 * K + 1, 0, 0, s);
  launch_row_stats(n_req * K, V, draft_logits, inv_temp, nullptr, 0, stats, stats + 1, 2, K, 2 * K + 1, K + 1, 0, s);
  if (nuc) {   // top-p sets of the target rows and of the draft rows, at the statistics' indices
    launch_nucleus(n_req * (K + 1), V, target, K + 1, 2 * K + 1, 0, stats, 2, inv_temp, top_p, nuc, s);
    launch_nucleus(n_req * K, V, draft_logits, K, 2 * K + 1, K + 1, stats, 2, inv_temp, top_p, nuc, s);
  }
  verify_accept_kernel<<<n_req, 64, 0, s>>>(K, V, 0, slots, draft_ids, draft_logits, target, inv_temp, stats, 0,
                                            nullptr, nullptr, seed, step, acc, err, nuc);
  const int per_wg = RESID_CHUNKS_PER_WG;
  float* csp = chunks;
  float* csr = chunks + (int64_t)n_req * nch;
  resid_chunks_kernel<<<dim3(cdiv(nch, per_wg), n_req), 256, 0, s>>>(K, V, 1, draft_logits, target, inv_temp, stats,
                                                                     vec, acc, per_wg, csp, csr, nuc);
  verify_draw_kernel<<<n_req, 256, draw_lds_bytes(V), s>>>(K, V, 0, slots, draft_ids, draft_logits, target, inv_temp,
                                                           stats, vec, 0, nullptr, nullptr, acc, csp, csr, seed, step,
                                                           out_tokens, out_len, accept_len, next_anchor, nuc);
}

void launch_verify_subset(int n_req, int K, int C, int V, const int32_t* slots, const int32_t* draft_ids,
                          const int32_t* cand_ids, const float* cand_probs, const float* target, float inv_temp,
                          uint64_t seed, uint64_t step, float* stats, int32_t* acc, float* chunks,
                          int32_t* out_tokens, int32_t* out_len, int32_t* accept_len, int32_t* next_anchor,
                          int32_t* err, hipStream_t s, Nucleus* nuc, float top_p) {
  const int vec = rows_vec_ok(V, target);
  const int nch = (V + DRAW_CHUNK - 1) / DRAW_CHUNK;
  launch_row_stats(n_req * (K + 1), V, target, inv_temp, nullptr, 0, stats, stats + 1, 2, 1 << 30, 1 << 30, 0, 0, s);
  if (nuc) launch_nucleus(n_req * (K + 1), V, target, 1 << 30, 1 << 30, 0, stats, 2, inv_temp, top_p, nuc, s);
  verify_accept_kernel<<<n_req, 64, 0, s>>>(K, V, 1, slots, draft_ids, nullptr, target, inv_temp, stats, C, cand_ids,
                                            cand_probs, seed, step, acc, err, nuc);
  const int per_wg = RESID_CHUNKS_PER_WG;
  resid_chunks_kernel<<<dim3(cdiv(nch, per_wg), n_req), 256, 0, s>>>(K, V, 0, nullptr, target, inv_temp, stats, vec,
                                                                     acc, per_wg, chunks, chunks, nuc);
  verify_draw_kernel<<<n_req, 256, draw_lds_bytes(V), s>>>(K, V, 1, slots, draft_ids, nullptr, target, inv_temp,
                                                           stats, vec, C, cand_ids, cand_probs, acc, chunks, chunks,
                                                           seed, step, out_tokens, out_len, accept_len, next_anchor,
                                                           nuc);
}

void launch_dyn_conv(int dtype, int M, int R, int H, int G, const float* X, const float* rs, const void* gain,
                     const float* corr, int corr_ld, int splits, int64_t split_stride, float scale, const void* base,
                     void* y, hipStream_t s) {
  const int64_t n = (int64_t)M * (H / 4);
  if (n == 0) return;
  const unsigned blocks = (unsigned)((n + 255) / 256);
  if (dtype == DT_BF16)
    dyn_conv_kernel<f16_t><<<blocks, 256, 0, s>>>(M, R, H, G, X, rs, (const bf16_t*)gain, corr, corr_ld, splits,
                                                  split_stride, scale, (const bf16_t*)base, (f16_t*)y);
  else
    dyn_conv_kernel<float><<<blocks, 256, 0, s>>>(M, R, H, G, X, rs, (const float*)gain, corr, corr_ld, splits,
                                                  split_stride, scale, (const float*)base, (float*)y);
}

void launch_sel_walk(int dtype, int n_req, int K, int C, int rank, int V, const int32_t* slots,
                     const int32_t* anchors, const float* logits, const int32_t* cand, const float* gate,
                     const void* A, const void* B, float temperature, uint64_t seed, uint64_t step, float* table,
                     int32_t* draft_ids, int32_t* cand_out, float* probs_out, int32_t* err, hipStream_t s) {
  const size_t lds = (size_t)2 * C * SEL_LD * sizeof(float);
  const dim3 grid(K, n_req);
  if (dtype == DT_BF16)
    sel_table_kernel<bf16_t><<<grid, 256, lds, s>>>(K, C, rank, V, anchors, logits, cand, gate, (const bf16_t*)A,
                                                    (const bf16_t*)B, table, err);
  else
    sel_table_kernel<float><<<grid, 256, lds, s>>>(K, C, rank, V, anchors, logits, cand, gate, (const float*)A,
                                                   (const float*)B, table, err);
  sel_walk_kernel<<<n_req, 64, 0, s>>>(K, C, slots, cand, table, temperature > 0.f ? 1.0f / temperature : 0.f, seed,
                                       step, draft_ids, cand_out, probs_out);
}

void launch_nucleus(int rows, int V, const float* logits, int per, int nrow, int off, const float* st_max,
                    int st_stride, float inv_temp, float top_p, Nucleus* out, hipStream_t s) {
  if (rows <= 0) return;
  nucleus_kernel<<<rows, NUC_THREADS, 0, s>>>(V, logits, per, nrow, off, st_max, st_stride, inv_temp, top_p,
                                              rows_vec_ok(V, logits), out);
}

void launch_nucleus_sample(int rows, int K, int V, const int32_t* slots, uint64_t seed, uint64_t step,
                           float inv_temp, const float* logits, const float* row_max, const Nucleus* nuc,
                           int32_t* draft_ids, hipStream_t s) {
  if (rows <= 0) return;
  nucleus_sample_kernel<<<rows, 256, draw_lds_bytes(V), s>>>(K, V, slots, seed, step, inv_temp, logits, row_max, nuc,
                                                            rows_vec_ok(V, logits), draft_ids);
}

void launch_trunc_rows(int rows, int k, float top_p, const int32_t* ids_in, const float* probs_in,
                       int32_t* ids_out, float* probs_out, hipStream_t s) {
  if (rows > 0) trunc_rows_kernel<<<rows, 64, 0, s>>>(k, top_p, ids_in, probs_in, ids_out, probs_out);
}

void launch_sparse_sample(int rows, int K, int k, const int32_t* slots, uint64_t seed, uint64_t step,
                          const int32_t* ids, const float* probs, int32_t* draft_ids, hipStream_t s) {
  if (rows > 0) sparse_sample_kernel<<<rows, 64, 0, s>>>(K, k, slots, seed, step, ids, probs, draft_ids);
}

void launch_verify_sparse(int n_req, int K, int kp, int kq, const int32_t* slots, const int32_t* draft_ids,
                          const int32_t* p_ids, const float* p_probs, const int32_t* q_ids, const float* q_probs,
                          uint64_t seed, uint64_t step, int32_t* out_tokens, int32_t* out_len, int32_t* accept_len,
                          int32_t* next_anchor, int32_t* err, hipStream_t s) {
  rejection_sparse_kernel<<<n_req, 64, 0, s>>>(K, kp, kq, slots, draft_ids, p_ids, p_probs, q_ids, q_probs, seed,
                                                step, out_tokens, out_len, accept_len, next_anchor, err);
}

template <typename T>
__global__ void to_f32_kernel(int64_t n, const T* src, float* dst) {
  for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x)
    dst[i] = to_f32(src[i]);
}
template <typename T>
__global__ void from_f32_kernel(int64_t n, const float* src, T* dst) {
  for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x)
    dst[i] = from_f32<T>(src[i]);
}

void launch_to_f32(int dtype, int64_t n, const void* src, float* dst, hipStream_t s) {
  const int grid = (int)std::min<int64_t>(4096, (n + 255) / 256);
  if (n <= 0) return;
  if (dtype == DT_BF16) to_f32_kernel<f16_t><<<grid, 256, 0, s>>>(n, (const f16_t*)src, dst);
  else to_f32_kernel<float><<<grid, 256, 0, s>>>(n, (const float*)src, dst);
}

void launch_from_f32(int dtype, int64_t n, const float* src, void* dst, hipStream_t s) {
  const int grid = (int)std::min<int64_t>(4096, (n + 255) / 256);
  if (n <= 0) return;
  if (dtype == DT_BF16) from_f32_kernel<f16_t><<<grid, 256, 0, s>>>(n, src, (f16_t*)dst);
  else from_f32_kernel<float><<<grid, 256, 0, s>>>(n, src, (float*)dst);
}

__global__ void sanitize_slots_kernel(int n, const int32_t* in, int32_t* out, int max_batch, int32_t* err) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= n) return;
  const int s = in[i];
  if (s < 0 || s >= max_batch) {
    raise_error(err, ERR_BAD_SLOT);
    out[i] = max_batch;   // the spare, always-empty slot
  } else {
    out[i] = s;
  }
}

void launch_sanitize_slots(int n, const int32_t* in, int32_t* out, int max_batch, int32_t* err, hipStream_t s) {
  if (n <= 0) return;
  sanitize_slots_kernel<<<cdiv(n, 64), 64, 0, s>>>(n, in, out, max_batch, err);
}

void launch_synth_target(int n_req, int K, int V, const float* draft_logits, float sigma, uint64_t seed,
                         uint64_t step, float* out, hipStream_t s) {
  dim3 grid(cdiv(V, 256), n_req * (K + 1));
  synth_target_kernel<<<grid, 256, 0, s>>>(K, V, draft_logits, sigma, seed, step, out);
}

void launch_page_check(int n_req, const int32_t* slots, const int32_t* ctx_len, int max_batch, const KvPages& pages,
                       int32_t* err, hipStream_t s) {
  if (n_req > 0 && pages.table) page_check_kernel<<<n_req, 64, 0, s>>>(n_req, slots, ctx_len, max_batch, pages, err);
}

void launch_copy_cache(int dtype, const void* cache_k, const void* cache_v, int layer, int slot, int start, int n,
                       int max_batch, int n_kv, int d, int64_t ctx_alloc, const KvPages& pages, void* k_out,
                       void* v_out, hipStream_t s) {
  const int64_t total = (int64_t)n * n_kv * d;
  if (total <= 0) return;
  if (dtype == DT_BF16)
    copy_cache_kernel<f16_t><<<cdiv(total, 256), 256, 0, s>>>((const f16_t*)cache_k, (const f16_t*)cache_v, layer,
                                                               slot, start, n, max_batch, n_kv, d, ctx_alloc, pages,
                                                               (f16_t*)k_out, (f16_t*)v_out);
  else
    copy_cache_kernel<float><<<cdiv(total, 256), 256, 0, s>>>((const float*)cache_k, (const float*)cache_v, layer,
                                                               slot, start, n, max_batch, n_kv, d, ctx_alloc, pages,
                                                               (float*)k_out, (float*)v_out);
}

void launch_absmax_bf16(const void* w, int64_t n, uint32_t* out, hipStream_t s) {
  if (n <= 0) return;
  absmax_bf16_kernel<<<(unsigned)std::min<int64_t>(cdiv(n, 256), 4096), 256, 0, s>>>((const bf16_t*)w, n, out);
}

void launch_absmax_f32(const float* w, int64_t n, uint32_t* out, hipStream_t s) {
  if (n <= 0) return;
  absmax_f32_kernel<<<(unsigned)std::min<int64_t>(cdiv(n, 256), 4096), 256, 0, s>>>(w, n, out);
}

void launch_convert_f32_f16(const float* w, int64_t n, float scale, void* out, hipStream_t s) {
  if (n <= 0) return;
  convert_f32_f16_kernel<<<(unsigned)std::min<int64_t>(cdiv(n, 256), 65536), 256, 0, s>>>(w, n, scale, (f16_t*)out);
}

void launch_matmul_nn(int dtype, int Rn, int J, int Kn, const void* A, const void* B, float* C, hipStream_t s) {
  if (Rn <= 0 || J <= 0) return;
  const dim3 grid(cdiv(J, 64), cdiv(Rn, 64));
  if (dtype == DT_BF16)
    matmul_nn_kernel<bf16_t><<<grid, 256, 0, s>>>(Rn, J, Kn, (const bf16_t*)A, (const bf16_t*)B, C);
  else
    matmul_nn_kernel<float><<<grid, 256, 0, s>>>(Rn, J, Kn, (const float*)A, (const float*)B, C);
}

void launch_convert_bf16_f16(const void* w, int64_t n, float scale, void* out, hipStream_t s) {
  if (n <= 0) return;
  convert_bf16_f16_kernel<<<(unsigned)std::min<int64_t>(cdiv(n, 256), 65536), 256, 0, s>>>((const bf16_t*)w, n, scale,
                                                                                           (f16_t*)out);
}

void launch_reset_slots(int n, const int32_t* slots, int32_t* ctx_len, int max_batch, int32_t* err, hipStream_t s) {
  if (n <= 0) return;
  reset_slots_kernel<<<cdiv(n, 64), 64, 0, s>>>(n, slots, ctx_len, max_batch, err);
}

void launch_philox_fill(int n, uint64_t seed, uint32_t slot, uint64_t step, uint32_t purpose, float* out,
                        hipStream_t s) {
  if (n <= 0) return;
  philox_fill_kernel<<<cdiv(n, 256), 256, 0, s>>>(n, seed, slot, step, purpose, out);
}

}  // namespace dfl
