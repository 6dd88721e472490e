// Block attention kernels: balanced work plan, streamed attention, partial combine.
#include <type_traits>

#include "attention.h"
#include "lds_dma.h"
#include "ops.h"

namespace dfl {

// ---------------------------------------------------------------------------
// Plan (one work-group): group counts per segment -> seg_start (exclusive scan),
// the equal range length per_wg, and the first partial record (chunk) of each
// segment.
// ---------------------------------------------------------------------------
__device__ int block_exclusive_scan(int v, int* buf, int* carry) {
  const int tid = threadIdx.x;
  buf[tid] = v;
  __syncthreads();
  for (int off = 1; off < 256; off <<= 1) {
    const int add = tid >= off ? buf[tid - off] : 0;
    __syncthreads();
    buf[tid] += add;
    __syncthreads();
  }
  const int excl = *carry + buf[tid] - v;
  __syncthreads();
  if (tid == 255) *carry += buf[255];
  __syncthreads();
  return excl;
}

__global__ __launch_bounds__(256) void attn_plan_kernel(const int32_t* slots, const int32_t* ctx_len, int n_req,
                                                         int n_kv, int splits, int n_wg_max, int min_per_wg,
                                                         int chunk_min, int chunk_max, AttnPlan* plan,
                                                         int32_t* seg_start, int32_t* chunk_base, int4* seg_desc,
                                                         int4* wg_range) {
  __shared__ int buf[256];
  __shared__ int carry;
  // the segment starts are searched once per work-group range: an LDS copy when
  // they fit (a search through global memory waits for each of its loads)
  constexpr int LDS_SEGS = 8192;
  __shared__ int ssl[LDS_SEGS + 1];
  const int tid = threadIdx.x;
  const int per_req = n_kv * splits, n_seg = n_req * per_req;
  const bool in_lds = n_seg <= LDS_SEGS;
  if (tid == 0) carry = 0;
  __syncthreads();
  for (int b = 0; b < n_seg; b += 256) {
    const int s = b + tid;
    int cnt = 0;
    if (s < n_seg) cnt = (ctx_len[slots[s / per_req]] + KV_BLOCK - 1) / KV_BLOCK + 1;
    const int st = block_exclusive_scan(cnt, buf, &carry);
    if (s < n_seg) {
      seg_start[s] = st;
      if (in_lds) ssl[s] = st;
    }
  }
  const int total = carry;
  const int per_wg = max(min_per_wg, (total + n_wg_max - 1) / max(n_wg_max, 1));
  __syncthreads();
  if (tid == 0) {
    seg_start[n_seg] = total;
    if (in_lds) ssl[n_seg] = total;
    plan->total = total;
    plan->per_wg = per_wg;
    plan->n_wg = (total + per_wg - 1) / per_wg;
    carry = 0;
  }
  __syncthreads();
  const int* ss = in_lds ? ssl : seg_start;
  for (int b = 0; b < n_seg; b += 256) {
    const int s = b + tid;
    int cnt = 0;
    if (s < n_seg) {
      const int len = ss[s + 1] - ss[s];
      const int cg = attn_chunk_groups(len, chunk_min, chunk_max);
      cnt = (len + cg - 1) / cg;
    }
    const int cb = block_exclusive_scan(cnt, buf, &carry);
    if (s < n_seg) chunk_base[s] = cb;
  }
  // per-segment descriptors and per-work-group ranges, so that an attention
  // work-group starts with two loads instead of dependent searches
  for (int s = tid; s < n_seg; s += 256)
    seg_desc[s] = make_int4(slots[s / per_req], ctx_len[slots[s / per_req]], ss[s], ss[s + 1] - ss[s]);
  auto find_seg = [&](int x) {   // last s with seg_start[s] <= x
    int lo = 0, hi = n_seg - 1;
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (ss[mid] <= x) lo = mid;
      else hi = mid - 1;
    }
    return lo;
  };
  auto chunk_start = [&](int x) {   // first chunk start at or after group x
    if (x >= total) return total;
    const int sg = find_seg(x);
    const int b = ss[sg], e = ss[sg + 1];
    const int cg = attn_chunk_groups(e - b, chunk_min, chunk_max);
    return min(e, b + (x - b + cg - 1) / cg * cg);
  };
  for (int w = tid; w < n_wg_max; w += 256) {
    const int g0 = chunk_start(min(w * per_wg, total));
    const int g1 = chunk_start(min((w + 1) * per_wg, total));
    wg_range[w] = make_int4(g0, g1, g0 < total ? find_seg(g0) : 0, 0);
  }
}

template <typename T>
__device__ __forceinline__ typename Frag<T>::type load_frag8(const T* p) {
  typename Frag<T>::type f;
  if constexpr (sizeof(T) == 2) {
    *(uint4*)&f = *(const uint4*)p;
  } else {
    ((uint4*)&f)[0] = ((const uint4*)p)[0];
    ((uint4*)&f)[1] = ((const uint4*)p)[1];
  }
  return f;
}

// s_waitcnt vmcnt(allowed * PER), allowed clamped to [0, MAXA] (a smaller count only waits longer)
template <int PER, int MAXA>
__device__ __forceinline__ void wait_groups(int allowed) {
  if constexpr (MAXA > 0) {
    if (allowed >= MAXA) {
      wait_vmcnt<MAXA * PER>();
      return;
    }
    wait_groups<PER, MAXA - 1>(allowed);
  } else {
    wait_vmcnt<0>();
  }
}

// One segment (request r, kv head, q-row part z) as seen by a work-group.
template <typename T>
struct AttnSeg {
  const T* kc;   // cache K of (slot, head), group 0 (contiguous storage)
  const T* vc;
  const T* kb;   // the block's own K / V group
  const T* vb;
  int start, len, ncache, C, cg;   // cg: groups per chunk
  int slot, kv;
  int64_t qrow;  // this lane's query row in qb (in rows of D elements)
};

// K / V of context group g (32 keys) of (slot, kv head): contiguous, or through
// the page table (an unmapped page reads page 0; the draft's page check flags
// it).  A copy wave keeps the current page's id and loads the next page's id
// when it enters a page, so the table read is off the copy issue's path.
struct PageCursor {
  int g, gin;                 // last group looked up (-1: none) and its index inside its page
  int pi, page, npi, npage;   // current page index and id; prefetched next index (-1: none) and id
};
__device__ __forceinline__ void page_cursor_reset(PageCursor& pc) {
  pc.g = -1;
  pc.gin = 0;
  pc.pi = -1;
  pc.npi = -1;
  pc.page = pc.npage = 0;
}

template <typename T, int D, bool PAGED>
__device__ __forceinline__ void ctx_group_ptrs(const AttnArgs& a, PageCursor& pc, const T* kc, const T* vc, int slot,
                                               int kv, int g, int ncache, const T** kp, const T** vp) {
  constexpr int BLK = KV_BLOCK * D;
  if constexpr (!PAGED) {
    *kp = kc + (int64_t)g * BLK;
    *vp = vc + (int64_t)g * BLK;
    return;
  }
  // groups are visited in order inside a segment: step the in-page index, divide only on a jump
  int pi;
  if (g == pc.g + 1 && pc.g >= 0) {
    pi = pc.pi;
    if (++pc.gin == a.gpp) {
      pc.gin = 0;
      ++pi;
    }
  } else {
    pi = g / a.gpp;
    pc.gin = g - pi * a.gpp;
  }
  pc.g = g;
  if (pi != pc.pi) {
    const int32_t* row = a.page_table + (int64_t)(slot < a.table_rows ? slot : 0) * a.pages_per_slot;
    pc.page = pi == pc.npi ? pc.npage : row[pi];
    pc.pi = pi;
    pc.npi = (pi + 1) * a.gpp < ncache ? pi + 1 : -1;
    if (pc.npi >= 0) pc.npage = row[pc.npi];
  }
  const int page = slot < a.table_rows && (unsigned)pc.page < (unsigned)a.n_pages ? pc.page : 0;
  const int64_t off = page * a.page_elems + ((int64_t)kv * a.gpp + pc.gin) * BLK;
  *kp = (const T*)a.cache_k + off;
  *vp = (const T*)a.cache_v + off;
}

// Streamed attention.  Work-group w takes the chunks that start in groups
// [w*per_wg, (w+1)*per_wg) of the global group order; one wave per 16-row query
// tile of the segment's rows.
// Copying waves move each group (K block then V block, 1 KB per wave copy) into
// a ring of S LDS stages, S - 2 groups ahead of the compute; a step computes one
// or two groups of the same segment after the copying waves' vmcnt wait and a
// barrier, which also retires the stages the next copies overwrite.
//
// Per group and tile: S^T (32 x 16) = K Q^T (MFMA, K from LDS, Q in registers),
// P = exp2(scale*s - m) rounded to the operand type, O^T += V^T P^T, with l the
// sum of the unrounded P.  The reference m is an integer in the exp2 domain and
// moves lazily: only when a scaled score passes it by more than 8 is it raised
// (to the ceiling of the row max) and O, l rescaled by an exact power of two, so
// P <= 2^8 and the rounding of P to the operand type does not depend on where
// the reference sits (a power-of-two shift leaves the significand alone).  Keys
// past a segment's end are masked out of the scores and their values zeroed
// (stale cache contents must not turn 0 * x into NaN).
//
// Register budget: three waves per SIMD (<= 168 VGPRs) so that two 5-wave
// work-groups share a CU.
template <typename T, int D, int QRT, int S, bool PAGED>
__global__ __launch_bounds__(QRT * 64) __attribute__((amdgpu_waves_per_eu(sizeof(T) == 2 && QRT == 5 ? 3 : 1)))
void attn_kernel(const AttnArgs a) {
  constexpr int KS = D / 32, DT = D / 16, ROWS = QRT * 16;
  constexpr int BLK = KV_BLOCK * D;                        // elements of a K (or V) block
  constexpr int EPC = 16 / (int)sizeof(T);                 // elements per 16-byte copy
  constexpr int IPG = 2 * BLK / (64 * EPC);                // 1 KB wave copies per group (K, then V)
  constexpr int CW = QRT >= 4 ? 4 : (QRT >= 2 ? 2 : 1);    // waves that issue copies
  constexpr int PER = IPG / CW;                            // copies per copying wave per group
  constexpr int VOFF = IPG / 2 * 64;                       // first uint4 of the V block in a stage
  constexpr int MAXA = (S - 1) * PER < 64 ? S - 1 : 63 / PER;  // groups a wait may leave in flight
  constexpr float TAU = 8.f;                               // lazy-rescale threshold (exp2 units)
  static_assert(IPG % CW == 0 && PER < 64 && S >= 4 && S <= 8, "copy split / vmcnt range");
  typedef typename Frag<T>::type FragT;
  __shared__ uint4 ring[S][IPG * 64];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int grp = lane >> 4, r16 = lane & 15;
  const int4 rg = a.wg_range[blockIdx.x];   // (first group, end group, first segment), from the plan
  const int g0 = rg.x, g1 = rg.y;
  if (g0 >= g1) return;

  auto decode = [&](int s, AttnSeg<T>& d) {
    const int per_req = a.n_kv * a.splits;
    const int r = s / per_req, rem = s - r * per_req, kv = rem / a.splits, z = rem - kv * a.splits;
    const int4 sd = a.seg_desc[s];   // (slot, context length, first group, group count)
    const int slot = sd.x;
    d.C = sd.y;
    d.ncache = (d.C + KV_BLOCK - 1) / KV_BLOCK;
    d.start = sd.z;
    d.len = sd.w;
    d.cg = attn_chunk_groups(d.len, a.chunk_min, a.chunk_max);
    d.slot = slot;
    d.kv = kv;
    const int64_t head = (int64_t)slot * a.n_kv + kv;
    d.kc = (const T*)a.cache_k + head * a.ctx_alloc * D;
    d.vc = (const T*)a.cache_v + head * a.ctx_alloc * D;
    const int64_t bh = (int64_t)r * a.n_kv + kv;
    d.kb = (const T*)a.kb + bh * a.Rpad * D;
    d.vb = (const T*)a.vb + bh * a.Rpad * D;
    d.qrow = bh * a.QRpad + (int64_t)z * a.rows_per_split + wave * 16 + r16;
  };

  const int s0 = rg.z;

  // copy cursor
  AttnSeg<T> is;
  decode(s0, is);
  int is_s = s0, is_l = g0 - is.start, issued = g0, is_stage = 0;
  PageCursor pcur;
  page_cursor_reset(pcur);
  auto issue = [&]() {
    if (wave < CW) {
      const int st = is_stage;
      const bool in_cache = is_l < is.ncache;
      const T* kp = is.kb;
      const T* vp = is.vb;
      if (in_cache) ctx_group_ptrs<T, D, PAGED>(a, pcur, is.kc, is.vc, is.slot, is.kv, is_l, is.ncache, &kp, &vp);
      kp += lane * EPC;
      vp += lane * EPC;
#pragma unroll
      for (int c = 0; c < PER; ++c) {
        const int i = wave * PER + c;
        const T* src = i < IPG / 2 ? kp + i * 64 * EPC : vp + (i - IPG / 2) * 64 * EPC;
        copy16_to_lds(src, &ring[st][i * 64]);
      }
    }
    ++issued;
    if (++is_stage == S) is_stage = 0;
    if (++is_l == is.len && issued < g1) {
      ++is_s;
      decode(is_s, is);
      is_l = 0;
      page_cursor_reset(pcur);
    }
  };

  // compute cursor
  AttnSeg<T> cs = is;
  int cs_s = s0, cl = g0 - cs.start;
  FragT qf[KS];
  auto load_q = [&]() {
    const T* q = (const T*)a.qb + cs.qrow * D;
#pragma unroll
    for (int s = 0; s < KS; ++s) qf[s] = load_frag8<T>(q + s * 32 + grp * 8);
  };
  load_q();

  f32x4 acc[DT];
  const float c = a.scale_log2;
  float m_ref, l_sum;   // m_ref: integer reference in the exp2 domain of the scaled scores
  auto reset = [&]() {
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) acc[dt] = f32x4{0.f, 0.f, 0.f, 0.f};
    m_ref = -INFINITY;
    l_sum = 0.f;
  };
  reset();

  auto frag_at = [&](const uint4* stage, int f) {  // fragment f (in 64-lane units) of this lane
    FragT x;
    if constexpr (sizeof(T) == 2) {
      *(uint4*)&x = stage[f * 64 + lane];
    } else {
      ((uint4*)&x)[0] = stage[2 * (f * 64 + lane)];
      ((uint4*)&x)[1] = stage[2 * (f * 64 + lane) + 1];
    }
    return x;
  };

  auto compute = [&](auto ngc, int stage) {
    constexpr int NG = decltype(ngc)::value;
    const uint4* st[NG];
    int nval[NG];
    f32x4 sc[NG][2];
#pragma unroll
    for (int g = 0; g < NG; ++g) {
      st[g] = ring[stage + g < S ? stage + g : stage + g - S];
      const int lg = cl + g;
      nval[g] = lg < cs.ncache ? min(KV_BLOCK, cs.C - KV_BLOCK * lg) : a.R;
      sc[g][0] = sc[g][1] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
#pragma unroll
    for (int s = 0; s < KS; ++s)
#pragma unroll
      for (int g = 0; g < NG; ++g) {
        Frag<T>::mma(sc[g][0], frag_at(st[g], s), qf[s]);
        Frag<T>::mma(sc[g][1], frag_at(st[g], KS + s), qf[s]);
      }
    // lane holds keys 8*grp + i (sc[.][0]) and 8*grp + 4 + i (sc[.][1]) of each group, query row r16
#pragma unroll
    for (int g = 0; g < NG; ++g) {
      if (nval[g] < KV_BLOCK) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          if (8 * grp + i >= nval[g]) sc[g][0][i] = -INFINITY;
          if (8 * grp + 4 + i >= nval[g]) sc[g][1][i] = -INFINITY;
        }
      }
      if (a.causal && cl + g >= cs.ncache) {   // the block's own keys: key j visible to block rows >= j
        const int jrow = (wave * 16 + r16) % a.R;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          if (8 * grp + i > jrow) sc[g][0][i] = -INFINITY;
          if (8 * grp + 4 + i > jrow) sc[g][1][i] = -INFINITY;
        }
      }
    }
    // lane-local max; the row max over the 4 lane groups is only formed when some
    // score passes the reference by more than the threshold (the rare rescale)
    float mx = -INFINITY;
#pragma unroll
    for (int g = 0; g < NG; ++g)
#pragma unroll
      for (int i = 0; i < 4; ++i) mx = fmaxf(mx, fmaxf(sc[g][0][i], sc[g][1][i]));
    mx *= c;
    if (__any(mx > m_ref + TAU)) {
      mx = fmaxf(mx, __shfl_xor(mx, 16, 64));
      mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
      const float mnew = fmaxf(m_ref, ceilf(mx));
      const float alpha = mnew > m_ref ? __builtin_amdgcn_exp2f(m_ref - mnew) : 1.f;   // a power of two
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) acc[dt] *= alpha;
      l_sum *= alpha;
      m_ref = mnew;
    }
    FragT pf[NG];
#pragma unroll
    for (int g = 0; g < NG; ++g)
#pragma unroll
      for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float p = __builtin_amdgcn_exp2f(fmaf(sc[g][t][i], c, -m_ref));
          l_sum += p;
          pf[g][4 * t + i] = (T)p;
        }
#pragma unroll
    for (int g = 0; g < NG; ++g) {
      FragT vf[DT];
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) vf[dt] = frag_at(st[g] + VOFF, dt);
      if (nval[g] < KV_BLOCK) {
#pragma unroll
        for (int dt = 0; dt < DT; ++dt)
#pragma unroll
          for (int e = 0; e < 8; ++e)
            if (grp * 8 + e >= nval[g]) vf[dt][e] = (T)0.f;
      }
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) Frag<T>::mma(acc[dt], vf[dt], pf[g]);
    }
  };

  // partial record of chunk `ck` of segment cs_s: O rows of this wave, max (exp2 domain), sum
  auto flush = [&](int ck) {
    float l = l_sum;
    l += __shfl_xor(l, 16, 64);
    l += __shfl_xor(l, 32, 64);
    const int64_t piece = a.chunk_base[cs_s] + ck;
    const int row = wave * 16 + r16;
    if (row >= a.rows_per_split) return;  // padding rows of the last tile are never combined
    float* op = a.o_part + (piece * ROWS + row) * D + 4 * grp;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) *(f32x4*)(op + dt * 16) = acc[dt];
    if (grp == 0) {
      a.m_part[piece * ROWS + row] = m_ref;
      a.l_part[piece * ROWS + row] = l;
    }
  };

  while (issued < min(g1, g0 + S - 2)) issue();
  int stage = 0;                                   // ring stage of group gi
  int ck = cl / cs.cg;                             // chunk being computed (segment-local index)
  int cend = min(cs.len, (ck + 1) * cs.cg);        // its end (segment-local group)
  for (int gi = g0; gi < g1;) {
    const int n = cl + 1 < cend ? 2 : 1;
    if (wave < CW) wait_groups<PER, MAXA>(issued - (gi + n));
    lds_barrier();
    while (issued < min(g1, gi + S)) issue();
    if (n == 2) compute(std::integral_constant<int, 2>{}, stage);
    else compute(std::integral_constant<int, 1>{}, stage);
    stage += n;
    if (stage >= S) stage -= S;
    gi += n;
    cl += n;
    if (cl == cend) {  // chunk done (ranges end on chunk starts, so never mid-chunk)
      flush(ck);
      reset();
      ++ck;
      cend = min(cs.len, cend + cs.cg);
    }
    if (cl == cs.len && gi < g1) {  // next segment: its pointers and query rows
      ++cs_s;
      decode(cs_s, cs);
      cl = 0;
      ck = 0;
      cend = min(cs.len, cs.cg);
      load_q();
    }
  }
}

// Streamed attention for 16-bit K/V: NWV waves per work-group share one LDS ring.
// The groups of all segments, laid end to end, are cut into equal ranges of
// a.plan->per_wg groups, one per work-group (no snapping: a range may start or
// end inside a segment).  The work-group streams its range through a ring of S
// LDS stages, S - 1 groups ahead: each group (K block then V block; the cache's
// 32-key blocks are stored in MFMA operand order, so each fragment is one
// coalesced 1 KB wave copy) is copied global -> LDS with 16-byte direct copies,
// each wave copying its share of the fragments.  Per group: every wave waits
// for its own copies, then one barrier publishes the group and retires the
// stage the next copies overwrite.  The segment's query tiles are divided among
// the waves (Q fragments and O accumulators in registers), so each wave holds
// at most ceil(QRT / NWV) tiles and two waves fit on a SIMD.  Each (work-group,
// segment) piece of work ends in one partial record (unnormalised O,
// reference max, sum) at index w + s, which is unique: a work-group meets
// consecutive segments and a segment consecutive work-groups.  The combine
// merges a segment's records in work-group order.
//
// Per group and tile: S^T (32 x 16) = K Q^T (MFMA), P = exp2(scale*s - m)
// rounded to the operand type, O^T += V^T P^T, with l the sum of the unrounded
// P.  The reference m is an integer in the exp2 domain and moves lazily: only
// when a scaled score passes it by more than 8 is it raised (to the ceiling of
// the row max) and O, l rescaled by an exact power of two, so P <= 2^8 and the
// rounding of P to the operand type does not depend on where the reference
// sits (a power-of-two shift leaves the significand alone).  Keys past a
// segment's end are masked out of the scores and their values zeroed (stale
// cache contents must not turn 0 * x into NaN).
template <typename T, int D, int QRT, int NWV, int S, int WPE, bool PAGED>
__global__ __launch_bounds__(NWV * 64) __attribute__((amdgpu_waves_per_eu(WPE, WPE))) void attn_wave_kernel(
    const AttnArgs a) {
  constexpr int KS = D / 32, DT = D / 16, ROWS = QRT * 16;
  constexpr int NF = 2 * KS + DT;                          // 1 KB fragments per group (K then V)
  constexpr int CPW = NF / NWV;                            // copies per wave per group
  constexpr int QLO = QRT / NWV, QHI = (QRT + NWV - 1) / NWV;   // tiles per wave: wave v holds [vQRT/NWV, (v+1)QRT/NWV)
  constexpr float TAU = 8.f;
  static_assert(sizeof(T) == 2, "16-bit K/V");
  static_assert(NF % NWV == 0 && (S - 2) * CPW < 64 && S >= 2, "ring");
  static_assert(QLO >= 1, "every wave holds a tile");
  typedef typename Frag<T>::type FragT;

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int grp = lane >> 4, r16 = lane & 15;
  const int t0 = wave * QRT / NWV;                         // first tile of this wave
  const int w = blockIdx.x;
  const int4 rg = a.wg_range[w];
  const int g0 = rg.x, g1 = rg.y;
  if (g0 >= g1) return;

  __shared__ uint4 ring[S][NF * 64];
  const uint32_t ring_lds = lds_addr(&ring[0][0]);

  struct Seg {
    const T* kc; const T* vc; const T* kb; const T* vb;
    int start, len, ncache, C, slot, kv;
    int64_t q0;
  };
  auto decode = [&](int s, Seg& d) {
    const int per_req = a.n_kv * a.splits;
    const int r = s / per_req, rem = s - r * per_req, kv = rem / a.splits, z = rem - kv * a.splits;
    const int4 sd = a.seg_desc[s];
    d.slot = sd.x;
    d.C = sd.y;
    d.ncache = (d.C + KV_BLOCK - 1) / KV_BLOCK;
    d.start = sd.z;
    d.len = sd.w;
    d.kv = kv;
    const int64_t head = (int64_t)d.slot * a.n_kv + kv;
    d.kc = (const T*)a.cache_k + head * a.ctx_alloc * D;
    d.vc = (const T*)a.cache_v + head * a.ctx_alloc * D;
    const int64_t bh = (int64_t)r * a.n_kv + kv;
    d.kb = (const T*)a.kb + bh * a.Rpad * D;
    d.vb = (const T*)a.vb + bh * a.Rpad * D;
    d.q0 = bh * a.QRpad + (int64_t)z * a.rows_per_split;
  };

  // ---- copy cursor: the next group to copy into the ring (stage = its index in the range mod S)
  int ls_s = rg.z;
  Seg ls;
  decode(ls_s, ls);
  int ls_l = g0 - ls.start;
  int ls_stage = 0;
  PageCursor pcur;
  page_cursor_reset(pcur);
  auto issue = [&]() {
    const T* kp = ls.kb;
    const T* vp = ls.vb;
    if (ls_l < ls.ncache) ctx_group_ptrs<T, D, PAGED>(a, pcur, ls.kc, ls.vc, ls.slot, ls.kv, ls_l, ls.ncache, &kp, &vp);
#pragma unroll
    for (int c = 0; c < CPW; ++c) {
      const int f = wave * CPW + c;
      const T* src = f < 2 * KS ? kp + (f * 64 + lane) * 8 : vp + ((f - 2 * KS) * 64 + lane) * 8;
      copy16_to_lds_m0(src, ring_lds + (uint32_t)(ls_stage * NF + f) * 1024u);
    }
    if (++ls_stage == S) ls_stage = 0;
    if (++ls_l == ls.len) {   // the next segment (decoded even when the range ends here: its descriptor exists)
      if (ls_s + 1 < a.n_seg) {
        ++ls_s;
        decode(ls_s, ls);
      }
      ls_l = 0;
      page_cursor_reset(pcur);
    }
  };

  // ---- compute: this wave's NT tiles (Q fragments and O accumulators in registers)
  auto run = [&](auto ntc) {
  constexpr int NT = decltype(ntc)::value;
  int cs_s = rg.z;
  Seg cs;
  decode(cs_s, cs);
  int cl = g0 - cs.start;
  FragT qf[NT][KS];
  auto load_q = [&]() {
#pragma unroll
    for (int i = 0; i < NT; ++i) {
      const int row = (t0 + i) * 16 + r16;
#pragma unroll
      for (int s = 0; s < KS; ++s) {
        uint4 v = make_uint4(0, 0, 0, 0);
        if (row < a.rows_per_split) v = *(const uint4*)((const T*)a.qb + (cs.q0 + row) * D + s * 32 + grp * 8);
        *(uint4*)&qf[i][s] = v;
      }
    }
  };
  load_q();

  f32x4 acc[NT][DT];
  float m_ref[NT], l_sum[NT];
  const float c = a.scale_log2;
  auto reset = [&]() {
#pragma unroll
    for (int i = 0; i < NT; ++i) {
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) acc[i][dt] = f32x4{0.f, 0.f, 0.f, 0.f};
      m_ref[i] = -INFINITY;
      l_sum[i] = 0.f;
    }
  };
  reset();

  // one group from ring stage st; three phases over this wave's tiles, so that
  // each phase's MFMAs and VALU work are independent across tiles
  // masked: a group with keys past the segment's end or the block's own keys
  auto compute = [&](bool masked, int st) {
    const int nval = cl < cs.ncache ? min(KV_BLOCK, cs.C - KV_BLOCK * cl) : a.R;
    // S^T = K Q^T; lane holds keys 8*grp + i (sc[i][0]) and 8*grp + 4 + i (sc[i][1])
    f32x4 sc[NT][2];
#pragma unroll
    for (int i = 0; i < NT; ++i) sc[i][0] = sc[i][1] = f32x4{0.f, 0.f, 0.f, 0.f};
    // K fragments in two halves of the head dim, each read at once (one LDS latency per half)
    constexpr int KH = KS / 2;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      FragT kf[2 * KH];
#pragma unroll
      for (int s = 0; s < KH; ++s) {
        *(uint4*)&kf[s] = ring[st][(h * KH + s) * 64 + lane];
        *(uint4*)&kf[KH + s] = ring[st][(KS + h * KH + s) * 64 + lane];
      }
#pragma unroll
      for (int s = 0; s < KH; ++s) {
#pragma unroll
        for (int i = 0; i < NT; ++i) {
          Frag<T>::mma(sc[i][0], kf[s], qf[i][h * KH + s]);
          Frag<T>::mma(sc[i][1], kf[KH + s], qf[i][h * KH + s]);
        }
      }
    }
    // the first half of the V fragments is read before the softmax, whose work
    // hides the latency; the second half when the products start
    constexpr int VH = DT / 2;
    FragT vf[DT];
#pragma unroll
    for (int dt = 0; dt < VH; ++dt) *(uint4*)&vf[dt] = ring[st][(2 * KS + dt) * 64 + lane];
    // masks, lazy reference, probabilities
    FragT pf[NT];
#pragma unroll
    for (int i = 0; i < NT; ++i) {
      const int t = t0 + i;
      if (masked) {
        // keys below lim are visible: the valid keys, and for the block's own
        // keys under the causal mask key j only to block rows >= j
        int lim = nval;
        if (a.causal && cl >= cs.ncache) lim = min(lim, (t * 16 + r16) % a.R + 1);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          if (8 * grp + j >= lim) sc[i][0][j] = -INFINITY;
          if (8 * grp + 4 + j >= lim) sc[i][1][j] = -INFINITY;
        }
      }
      float mx = -INFINITY;
#pragma unroll
      for (int j = 0; j < 4; ++j) mx = fmaxf(mx, fmaxf(sc[i][0][j], sc[i][1][j]));
      mx *= c;
      if (__any(mx > m_ref[i] + TAU)) {
        mx = fmaxf(mx, __shfl_xor(mx, 16, 64));
        mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
        const float mnew = fmaxf(m_ref[i], ceilf(mx));
        const float alpha = mnew > m_ref[i] ? __builtin_amdgcn_exp2f(m_ref[i] - mnew) : 1.f;   // a power of two
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) acc[i][dt] *= alpha;
        l_sum[i] *= alpha;
        m_ref[i] = mnew;
      }
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const float p0 = __builtin_amdgcn_exp2f(fmaf(sc[i][0][j], c, -m_ref[i]));
        const float p1 = __builtin_amdgcn_exp2f(fmaf(sc[i][1][j], c, -m_ref[i]));
        l_sum[i] += p0 + p1;
        pf[i][j] = (T)p0;
        pf[i][4 + j] = (T)p1;
      }
    }
    // O^T += V^T P^T; values of keys past the end are zeroed (stale cache contents
    // must not turn 0 * x into NaN): the halves of this lane's eight keys that
    // hold valid values (all of them in a full group)
    const int nv = nval - grp * 8;
    uint32_t mk[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) mk[j] = (2 * j < nv ? 0xFFFFu : 0u) | (2 * j + 1 < nv ? 0xFFFF0000u : 0u);
#pragma unroll
    for (int dt = VH; dt < DT; ++dt) *(uint4*)&vf[dt] = ring[st][(2 * KS + dt) * 64 + lane];
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) {
#pragma unroll
      for (int j = 0; j < 4; ++j) ((uint32_t*)&vf[dt])[j] &= mk[j];
#pragma unroll
      for (int i = 0; i < NT; ++i) Frag<T>::mma(acc[i][dt], vf[dt], pf[i]);
    }
  };

  // The record of a piece holds O / l, the piece's own normalised output, as
  // fp16 (|O / l| is at most the largest |value|; one more rounding of the same
  // size as the output's own), in the accumulators' fragment order, so that every
  // store is one contiguous 512-byte wave write: tile t, 16-column block dt,
  // lane, 4 values (row 16t + lane % 16, columns 16dt + 4(lane / 16) + i), all 16
  // rows of a tile (rows past rows_per_split are never read).  Reference max and
  // sum per row in fp32.
  auto flush = [&](int64_t piece) {
    typedef _Float16 h4 __attribute__((ext_vector_type(4)));
#pragma unroll
    for (int i = 0; i < NT; ++i) {
      float l = l_sum[i];
      l += __shfl_xor(l, 16, 64);
      l += __shfl_xor(l, 32, 64);
      const float il = 1.f / l;
      h4* op = (h4*)a.o_part + ((piece * QRT + t0 + i) * DT) * 64 + lane;
#pragma unroll
      for (int dt = 0; dt < DT; ++dt)
        op[dt * 64] = h4{(_Float16)(acc[i][dt][0] * il), (_Float16)(acc[i][dt][1] * il),
                         (_Float16)(acc[i][dt][2] * il), (_Float16)(acc[i][dt][3] * il)};
      const int row = (t0 + i) * 16 + r16;
      if (grp == 0) {
        a.m_part[piece * ROWS + row] = m_ref[i];
        a.l_part[piece * ROWS + row] = l;
      }
    }
  };

  // Ring discipline.  Group k of the range lives in stage k mod S.  Only the
  // ring's copies and, at a segment change, the record stores and Q loads use
  // the vector-memory counter; loads complete in issue order, so "at most n
  // operations outstanding" with n the copies of the groups issued after group
  // k means this wave's copies of group k have landed (extra operations after
  // them only make the wait stricter).  The barrier then makes every wave's
  // copies visible, and (each wave having drained its LDS reads first) frees
  // the stage of group k - 1 for group k + S - 1.
  int issued = g0;
  for (; issued < g1 && issued < g0 + S - 1; ++issued) issue();
  int stage = 0;
  for (int gi = g0; gi < g1; ++gi) {
    const int ahead = issued - gi - 1;   // groups issued after this one
    if constexpr (S >= 4) {
      if (ahead >= 2) wait_vmcnt<2 * CPW>();
      else if (ahead == 1) wait_vmcnt<CPW>();
      else wait_vmcnt<0>();
    } else if constexpr (S == 3) {
      if (ahead >= 1) wait_vmcnt<CPW>();
      else wait_vmcnt<0>();
    } else {
      wait_vmcnt<0>();
    }
    wait_lgkmcnt0();
    lds_barrier();
    if (issued < g1) {
      issue();
      ++issued;
    }
    // the cache part's last group may be partial; the block's own group is masked when causal or partial
    const bool full = cl < cs.ncache ? cs.C - KV_BLOCK * cl >= KV_BLOCK : (a.R >= KV_BLOCK && !a.causal);
    compute(!full, stage);
    if (++stage == S) stage = 0;
    ++cl;
    const bool seg_end = cl == cs.len;
    if (seg_end || gi + 1 == g1) {
      const int64_t piece = (int64_t)w + cs_s;
      if (seg_end && gi + 1 < g1) {   // the next segment's Q loads go out before the record stores
        ++cs_s;
        decode(cs_s, cs);
        cl = 0;
        load_q();
      }
      flush(piece);
      if (seg_end && gi + 1 < g1) reset();
    }
  }
  };
  // every wave runs the same group sequence and barriers; only the tile count differs
  if constexpr (QLO == QHI) {
    run(std::integral_constant<int, QLO>{});
  } else {
    if ((wave + 1) * QRT / NWV - t0 == QHI) run(std::integral_constant<int, QHI>{});
    else run(std::integral_constant<int, QLO>{});
  }
}

// Combine of the 16-bit path's piece records (fp16 O / l in fragment order, see
// attn_wave_kernel).  One work-group per (request, kv head and q-row part, 16-row
// tile): thread x owns the 4-value elements x + 256k of the tile's record (all of
// one row, lane x % 64), so every record load is one contiguous 2 KB block read;
// the segment's records are merged in work-group order in one pass (running
// max, earlier sums rescaled), each weighted by its own sum.
template <typename T, int D>
__global__ __launch_bounds__(256) void attn_combine_frag_kernel(const AttnCombineArgs a) {
  typedef _Float16 h4 __attribute__((ext_vector_type(4)));
  constexpr int DT = D / 16, EPT = DT * 64 / 256;   // elements per thread
  constexpr int CB = 8;   // records whose loads are issued together (measured: 8 over 4 and 16)
  const int req = blockIdx.x;
  const int kv = blockIdx.y / a.splits, z = blockIdx.y % a.splits;
  const int t = blockIdx.z, lane = threadIdx.x & 63;
  const int row = t * 16 + (lane & 15);
  if (row >= a.rows_per_split) return;
  const int seg = (req * a.n_kv + kv) * a.splits + z;
  // one record per work-group range the segment meets, at w + seg
  const int per = a.wave_plan->per_wg;
  const int w0 = a.seg_start[seg] / per, w1 = (a.seg_start[seg + 1] - 1) / per;
  const int n = w1 - w0 + 1;
  const int64_t p0 = (int64_t)w0 + seg;
  const int QRT = a.QRT16 >> 4;
  float M = -INFINITY, L = 0.f;
  float O[EPT][4];
#pragma unroll
  for (int k = 0; k < EPT; ++k) O[k][0] = O[k][1] = O[k][2] = O[k][3] = 0.f;
  for (int c0 = 0; c0 < n; c0 += CB) {   // CB records' loads issued together
    float mc[CB], lc[CB];
    h4 hc[CB][EPT];
#pragma unroll
    for (int u = 0; u < CB; ++u) {
      const int64_t b = p0 + min(c0 + u, n - 1);
      mc[u] = c0 + u < n ? a.m_part[b * a.QRT16 + row] : -INFINITY;
      lc[u] = a.l_part[b * a.QRT16 + row];
      const h4* hp = (const h4*)a.o_part + (b * QRT + t) * DT * 64 + threadIdx.x;
#pragma unroll
      for (int k = 0; k < EPT; ++k) hc[u][k] = hp[256 * k];
    }
#pragma unroll
    for (int u = 0; u < CB; ++u) {
      const float m = mc[u];
      if (m == -INFINITY) continue;
      if (m > M) {
        const float sc = exp2f(M - m);   // 0 while M is -inf
        L *= sc;
#pragma unroll
        for (int k = 0; k < EPT; ++k)
#pragma unroll
          for (int i = 0; i < 4; ++i) O[k][i] *= sc;
        M = m;
      }
      const float wl = lc[u] * exp2f(m - M);   // the record's sum, at the running reference
      L += wl;
#pragma unroll
      for (int k = 0; k < EPT; ++k)
#pragma unroll
        for (int i = 0; i < 4; ++i) O[k][i] += (float)hc[u][k][i] * wl;
    }
  }
  const float inv = 1.0f / L;
  const int gps = a.group / a.splits;
  const int gi = row / a.R, j = row % a.R;
  const int qh = kv * a.group + z * gps + gi;
  T* dst = (T*)a.out + ((int64_t)req * a.R + j) * a.q_dim + qh * D + 4 * (lane >> 4);
#pragma unroll
  for (int k = 0; k < EPT; ++k) {
    const int dt = (threadIdx.x >> 6) + 4 * k;
#pragma unroll
    for (int i = 0; i < 4; ++i) dst[dt * 16 + i] = from_f32<T>(O[k][i] * inv);
  }
}

// One work-group per (request, kv head and q-row part, block of 16 rows): each
// thread owns one row and D/16 consecutive head dims and merges the segment's
// chunk records in order in one pass (running max, earlier sums rescaled).
// fp32 K/V path (row-layout fp32 records of chunks).
template <typename T, int D>
__global__ __launch_bounds__(256) void attn_combine_kernel(const AttnCombineArgs a) {
  constexpr int EPT = D / 16;
  const int req = blockIdx.x;
  const int kv = blockIdx.y / a.splits, z = blockIdx.y % a.splits;
  const int row = blockIdx.z * 16 + (threadIdx.x >> 4);
  const int e0 = (threadIdx.x & 15) * EPT;
  if (row >= a.rows_per_split) return;
  const int seg = (req * a.n_kv + kv) * a.splits + z;
  const int len = a.seg_start[seg + 1] - a.seg_start[seg];
  int n;
  int64_t p0;
  {
    const int cg = attn_chunk_groups(len, a.chunk_min, a.chunk_max);
    n = (len + cg - 1) / cg;
    p0 = a.chunk_base[seg];
  }
  // one pass, four chunk records' loads issued together; the running max rescales what came before
  float M = -INFINITY, L = 0.f;
  float O[EPT];
#pragma unroll
  for (int i = 0; i < EPT; ++i) O[i] = 0.f;
  for (int c0 = 0; c0 < n; c0 += 4) {
    float mc[4], lc[4];
    float4 oc[4][EPT / 4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int64_t b = p0 + min(c0 + u, n - 1);
      mc[u] = c0 + u < n ? a.m_part[b * a.QRT16 + row] : -INFINITY;
      lc[u] = a.l_part[b * a.QRT16 + row];
      const float4* op = (const float4*)(a.o_part + (b * a.QRT16 + row) * D + e0);
#pragma unroll
      for (int i = 0; i < EPT / 4; ++i) oc[u][i] = op[i];
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const float m = mc[u];
      if (m == -INFINITY) continue;
      if (m > M) {
        const float sc = exp2f(M - m);   // 0 while M is -inf
        L *= sc;
#pragma unroll
        for (int i = 0; i < EPT; ++i) O[i] *= sc;
        M = m;
      }
      const float wgt = exp2f(m - M);
      L += lc[u] * wgt;
#pragma unroll
      for (int i = 0; i < EPT / 4; ++i) {
        O[4 * i] += oc[u][i].x * wgt;
        O[4 * i + 1] += oc[u][i].y * wgt;
        O[4 * i + 2] += oc[u][i].z * wgt;
        O[4 * i + 3] += oc[u][i].w * wgt;
      }
    }
  }
  const float inv = 1.0f / L;
  const int gps = a.group / a.splits;
  const int gi = row / a.R, j = row % a.R;
  const int qh = kv * a.group + z * gps + gi;
  T* dst = (T*)a.out + ((int64_t)req * a.R + j) * a.q_dim + qh * D + e0;
#pragma unroll
  for (int i = 0; i < EPT; ++i) dst[i] = from_f32<T>(O[i] * inv);
}

// ---------------------------------------------------------------------------
template <typename T, int D, bool PG>
static void launch_attn_t(const AttnArgs& a, int qrt, int grid, hipStream_t s) {
  constexpr int S = (sizeof(T) == 4 && D == 128) ? 4 : 5;  // LDS ring stages (16 or 32 KB each)
  switch (qrt) {
    case 1: attn_kernel<T, D, 1, S, PG><<<grid, 64, 0, s>>>(a); break;
    case 2: attn_kernel<T, D, 2, S, PG><<<grid, 128, 0, s>>>(a); break;
    case 3: attn_kernel<T, D, 3, S, PG><<<grid, 192, 0, s>>>(a); break;
    case 4: attn_kernel<T, D, 4, S, PG><<<grid, 256, 0, s>>>(a); break;
    case 5: attn_kernel<T, D, 5, S, PG><<<grid, 320, 0, s>>>(a); break;
  }
}

// Shape of the 16-bit streamed attention: waves per work-group, ring stages
// (one 16 KB group at head dim 128 each) and work-groups per CU.  Two waves,
// two stages, four work-groups: 128 KB of the CU's 160 KB of LDS, two waves per
// SIMD (at most 256 registers each).
#ifndef ATTN_WAVE_SHAPE
#define ATTN_WAVE_SHAPE 2, 2, 4
#endif
static constexpr int kWaveShape[3] = {ATTN_WAVE_SHAPE};
static constexpr int kWaveNW = kWaveShape[0], kWaveRing = kWaveShape[1], kWaveWgPerCu = kWaveShape[2];
int attn_waves_wg_per_cu() { return kWaveWgPerCu; }

template <int D, int QRT, bool PG>
static void launch_attn_wave_q(const AttnArgs& a, int grid, hipStream_t s) {
  // waves per work-group: a power of two (they share a group's fragments) holding at least a tile each
  constexpr int NWV = QRT >= kWaveNW ? kWaveNW : QRT >= 2 ? 2 : 1;
  constexpr int WPE = (NWV * kWaveWgPerCu + 3) / 4;
  attn_wave_kernel<f16_t, D, QRT, NWV, kWaveRing, WPE, PG><<<grid, NWV * 64, 0, s>>>(a);
}

template <int D, bool PG>
static void launch_attn_wave(const AttnArgs& a, int qrt, int grid, hipStream_t s) {
  switch (qrt) {
    case 1: launch_attn_wave_q<D, 1, PG>(a, grid, s); break;
    case 2: launch_attn_wave_q<D, 2, PG>(a, grid, s); break;
    case 3: launch_attn_wave_q<D, 3, PG>(a, grid, s); break;
    case 4: launch_attn_wave_q<D, 4, PG>(a, grid, s); break;
    case 5: launch_attn_wave_q<D, 5, PG>(a, grid, s); break;
  }
}

void launch_attn_waves(int D, int qrt, const AttnArgs& a, int grid, hipStream_t s) {
  const bool pg = a.page_table != nullptr;
  if (D == 128) pg ? launch_attn_wave<128, true>(a, qrt, grid, s) : launch_attn_wave<128, false>(a, qrt, grid, s);
  else pg ? launch_attn_wave<64, true>(a, qrt, grid, s) : launch_attn_wave<64, false>(a, qrt, grid, s);
}

void launch_attn_plan(const int32_t* slots, const int32_t* ctx_len, int n_req, int n_kv, int splits, int n_wg_max,
                      int min_per_wg, int chunk_min, int chunk_max, AttnPlan* plan, int32_t* seg_start,
                      int32_t* chunk_base, int4* seg_desc, int4* wg_range, hipStream_t s) {
  attn_plan_kernel<<<1, 256, 0, s>>>(slots, ctx_len, n_req, n_kv, splits, n_wg_max, min_per_wg, chunk_min, chunk_max,
                                      plan, seg_start, chunk_base, seg_desc, wg_range);
}

void launch_attn(int D, int qrt, const AttnArgs& a, int grid, hipStream_t s) {
  // fp32 K/V; the paged cache has instantiations of its own: its page cursor stays
  // out of the contiguous kernels
  const bool pg = a.page_table != nullptr;
  if (D == 128) pg ? launch_attn_t<float, 128, true>(a, qrt, grid, s) : launch_attn_t<float, 128, false>(a, qrt, grid, s);
  else pg ? launch_attn_t<float, 64, true>(a, qrt, grid, s) : launch_attn_t<float, 64, false>(a, qrt, grid, s);
}

void launch_attn_combine(int dtype, int D, const AttnCombineArgs& a, dim3 grid, hipStream_t s) {
  if (dtype == DT_BF16) {   // records of the 16-bit streamed attention
    if (D == 128) attn_combine_frag_kernel<f16_t, 128><<<grid, 256, 0, s>>>(a);
    else attn_combine_frag_kernel<f16_t, 64><<<grid, 256, 0, s>>>(a);
  } else {
    if (D == 128) attn_combine_kernel<float, 128><<<grid, 256, 0, s>>>(a);
    else attn_combine_kernel<float, 64><<<grid, 256, 0, s>>>(a);
  }
}

}  // namespace dfl
