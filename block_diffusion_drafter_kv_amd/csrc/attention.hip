// Block attention kernels: work plan, split-context attention, chunk combine.
#include "attention.h"
#include "ops.h"
#include "lds_dma.h"

namespace dfl {

// ---------------------------------------------------------------------------
// Plan: choose the chunk size from the real context lengths and list the work
// items (request, first key, end key, last-chunk flag).  One work-group.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void attn_plan_kernel(const int32_t* slots, const int32_t* ctx_len, int n_req,
                                                         int n_kv, int splits, int target_wg, int item_cap,
                                                         AttnPlan* plan, int4* items, int32_t* first_item,
                                                         int32_t* n_items, int32_t* err) {
  __shared__ long long s_total;
  __shared__ int s_ck;
  if (threadIdx.x == 0) s_total = 0;
  __syncthreads();
  long long part = 0;
  for (int r = threadIdx.x; r < n_req; r += blockDim.x) part += ctx_len[slots[r]];
  atomicAdd((unsigned long long*)&s_total, (unsigned long long)part);
  __syncthreads();
  if (threadIdx.x == 0) {
    long long want = (s_total * n_kv * splits + target_wg - 1) / target_wg;
    long long ck = ((want + 127) / 128) * 128;
    if (ck < 256) ck = 256;
    s_ck = (int)ck;
    int pos = 0;
    for (int r = 0; r < n_req; ++r) {
      const int C = ctx_len[slots[r]];
      const int n = C > 0 ? (C + (int)ck - 1) / (int)ck : 1;
      first_item[r] = pos;
      n_items[r] = n;
      pos += n;
    }
    if (pos > item_cap) {  // cannot happen with the host-side capacity; keep the grid safe
      raise_error(err, ERR_ROWS);
      pos = item_cap;
    }
    plan->count = pos;
    plan->ck = (int)ck;
  }
  __syncthreads();
  const int ck = s_ck;
  for (int r = threadIdx.x; r < n_req; r += blockDim.x) {
    const int C = ctx_len[slots[r]];
    const int f = first_item[r], n = n_items[r];
    for (int c = 0; c < n; ++c) {
      if (f + c >= item_cap) break;
      items[f + c] = make_int4(r, c * ck, min(C, (c + 1) * ck), c == n - 1 ? 1 : 0);
    }
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

// One work-group = (work item, kv head, q-row part) with one wave per 16-row
// query tile.  The item's keys [kbeg, kend) (and, for a request's last item, the
// block's own R keys) are streamed in 32-key groups through a ring of S LDS
// stages by direct global->LDS copies; every wave reads each group from LDS and
// runs its own online softmax over all of the item's keys, so no cross-wave
// merge is needed.  Per group: S^T (32 x 16) = K Q^T, scale, mask, softmax
// update, O^T += V^T P^T.  Copies run S - 1 groups ahead; a group is published
// by the copying waves' vmcnt wait plus a barrier, which also retires the stage
// that the next copy overwrites.
//
// The running maximum is raised lazily: probabilities are taken relative to a
// reference m_ref, which only moves (rescaling O and l) when a score exceeds it
// by more than 2^8 in the exp2 domain; the result is unchanged up to rounding
// (bf16 rounding of P is relative, and P <= 256 stays far from overflow).
template <typename T, int D, int QRT, int S>
__global__ __launch_bounds__(QRT * 64) void attn_kernel(const AttnArgs a) {
  constexpr int KS = D / 32, DT = D / 16;
  constexpr int BLK = KV_BLOCK * D;                        // elements of a K (or V) block
  constexpr int EPC = 16 / (int)sizeof(T);                 // elements per 16-byte copy
  constexpr int IPG = 2 * BLK / (64 * EPC);                // 1 KB wave copies per group (K, then V)
  constexpr int CW = QRT >= 4 ? 4 : (QRT >= 2 ? 2 : 1);    // waves that issue copies
  constexpr int PER = IPG / CW;                            // copies per copying wave per group
  constexpr int VOFF = IPG / 2 * 64;                       // first uint4 of the V block in a stage
  constexpr float TAU = 8.f;                               // lazy-rescale threshold (log2 units)
  static_assert(IPG % CW == 0 && (S - 2) * PER < 64 && S >= 2 && S <= 4, "copy split / vmcnt range");
  typedef typename Frag<T>::type FragT;
  __shared__ uint4 ring[S][IPG * 64];

  const int item = blockIdx.x, kv = blockIdx.y, z = blockIdx.z;
  if (item >= a.plan->count) return;
  const int4 it = a.items[item];
  const int req = it.x, kbeg = it.y, kend = it.z, is_last = it.w;
  const int slot = a.slots[req];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int grp = lane >> 4, r16 = lane & 15;

  // this wave's 16 query rows as B-operand fragments (row r16, dims 32 s + 8 grp ..)
  FragT qf[KS];
  {
    const T* qrow = (const T*)a.qb +
                    ((int64_t)(req * a.n_kv + kv) * a.QRpad + (int64_t)z * a.rows_per_split + wave * 16 + r16) * D;
#pragma unroll
    for (int s = 0; s < KS; ++s) qf[s] = load_frag8<T>(qrow + s * 32 + grp * 8);
  }
  wait_vmcnt<0>();

  const int ncache = (kend - kbeg + KV_BLOCK - 1) / KV_BLOCK;
  const int ng = ncache + (is_last ? 1 : 0);
  const int64_t head = (int64_t)slot * a.n_kv + kv;
  const T* kc = (const T*)a.cache_k + head * a.ctx_alloc * D + (int64_t)kbeg * D;
  const T* vc = (const T*)a.cache_v + head * a.ctx_alloc * D + (int64_t)kbeg * D;
  const int64_t bh = (int64_t)req * a.n_kv + kv;
  const T* kblk = (const T*)a.kb + bh * a.Rpad * D;
  const T* vblk = (const T*)a.vb + bh * a.Rpad * D;

  auto issue = [&](int gi, int st) {
    if (wave < CW) {
      const bool in_cache = gi < ncache;
      const T* kp = (in_cache ? kc + (int64_t)gi * BLK : kblk) + lane * EPC;
      const T* vp = (in_cache ? vc + (int64_t)gi * BLK : vblk) + lane * EPC;
#pragma unroll
      for (int c = 0; c < PER; ++c) {
        const int i = wave * PER + c;
        const T* src = i < IPG / 2 ? kp + i * 64 * EPC : vp + (i - IPG / 2) * 64 * EPC;
        copy16_to_lds(src, &ring[st][i * 64]);
      }
    }
  };

  f32x4 acc[DT];
#pragma unroll
  for (int dt = 0; dt < DT; ++dt) acc[dt] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m_ref = -INFINITY, l_sum = 0.f;

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

  auto compute = [&](const uint4* stage, int gi) {
    const int nvalid = gi < ncache ? min(KV_BLOCK, kend - kbeg - KV_BLOCK * gi) : a.R;
    f32x4 s0 = {0.f, 0.f, 0.f, 0.f}, s1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      Frag<T>::mma(s0, frag_at(stage, s), qf[s]);
      Frag<T>::mma(s1, frag_at(stage, KS + s), qf[s]);
    }
    // lane holds keys 8*grp + i (s0) and 8*grp + 4 + i (s1) of this group for query row r16
    float sv[8];
    float mx = -INFINITY;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int k0 = 8 * grp + i;
      sv[i] = k0 < nvalid ? s0[i] * a.scale_log2 : -INFINITY;
      sv[4 + i] = k0 + 4 < nvalid ? s1[i] * a.scale_log2 : -INFINITY;
      mx = fmaxf(mx, fmaxf(sv[i], sv[4 + i]));
    }
    mx = fmaxf(mx, __shfl_xor(mx, 16, 64));
    mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
    if (__any(mx > m_ref + TAU)) {
      const float mnew = fmaxf(m_ref, mx);
      const float alpha = mnew > m_ref ? exp2f(m_ref - mnew) : 1.f;
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) acc[dt] *= alpha;
      l_sum *= alpha;
      m_ref = mnew;
    }
    FragT pf;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float p = exp2f(sv[e] - m_ref);
      l_sum += p;
      pf[e] = (T)p;
    }
    const uint4* vst = stage + VOFF;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) {
      FragT vf = frag_at(vst, dt);
      if (nvalid < KV_BLOCK) {  // keys past the end hold stale or unwritten data
#pragma unroll
        for (int e = 0; e < 8; ++e)
          if (grp * 8 + e >= nvalid) vf[e] = (T)0.f;
      }
      Frag<T>::mma(acc[dt], vf, pf);
    }
  };

  for (int p = 0; p < S - 1 && p < ng; ++p) issue(p, p);
  for (int gi = 0; gi < ng; ++gi) {
    if (wave < CW) {
      const int ahead = min(S - 2, ng - 1 - gi);  // groups issued after gi that may stay in flight
      if (S >= 4 && ahead >= 2) wait_vmcnt<(S >= 4 ? 2 * PER : 0)>();
      else if (S >= 3 && ahead >= 1) wait_vmcnt<(S >= 3 ? PER : 0)>();
      else wait_vmcnt<0>();
    }
    lds_barrier();
    if (gi + S - 1 < ng) issue(gi + S - 1, (gi + S - 1) % S);
    compute(ring[gi % S], gi);
  }

  // partial result of this item: O (unnormalised, relative to m_ref), m_ref, l
  l_sum += __shfl_xor(l_sum, 16, 64);
  l_sum += __shfl_xor(l_sum, 32, 64);
  const int row = wave * 16 + r16;
  const int64_t base = ((int64_t)item * a.n_kv + kv) * a.splits + z;
  float* op = a.o_part + (base * (QRT * 16) + row) * D + 4 * grp;
#pragma unroll
  for (int dt = 0; dt < DT; ++dt) *(f32x4*)(op + dt * 16) = acc[dt];
  if (grp == 0) {
    a.m_part[base * (QRT * 16) + row] = m_ref;
    a.l_part[base * (QRT * 16) + row] = l_sum;
  }
}

// One work-group per (request, kv head and q-row half, block of 16 rows): each
// thread owns one row and D/16 consecutive head dims and merges the request's
// chunks in chunk order (max first, then the rescaled sums).
template <typename T, int D>
__global__ __launch_bounds__(256) void attn_combine_kernel(const AttnCombineArgs a) {
  constexpr int EPT = D / 16;
  const int req = blockIdx.x;
  const int kv = blockIdx.y / a.splits, z = blockIdx.y % a.splits;
  const int row = blockIdx.z * 16 + (threadIdx.x >> 4);
  const int e0 = (threadIdx.x & 15) * EPT;
  if (row >= a.rows_per_split) return;
  const int f = a.first_item[req], n = a.n_items[req];
  const int64_t stride_item = (int64_t)a.n_kv * a.splits;         // partial blocks per item
  const int64_t b0 = ((int64_t)f * a.n_kv + kv) * a.splits + z;
  float M = -INFINITY;
  for (int c = 0; c < n; ++c) M = fmaxf(M, a.m_part[(b0 + c * stride_item) * a.QRT16 + row]);
  float L = 0.f;
  float O[EPT];
#pragma unroll
  for (int i = 0; i < EPT; ++i) O[i] = 0.f;
  for (int c = 0; c < n; ++c) {
    const int64_t b = b0 + c * stride_item;
    const float m = a.m_part[b * a.QRT16 + row];
    if (m == -INFINITY) continue;
    const float w = exp2f(m - M);
    L += a.l_part[b * a.QRT16 + row] * w;
    const float4* op = (const float4*)(a.o_part + (b * a.QRT16 + row) * D + e0);
#pragma unroll
    for (int i = 0; i < EPT / 4; ++i) {
      const float4 v = op[i];
      O[4 * i] += v.x * w;
      O[4 * i + 1] += v.y * w;
      O[4 * i + 2] += v.z * w;
      O[4 * i + 3] += v.w * w;
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
template <typename T, int D>
static void launch_attn_t(const AttnArgs& a, int qrt, dim3 grid, hipStream_t s) {
  constexpr int S = (sizeof(T) == 4 && D == 128) ? 3 : 4;  // LDS ring stages (16 or 32 KB each)
  switch (qrt) {
    case 1: attn_kernel<T, D, 1, S><<<grid, 64, 0, s>>>(a); break;
    case 2: attn_kernel<T, D, 2, S><<<grid, 128, 0, s>>>(a); break;
    case 3: attn_kernel<T, D, 3, S><<<grid, 192, 0, s>>>(a); break;
    case 4: attn_kernel<T, D, 4, S><<<grid, 256, 0, s>>>(a); break;
    case 5: attn_kernel<T, D, 5, S><<<grid, 320, 0, s>>>(a); break;
  }
}

void launch_attn_plan(const int32_t* slots, const int32_t* ctx_len, int n_req, int n_kv, int splits, int target_wg,
                      int item_cap, AttnPlan* plan, int4* items, int32_t* first_item, int32_t* n_items, int32_t* err,
                      hipStream_t s) {
  attn_plan_kernel<<<1, 256, 0, s>>>(slots, ctx_len, n_req, n_kv, splits, target_wg, item_cap, plan, items,
                                      first_item, n_items, err);
}

void launch_attn(int dtype, int D, int qrt, const AttnArgs& a, dim3 grid, hipStream_t s) {
  if (dtype == DT_BF16) {
    if (D == 128) launch_attn_t<bf16_t, 128>(a, qrt, grid, s);
    else launch_attn_t<bf16_t, 64>(a, qrt, grid, s);
  } else {
    if (D == 128) launch_attn_t<float, 128>(a, qrt, grid, s);
    else launch_attn_t<float, 64>(a, qrt, grid, s);
  }
}

void launch_attn_combine(int dtype, int D, const AttnCombineArgs& a, dim3 grid, hipStream_t s) {
  if (dtype == DT_BF16) {
    if (D == 128) attn_combine_kernel<bf16_t, 128><<<grid, 256, 0, s>>>(a);
    else attn_combine_kernel<bf16_t, 64><<<grid, 256, 0, s>>>(a);
  } else {
    if (D == 128) attn_combine_kernel<float, 128><<<grid, 256, 0, s>>>(a);
    else attn_combine_kernel<float, 64><<<grid, 256, 0, s>>>(a);
  }
}

}  // namespace dfl
