// Block attention kernels: work plan, split-context attention, chunk combine.
#include "attention.h"
#include "ops.h"

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

template <typename T, int D, int QRT>
__global__ __launch_bounds__(256) void attn_kernel(const AttnArgs a) {
  constexpr int KSTEPS = D / 32, DT = D / 16, ROWS = QRT * 16;
  constexpr int CH = (int)sizeof(T) * D / 16;  // 16-byte chunks per q row
  constexpr int SW = (CH < 16 ? CH : 16) - 1;
  constexpr int OLD = D + 1;                   // padded row stride of the merge buffer
  typedef typename Frag<T>::type FragT;
  __shared__ uint4 q_lds[ROWS * CH];
  __shared__ float o_acc[ROWS * OLD];
  __shared__ float m_w[4][ROWS], l_w[4][ROWS];

  const int item = blockIdx.x, kv = blockIdx.y, z = blockIdx.z;
  if (item >= a.plan->count) return;
  const int4 it = a.items[item];
  const int req = it.x, kbeg = it.y, kend = it.z, is_last = it.w;
  const int slot = a.slots[req];
  const int ck = a.plan->ck;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int grp = lane >> 4, r16 = lane & 15;

  {
    const T* qsrc = (const T*)a.qb + ((int64_t)(req * a.n_kv + kv) * a.QRpad + (int64_t)z * a.rows_per_split) * D;
    for (int c = tid; c < ROWS * CH; c += 256) {
      const int row = c / CH, ch = c % CH;
      q_lds[row * CH + (ch ^ (row & SW))] = ((const uint4*)(qsrc + (int64_t)row * D))[ch];
    }
  }
  __syncthreads();

  f32x4 acc_o[DT][QRT];
  float m_row[QRT], l_row[QRT];
#pragma unroll
  for (int rt = 0; rt < QRT; ++rt) {
    m_row[rt] = -INFINITY;
    l_row[rt] = 0.f;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) acc_o[dt][rt] = f32x4{0.f, 0.f, 0.f, 0.f};
  }

  auto run = [&](const T* kbase, const T* vtbase, int64_t vstride, int s0, int s1) {
    for (int g0 = s0; g0 < s1; g0 += 32) {
      FragT kf[2][KSTEPS];
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        const int key = g0 + 8 * (r16 >> 2) + 4 * t + (r16 & 3);
        const T* kp = kbase + (int64_t)key * D + grp * 8;
#pragma unroll
        for (int s = 0; s < KSTEPS; ++s) {
          if (key < s1) kf[t][s] = load_frag8<T>(kp + s * 32);
          else kf[t][s] = FragT{};
        }
      }
      FragT vf[DT];
      const int kv0 = g0 + grp * 8;
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) {
        vf[dt] = load_frag8<T>(vtbase + (int64_t)(dt * 16 + r16) * vstride + kv0);
        if (kv0 + 8 > s1) {
#pragma unroll
          for (int e = 0; e < 8; ++e)
            if (kv0 + e >= s1) vf[dt][e] = (T)0.f;
        }
      }
      f32x4 sacc[2][QRT];
#pragma unroll
      for (int rt = 0; rt < QRT; ++rt) sacc[0][rt] = sacc[1][rt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int s = 0; s < KSTEPS; ++s) {
#pragma unroll
        for (int rt = 0; rt < QRT; ++rt) {
          const int row = rt * 16 + r16;
          FragT qf;
          if constexpr (sizeof(T) == 2) {
            const int ch = s * 4 + grp;
            *(uint4*)&qf = q_lds[row * CH + (ch ^ (row & SW))];
          } else {
            const int ch = s * 8 + grp * 2;
            ((uint4*)&qf)[0] = q_lds[row * CH + (ch ^ (row & SW))];
            ((uint4*)&qf)[1] = q_lds[row * CH + ((ch + 1) ^ (row & SW))];
          }
          Frag<T>::mma(sacc[0][rt], kf[0][s], qf);
          Frag<T>::mma(sacc[1][rt], kf[1][s], qf);
        }
      }
      FragT pf[QRT];
#pragma unroll
      for (int rt = 0; rt < QRT; ++rt) {
        float sv[8];
        float mx = -INFINITY;
#pragma unroll
        for (int t = 0; t < 2; ++t)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int key = g0 + 8 * grp + 4 * t + i;
            const float v = key < s1 ? sacc[t][rt][i] * a.scale_log2 : -INFINITY;
            sv[4 * t + i] = v;
            mx = fmaxf(mx, v);
          }
        mx = fmaxf(mx, __shfl_xor(mx, 16, 64));
        mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
        const float mnew = fmaxf(m_row[rt], mx);
        float alpha = 1.f, sum = 0.f;
        if (mnew != -INFINITY) {
          alpha = exp2f(m_row[rt] - mnew);
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            const float p = exp2f(sv[e] - mnew);
            sv[e] = p;
            sum += p;
          }
        } else {
#pragma unroll
          for (int e = 0; e < 8; ++e) sv[e] = 0.f;
        }
        l_row[rt] = l_row[rt] * alpha + sum;
        m_row[rt] = mnew;
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) acc_o[dt][rt] *= alpha;
#pragma unroll
        for (int e = 0; e < 8; ++e) pf[rt][e] = (T)sv[e];
      }
#pragma unroll
      for (int dt = 0; dt < DT; ++dt)
#pragma unroll
        for (int rt = 0; rt < QRT; ++rt) Frag<T>::mma(acc_o[dt][rt], vf[dt], pf[rt]);
    }
  };

  const int quarter = ck / 4;
  {
    const int wb = kbeg + wave * quarter;
    const int we = min(kend, wb + quarter);
    if (wb < we) {
      const int64_t head = (int64_t)slot * a.n_kv + kv;
      const T* kbase = (const T*)a.cache_k + head * a.ctx_alloc * D;
      const T* vtbase = (const T*)a.cache_vt + head * D * a.ctx_alloc;
      // keys are addressed relative to the segment start so 32-key groups stay aligned
      run(kbase + (int64_t)wb * D, vtbase + wb, a.ctx_alloc, 0, we - wb);
    }
    if (is_last && wave == 3) {
      const int64_t bh = (int64_t)req * a.n_kv + kv;
      run((const T*)a.kb + bh * a.Rpad * D, (const T*)a.vbt + bh * D * a.Rpad, a.Rpad, 0, a.R);
    }
  }

#pragma unroll
  for (int rt = 0; rt < QRT; ++rt) {
    l_row[rt] += __shfl_xor(l_row[rt], 16, 64);
    l_row[rt] += __shfl_xor(l_row[rt], 32, 64);
    if (grp == 0) {
      m_w[wave][rt * 16 + r16] = m_row[rt];
      l_w[wave][rt * 16 + r16] = l_row[rt];
    }
  }
  __syncthreads();
  float sc[QRT];
#pragma unroll
  for (int rt = 0; rt < QRT; ++rt) {
    const int row = rt * 16 + r16;
    const float M = fmaxf(fmaxf(m_w[0][row], m_w[1][row]), fmaxf(m_w[2][row], m_w[3][row]));
    sc[rt] = (m_row[rt] == -INFINITY) ? 0.f : exp2f(m_row[rt] - M);
  }
  for (int w = 0; w < 4; ++w) {
    if (wave == w) {
#pragma unroll
      for (int dt = 0; dt < DT; ++dt)
#pragma unroll
        for (int rt = 0; rt < QRT; ++rt)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int idx = (rt * 16 + r16) * OLD + dt * 16 + 4 * grp + i;
            const float v = acc_o[dt][rt][i] * sc[rt];
            o_acc[idx] = (w == 0) ? v : o_acc[idx] + v;
          }
    }
    __syncthreads();
  }
  const int64_t base = ((int64_t)item * a.n_kv + kv) * a.splits + z;
  float* op = a.o_part + base * ROWS * D;
  for (int idx = tid; idx < ROWS * D; idx += 256) op[idx] = o_acc[(idx / D) * OLD + (idx % D)];
  for (int row = tid; row < ROWS; row += 256) {
    float M = -INFINITY;
    for (int w = 0; w < 4; ++w) M = fmaxf(M, m_w[w][row]);
    float L = 0.f;
    for (int w = 0; w < 4; ++w)
      if (m_w[w][row] != -INFINITY) L += l_w[w][row] * exp2f(m_w[w][row] - M);
    a.m_part[base * ROWS + row] = M;
    a.l_part[base * ROWS + row] = L;
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
  switch (qrt) {
    case 1: attn_kernel<T, D, 1><<<grid, 256, 0, s>>>(a); break;
    case 2: attn_kernel<T, D, 2><<<grid, 256, 0, s>>>(a); break;
    case 3: attn_kernel<T, D, 3><<<grid, 256, 0, s>>>(a); break;
    case 4:
      if constexpr (sizeof(T) == 2 || D == 64) attn_kernel<T, D, 4><<<grid, 256, 0, s>>>(a);
      break;
    case 5:
      if constexpr (sizeof(T) == 2 || D == 64) attn_kernel<T, D, 5><<<grid, 256, 0, s>>>(a);
      break;
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
