// MFMA GEMM  C[M, N] = A[M, K] . B[N, K]^T  with fp32 accumulation and a fused,
// LDS-staged epilogue.
//
// Both operands are K-contiguous (row-major activations, row-major
// [out_features, in_features] weights), which is exactly the MFMA operand
// layout: every lane loads 16-byte runs along K.  256 threads = 4 waves in a
// 2 x 2 arrangement; each wave owns a (BM/2) x (BN/2) sub-tile made of 16 x 16
// MFMA tiles.  K advances in 128-byte slabs (64 bf16 or 32 fp32 per row),
// double-buffered in LDS with an XOR swizzle of the 16-byte chunks so that
// fragment reads are conflict-free.
//
// Operand addressing supports what the drafter needs without copies:
//  * A may be a virtual concatenation along K of several buffers (the target
//    layers' hidden states feeding the fc projection) and may gather rows;
//  * B may be a virtual concatenation along N of several weight matrices
//    (q|k|v, the 2 x L per-layer k|v of the injection, gate/up interleaved in
//    blocks of BN/2 so that one tile holds matching gate and up columns).
// Split-K writes fp32 partial tiles; gemm_reduce_kernel sums them in a fixed
// order (deterministic) and runs the same epilogue.
#pragma once
#include "common.h"

namespace dfl {

static constexpr int MAX_ASEG = 8;
static constexpr int MAX_BSEG = 16;

struct GemmArgs {
  int M, N, K;
  const void* a_ptr[MAX_ASEG];
  int64_t a_ld[MAX_ASEG];       // the bf16 kernel requires one stride for all segments (a_ld[0])
  int a_nseg, a_segk;          // K = a_nseg * a_segk; segment s covers k in [s*a_segk, (s+1)*a_segk)
  const int32_t* a_rows;       // optional gather: source row for output row m (<0: zero row)
  const int32_t* m_valid;      // optional device row count: tiles at or past (*m_valid - m_valid_base) exit
  int m_valid_base;
  const void* b_ptr[MAX_BSEG];
  int b_begin[MAX_BSEG + 1];   // virtual row ranges of the B segments
  int b_nseg;
  int64_t b_ld;
  int b_interleave;            // 1: tile t's rows [0,BN/2) = gate rows t*BN/2.., [BN/2,BN) = up rows
  int a_wide;                  // 1: A rows need 64-bit byte offsets (caller buffers of 4 GiB or more)
  float out_scale;             // products are multiplied by this (a power of two undoing the weight scale)
  int splits;
  int k_per_split;             // multiple of the K slab
  float* partials;             // [splits][Mpad][Npad]
  int keep_partials;           // 1: a split product leaves its partial tiles to the consumer (no reduce pass)
  int Mpad, Npad;
  int tiles_m, tiles_n;
};

// XOR swizzles of the eight 16-byte chunks of a 128-byte LDS row: chunk c of
// row r is stored at slot c ^ swz(r).  Which lanes of a 16-byte LDS read share a
// cycle was measured on gfx950 (bank-conflict counter over a probe of each lane
// pattern), not assumed.  For the 32 x 32 x 16 fragments of gemm256.h (lane l:
// row l % 32, chunk l / 32), swz = (row & 7) ^ ((row >> 3) & 1) is conflict-free
// and plain row & 7 doubles the LDS cycles; for the 16 x 16 x 32 fragments of
// gemm2.h (row l % 16, chunk l / 16) it is the other way round, so gemm2.h
// stores with swz16 = row & 7.
__host__ __device__ __forceinline__ int swz(int row) { return (row & 7) ^ ((row >> 3) & 1); }
__host__ __device__ __forceinline__ int swz16(int row) { return row & 7; }

template <typename T> struct GemmTraits;
template <> struct GemmTraits<bf16_t> { static constexpr int BK = 64; static constexpr int VEC = 8; };
template <> struct GemmTraits<f16_t> { static constexpr int BK = 64; static constexpr int VEC = 8; };
template <> struct GemmTraits<float> { static constexpr int BK = 32; static constexpr int VEC = 4; };

// Grid of a tiled product: rounded up to a multiple of the 8 XCDs so that the
// remap below applies (work-groups past the tile count exit at once).
__host__ __device__ __forceinline__ int gemm_grid(int tiles) { return (tiles + 7) & ~7; }

__device__ __forceinline__ int xcd_remap(int b, int G) {
  // consecutive logical tiles land on the same XCD (8 XCDs, round-robin dispatch),
  // so the row tiles that share a weight tile share that XCD's L2
  if ((G & 7) != 0) return b;
  return (b & 7) * (G >> 3) + (b >> 3);
}

template <typename T, int BN>
__device__ __forceinline__ const T* b_row_ptr(const GemmArgs& g, int n) {
  if (n >= g.N) return nullptr;
  if (g.b_interleave) {
    const int half = BN / 2;
    const int t = n / BN, w = n % BN;
    const T* base = (const T*)(w < half ? g.b_ptr[0] : g.b_ptr[1]);
    return base + (int64_t)(t * half + (w % half)) * g.b_ld;
  }
  int s = 0;
#pragma unroll 1
  while (s + 1 < g.b_nseg && n >= g.b_begin[s + 1]) ++s;
  return (const T*)g.b_ptr[s] + (int64_t)(n - g.b_begin[s]) * g.b_ld;
}

// Stage accumulators of rows [pass*ROWS, (pass+1)*ROWS) of the tile into LDS (fp32, row stride BN+1),
// multiplied by the product's output scale (a power of two: exact).
template <int BM, int BN, int ROWS = EPI_ROWS>
__device__ __forceinline__ void stage_acc(float* stage, const f32x4 (&acc)[BM / 32][BN / 32], int wm, int wn,
                                          int lane, int pass, float scale) {
  constexpr int WM = BM / 2, WN = BN / 2, FM = WM / 16, FN = WN / 16;
  constexpr int LD = BN + 1;
  const int g = lane >> 4, r16 = lane & 15;
#pragma unroll
  for (int fi = 0; fi < FM; ++fi) {
    const int row0 = wm * WM + fi * 16;
    if (row0 < pass * ROWS || row0 >= (pass + 1) * ROWS) continue;
#pragma unroll
    for (int fj = 0; fj < FN; ++fj) {
      const int col = wn * WN + fj * 16 + r16;
#pragma unroll
      for (int i = 0; i < 4; ++i) stage[(row0 - pass * ROWS + g * 4 + i) * LD + col] = acc[fi][fj][i] * scale;
    }
  }
}

template <typename T, int BM, int BN, class Epi>
__global__ __launch_bounds__(256) void gemm_kernel(const GemmArgs g, const typename Epi::Params ep) {
  constexpr int BK = GemmTraits<T>::BK, VEC = GemmTraits<T>::VEC;
  constexpr int WM = BM / 2, WN = BN / 2, FM = WM / 16, FN = WN / 16;
  constexpr int KSTEPS = BK / 32;
  constexpr int AL = BM / 32, BL = BN / 32;  // 16-byte loads per thread per slab
  typedef typename Vec16<T>::type V16;
  typedef typename Frag<T>::type FragT;

  __shared__ uint4 smem[2][(BM + BN) * 8];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave & 1, wn = wave >> 1;
  const int logical = xcd_remap(blockIdx.x, gridDim.x);
  if (logical >= g.tiles_m * g.tiles_n) return;
  const int tm = logical % g.tiles_m, tn = logical / g.tiles_m;
  const int split = blockIdx.y;
  const int m_base = tm * BM, n_base = tn * BN;
  if (g.m_valid && m_base >= *g.m_valid - g.m_valid_base) return;
  const int k_begin = split * g.k_per_split;
  const int k_end = min(g.K, k_begin + g.k_per_split);
  const int nk = (k_end - k_begin) / BK;

  // per-thread load rows
  const int lchunk = tid & 7, lrow = tid >> 3;
  int64_t a_src[AL];
  bool a_ok[AL];
#pragma unroll
  for (int p = 0; p < AL; ++p) {
    const int m = m_base + lrow + 32 * p;
    int64_t src = m;
    bool ok = m < g.M;
    if (ok && g.a_rows) {
      const int s = g.a_rows[m];
      ok = s >= 0;
      src = s;
    }
    a_src[p] = src;
    a_ok[p] = ok;
  }
  const T* b_src[BL];
#pragma unroll
  for (int p = 0; p < BL; ++p) b_src[p] = b_row_ptr<T, BN>(g, n_base + lrow + 32 * p);

  V16 ra[AL], rb[BL];
  auto load_slab = [&](int k0) {
    const int seg = k0 / g.a_segk;
    const T* abase = (const T*)g.a_ptr[seg];
    const int64_t ald = g.a_ld[seg];
    const int kk = k0 - seg * g.a_segk + lchunk * VEC;
#pragma unroll
    for (int p = 0; p < AL; ++p) {
      if (a_ok[p]) ra[p] = *(const V16*)(abase + a_src[p] * ald + kk);
      else ra[p] = V16{};
    }
#pragma unroll
    for (int p = 0; p < BL; ++p) {
      if (b_src[p]) rb[p] = *(const V16*)(b_src[p] + k0 + lchunk * VEC);
      else rb[p] = V16{};
    }
  };
  auto store_slab = [&](int buf) {
#pragma unroll
    for (int p = 0; p < AL; ++p) {
      const int row = lrow + 32 * p;
      smem[buf][row * 8 + (lchunk ^ swz(row))] = *(const uint4*)&ra[p];
    }
#pragma unroll
    for (int p = 0; p < BL; ++p) {
      const int row = lrow + 32 * p;
      smem[buf][(BM + row) * 8 + (lchunk ^ swz(row))] = *(const uint4*)&rb[p];
    }
  };

  f32x4 acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  const int grp = lane >> 4, r16 = lane & 15;
  if (nk > 0) {
    load_slab(k_begin);
    store_slab(0);
  }
  __syncthreads();
  for (int kt = 0; kt < nk; ++kt) {
    const int cur = kt & 1;
    if (kt + 1 < nk) load_slab(k_begin + (kt + 1) * BK);
#pragma unroll
    for (int s = 0; s < KSTEPS; ++s) {
      FragT af[FM], bfr[FN];
#pragma unroll
      for (int fi = 0; fi < FM; ++fi) {
        const int row = wm * WM + fi * 16 + r16;
        if constexpr (VEC == 8) {
          const int c = s * 4 + grp;
          *(uint4*)&af[fi] = smem[cur][row * 8 + (c ^ swz(row))];
        } else {
          const int c = 2 * grp;
          ((uint4*)&af[fi])[0] = smem[cur][row * 8 + (c ^ swz(row))];
          ((uint4*)&af[fi])[1] = smem[cur][row * 8 + ((c + 1) ^ swz(row))];
        }
      }
#pragma unroll
      for (int fj = 0; fj < FN; ++fj) {
        const int row = BM + wn * WN + fj * 16 + r16;
        const int rr = wn * WN + fj * 16 + r16;
        if constexpr (VEC == 8) {
          const int c = s * 4 + grp;
          *(uint4*)&bfr[fj] = smem[cur][row * 8 + (c ^ swz(rr))];
        } else {
          const int c = 2 * grp;
          ((uint4*)&bfr[fj])[0] = smem[cur][row * 8 + (c ^ swz(rr))];
          ((uint4*)&bfr[fj])[1] = smem[cur][row * 8 + ((c + 1) ^ swz(rr))];
        }
      }
#pragma unroll
      for (int fi = 0; fi < FM; ++fi)
#pragma unroll
        for (int fj = 0; fj < FN; ++fj) Frag<T>::mma(acc[fi][fj], af[fi], bfr[fj]);
    }
    if (kt + 1 < nk) store_slab(cur ^ 1);
    __syncthreads();
  }

  if (g.splits > 1) {
    float* P = g.partials + (int64_t)split * g.Mpad * g.Npad;
#pragma unroll
    for (int fi = 0; fi < FM; ++fi)
#pragma unroll
      for (int fj = 0; fj < FN; ++fj) {
        const int col = n_base + wn * WN + fj * 16 + r16;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int row = m_base + wm * WM + fi * 16 + grp * 4 + i;
          P[(int64_t)row * g.Npad + col] = acc[fi][fj][i];
        }
      }
    return;
  }

  float* stage = (float*)&smem[0][0];
#pragma unroll
  for (int pass = 0; pass < BM / EPI_ROWS; ++pass) {
    if (m_base + pass * EPI_ROWS >= g.M) break;
    stage_acc<BM, BN>(stage, acc, wm, wn, lane, pass, g.out_scale);
    __syncthreads();
    Epi::template apply<BN, EPI_ROWS>(ep, stage, BN + 1, m_base + pass * EPI_ROWS, n_base, g.M, g.N, tn, tid);
    __syncthreads();
  }
}

// Sum split-K partials in split order and run the epilogue on one 64-row pass of
// a tile: work-group (tile, pass) = (blockIdx.x, blockIdx.y), so the reduction
// of a small grid still spreads over many CUs.
template <int BM, int BN, class Epi>
__global__ __launch_bounds__(256) void gemm_reduce_kernel(const GemmArgs g, const typename Epi::Params ep) {
  __shared__ float stage[EPI_ROWS * (BN + 1)];
  const int tid = threadIdx.x;
  const int logical = blockIdx.x;
  const int tm = logical % g.tiles_m, tn = logical / g.tiles_m;
  const int m_base = tm * BM, n_base = tn * BN;
  if (g.m_valid && m_base >= *g.m_valid - g.m_valid_base) return;
  const int m0 = m_base + blockIdx.y * EPI_ROWS;
  // rows of this tile (BM need not be a multiple of EPI_ROWS), cut at the device
  // row count when there is one (rows past it are neither summed nor passed on)
  int m_lim = min(g.M, m_base + BM);
  if (g.m_valid) m_lim = min(m_lim, *g.m_valid - g.m_valid_base);
  if (m0 >= m_lim) return;
  // 16-byte loads, two splits in flight at once; sums taken in split order
  constexpr int C4 = BN / 4, NV = EPI_ROWS * C4 / 256;
  static_assert(EPI_ROWS * C4 % 256 == 0, "reduce tiling");
  const int64_t split_stride = (int64_t)g.Mpad * g.Npad;
  float4 acc[NV];
#pragma unroll
  for (int j = 0; j < NV; ++j) acc[j] = make_float4(0.f, 0.f, 0.f, 0.f);
  auto load = [&](int sp, float4 (&v)[NV]) {
#pragma unroll
    for (int j = 0; j < NV; ++j) {
      const int idx = tid + j * 256, r = idx / C4, c4 = idx % C4;
      v[j] = m0 + r < m_lim ? *(const float4*)(g.partials + sp * split_stride + (int64_t)(m0 + r) * g.Npad + n_base + 4 * c4)
                          : make_float4(0.f, 0.f, 0.f, 0.f);
    }
  };
  auto add = [&](const float4 (&v)[NV]) {
#pragma unroll
    for (int j = 0; j < NV; ++j) {
      acc[j].x += v[j].x;
      acc[j].y += v[j].y;
      acc[j].z += v[j].z;
      acc[j].w += v[j].w;
    }
  };
  int sp = 0;
  for (; sp + 1 < g.splits; sp += 2) {
    float4 v0[NV], v1[NV];
    load(sp, v0);
    load(sp + 1, v1);
    add(v0);
    add(v1);
  }
  if (sp < g.splits) {
    float4 v0[NV];
    load(sp, v0);
    add(v0);
  }
#pragma unroll
  for (int j = 0; j < NV; ++j) {
    const int idx = tid + j * 256, r = idx / C4, c4 = idx % C4;
    float* d = stage + r * (BN + 1) + 4 * c4;
    d[0] = acc[j].x * g.out_scale;
    d[1] = acc[j].y * g.out_scale;
    d[2] = acc[j].z * g.out_scale;
    d[3] = acc[j].w * g.out_scale;
  }
  __syncthreads();
  Epi::template apply<BN, EPI_ROWS>(ep, stage, BN + 1, m0, n_base, m_lim, g.N, tn, tid);
}

// grid of the reduction of a BM-row tiling: one block per EPI_ROWS rows of every tile
template <int BM>
__host__ __forceinline__ dim3 reduce_grid(const GemmArgs& g) {
  return dim3(g.tiles_m * g.tiles_n, (BM + EPI_ROWS - 1) / EPI_ROWS);
}

}  // namespace dfl
