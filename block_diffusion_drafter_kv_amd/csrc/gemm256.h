// Large-tile 16-bit (fp16 or bf16 operands) MFMA GEMM for gfx950, for products
// with many rows (the injection's fc and K|V products) and the vocabulary
// product:  C[M, N] = A[M, K] . B[N, K]^T, fp32 accumulation.
//
// Shape.  A work-group of 8 waves (2 along M x 4 along N) owns a 256 x 256
// output tile, one work-group per CU; each wave owns 128 x 64 outputs as 4 x 2
// blocks of v_mfma_f32_32x32x16.  Per 16-wide k step a wave reads 6 fragments
// (6 KB) from LDS for 8 MFMAs, i.e. 43 flops per LDS byte; the work-group
// streams 64 KB of operands per 64-wide K slab for 8.4 MFLOP.
//
// Pipeline.  Two LDS stages of one 64-wide K slab each (A rows then B rows, 128
// bytes per row, 16-byte chunk c of row r at slot c ^ swz(r)).  During slab kt
// every thread issues its copies of slab kt+1 into the other stage (16-byte
// global_load_lds, four per k step, in the first two steps) and the fragments of
// k step s+1 are read while the MFMAs of step s run.  In the last step half the
// MFMAs are issued, then the wait for slab kt+1's copies and the barrier that
// publishes it, then the first fragments of slab kt+1 are read while the other
// half runs: the LDS latency after the barrier hides behind MFMAs.
//
// MFMA v_mfma_f32_32x32x16: lane l supplies row (l % 32) of A and column
// (l % 32) of B with k-values 8*(l/32) .. +7; result element i of lane l is row
// 8*(i/4) + 4*(l/32) + (i%4), column l % 32.
//
// Tile order: GM tile-rows per group with the column index running inside a
// group, so the tiles that run together on one XCD share both their A rows and
// their B columns slab by slab in that XCD's L2.
#pragma once
#include <type_traits>
#include "gemm.h"
#include "lds_dma.h"

namespace dfl {

typedef float f32x16 __attribute__((ext_vector_type(16)));

template <typename T> struct Mfma32;
template <> struct Mfma32<bf16_t> {
  typedef bf16x8 type;
  __device__ __forceinline__ static void mma(f32x16& c, const bf16x8& a, const bf16x8& b) {
    c = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
  }
};
template <> struct Mfma32<f16_t> {
  typedef f16x8 type;
  __device__ __forceinline__ static void mma(f32x16& c, const f16x8& a, const f16x8& b) {
    c = __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
  }
};

// (tm, tn) of logical tile q: GM tile-rows per group, the column index running
// inside a group (the last group may hold fewer rows).
__host__ __device__ __forceinline__ void grouped_tile(int q, int tiles_m, int tiles_n, int GM, int& tm, int& tn) {
  const int per_group = GM * tiles_n;
  const int grp = q / per_group, r = q - grp * per_group;
  const int rows = min(GM, tiles_m - grp * GM);
  tm = grp * GM + r % rows;
  tn = r / rows;
}

constexpr int GEMM256_TILE = 256, GEMM256_THREADS = 512, GEMM256_GROUP_M = 8;

template <typename T, class Epi, bool A64 = false>
__global__ __launch_bounds__(GEMM256_THREADS) void gemm256_kernel(const GemmArgs g, const typename Epi::Params ep) {
  static_assert(sizeof(T) == 2, "16-bit operands");
  typedef typename Mfma32<T>::type FragT;
  constexpr int FM = 4, FN = 2, WGM = 2;
  constexpr int NT = GEMM256_THREADS;
  constexpr int WM = 32 * FM, WN = 32 * FN;
  constexpr int BM = GEMM256_TILE, BN = GEMM256_TILE;
  constexpr int BK = 64;
  constexpr int RPC = NT / 8;                  // rows per copy round (8 chunks of 16 bytes per row)
  constexpr int NA = BM / RPC, NB = BN / RPC, NL = NA + NB;
  constexpr int CPS = 4;                       // copies per k step
  constexpr int ER = 32, EPI_GROUPS = NT / 256;   // epilogue: two 256-thread groups, one 32-row slab each
  static_assert(NL % CPS == 0 && NL / CPS <= 4, "copies fit the slab's k steps");
  static_assert(EPI_GROUPS * ER * (BN + 1) * 4 <= 2 * (BM + BN) * 128, "epilogue slabs must fit the stages");

  __shared__ uint4 smem[2 * (BM + BN) * 8];
  auto stA = [&](int st) { return smem + st * ((BM + BN) * 8); };
  auto stB = [&](int st) { return smem + st * ((BM + BN) * 8) + BM * 8; };
  // the stages as LDS byte addresses for the copies (integers: no generic pointer
  // round trip per copy)
  const uint32_t lds0 = lds_addr(smem);
  auto ldsA = [&](int st) { return lds0 + (uint32_t)(st * (BM + BN) * 128); };
  auto ldsB = [&](int st) { return lds0 + (uint32_t)((st * (BM + BN) + BM) * 128); };

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave % WGM, wn = wave / WGM;
  const int logical = xcd_remap(blockIdx.x, gridDim.x);
  if (logical >= g.tiles_m * g.tiles_n) return;
  int tm, tn;
  grouped_tile(logical, g.tiles_m, g.tiles_n, min(GEMM256_GROUP_M, g.tiles_m), tm, tn);
  const int split = blockIdx.y;
  const int m_base = tm * BM, n_base = tn * BN;
  if (g.m_valid && m_base >= *g.m_valid - g.m_valid_base) return;
  const int k_begin = split * g.k_per_split;
  const int k_end = min(g.K, k_begin + g.k_per_split);
  const int nk = max(0, (k_end - k_begin) / BK);

  // copy slots: round i covers rows [i*RPC, (i+1)*RPC); wave w's instruction of a
  // round fills rows i*RPC + 8w .. +7, lane l -> row +l/8, slot l%8, which holds
  // logical chunk (l%8) ^ swz(row).
  const int crow = wave * 8 + (lane >> 3);
  const int cchunk = (lane & 7) ^ swz(crow);
  typedef typename std::conditional<A64, int64_t, uint32_t>::type AOff;
  AOff a_off[NA];
#pragma unroll
  for (int i = 0; i < NA; ++i) {
    const int m = m_base + i * RPC + crow;
    int64_t s = 0;                             // rows outside the product read row 0 (discarded)
    if (m < g.M) {
      s = g.a_rows ? g.a_rows[m] : m;
      if (s < 0) s = 0;
    }
    a_off[i] = (AOff)(s * g.a_ld[0] * (int64_t)sizeof(T) + cchunk * 16);
  }
  const char* b_base[NB];
  uint32_t b_off[NB];
#pragma unroll
  for (int j = 0; j < NB; ++j) {
    const int r0 = n_base + j * RPC + wave * 8;        // first row of this wave's copy (uniform)
    const T* p0 = b_row_ptr<T, BN>(g, r0);
    const bool valid = p0 && r0 + (lane >> 3) < g.N;   // 8-row blocks never straddle a segment boundary
    b_base[j] = (const char*)(p0 ? p0 : (const T*)g.b_ptr[0]);
    b_off[j] = (uint32_t)((valid ? (lane >> 3) : 0) * g.b_ld * (int64_t)sizeof(T)) + cchunk * 16;
  }

  // running A slab pointer (kernel arguments are read again only when a slab
  // crosses into the next A segment)
  const int a_segk = g.a_segk, a_nseg = g.a_nseg;
  int a_seg = k_begin / a_segk, a_kk = k_begin - a_seg * a_segk;
  const char* a_slab = (const char*)g.a_ptr[a_seg] + (int64_t)a_kk * sizeof(T);
  auto copy = [&](int q, int kt, int st) {     // copy q of slab kt into stage st (A copies first)
    if (q < NA) {
      const uint32_t d = ldsA(st) + (uint32_t)((q * RPC * 8 + wave * 64) * 16);
      if constexpr (A64) copy16_to_lds_m0(a_slab + a_off[q], d);
      else copy16_to_lds_sv_m0(a_slab, a_off[q], d);
    } else {
      const int j = q - NA;
      const int k0 = k_begin + kt * BK;
      copy16_to_lds_sv_m0(b_base[j] + (int64_t)k0 * sizeof(T), b_off[j],
                          ldsB(st) + (uint32_t)((j * RPC * 8 + wave * 64) * 16));
    }
  };
  auto advance_a = [&]() {
    a_kk += BK;
    a_slab += BK * sizeof(T);
    if (a_kk == a_segk) {
      ++a_seg;
      a_kk = 0;
      if (a_seg < a_nseg) a_slab = (const char*)g.a_ptr[a_seg];
      wait_lgkmcnt0();   // no scalar load left pending on the loop's back edge
    }
  };

  f32x16 acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.f;

  const int r32 = lane & 31, khalf = lane >> 5;
  FragT af[2][FM], bfr[2][FN];
  auto read_frags = [&](int st, int s, int set) {
    const uint4* bufA = stA(st);
    const uint4* bufB = stB(st);
    const int c = s * 2 + khalf;
#pragma unroll
    for (int fi = 0; fi < FM; ++fi) {
      const int row = wm * WM + fi * 32 + r32;
      *(uint4*)&af[set][fi] = bufA[row * 8 + (c ^ swz(row))];
    }
#pragma unroll
    for (int fj = 0; fj < FN; ++fj) {
      const int row = wn * WN + fj * 32 + r32;
      *(uint4*)&bfr[set][fj] = bufB[row * 8 + (c ^ swz(row))];
    }
  };

  // prologue: slab 0 landed and its first fragments read
  if (nk > 0) {
#pragma unroll
    for (int q = 0; q < NL; ++q) copy(q, 0, 0);
    advance_a();
    wait_vmcnt<0>();
    lds_barrier();
    read_frags(0, 0, 0);
  }
  constexpr int HALF = FM * FN / 2;
  for (int kt = 0; kt < nk; ++kt) {
    const int st = kt & 1;
    const bool more = kt + 1 < nk;
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      // slab kt+1 into the other stage: free since the barrier that published slab kt
      if (more && s * CPS < NL) {
#pragma unroll
        for (int c = 0; c < CPS; ++c) copy(s * CPS + c, kt + 1, st ^ 1);
        if ((s + 1) * CPS >= NL) advance_a();
      }
      if (s < 3) {
        read_frags(st, s + 1, (s + 1) & 1);
#pragma unroll
        for (int fi = 0; fi < FM; ++fi)
#pragma unroll
          for (int fj = 0; fj < FN; ++fj) Mfma32<T>::mma(acc[fi][fj], af[s & 1][fi], bfr[s & 1][fj]);
      } else {
#pragma unroll
        for (int f = 0; f < HALF; ++f) Mfma32<T>::mma(acc[f / FN][f % FN], af[1][f / FN], bfr[1][f % FN]);
        __builtin_amdgcn_sched_barrier(0);
        if (more) {
          wait_vmcnt<0>();
          lds_barrier();
          read_frags(st ^ 1, 0, 0);
        }
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int f = HALF; f < FM * FN; ++f) Mfma32<T>::mma(acc[f / FN][f % FN], af[1][f / FN], bfr[1][f % FN]);
      }
    }
  }
  wait_vmcnt<0>();
  lds_barrier();

  if (g.splits > 1) {
    float* P = g.partials + (int64_t)split * g.Mpad * g.Npad;
#pragma unroll
    for (int fi = 0; fi < FM; ++fi)
#pragma unroll
      for (int fj = 0; fj < FN; ++fj) {
        const int col = n_base + wn * WN + fj * 32 + r32;
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const int row = m_base + wm * WM + fi * 32 + 8 * (e / 4) + 4 * khalf + (e % 4);
          P[(int64_t)row * g.Npad + col] = acc[fi][fj][e];
        }
      }
    return;
  }

  // epilogue: 64 rows per pass staged in LDS, one 32-row slab per 256-thread group
  float* stage = (float*)smem;
  constexpr int LD = BN + 1;
  const int eg = tid >> 8, etid = tid & 255;
#pragma unroll
  for (int pass = 0; pass < BM / (ER * EPI_GROUPS); ++pass) {
    const int row0 = pass * ER * EPI_GROUPS;
    if (m_base + row0 >= g.M) break;
#pragma unroll
    for (int fi = 0; fi < FM; ++fi) {
      const int fr = wm * WM + fi * 32;
      if (fr + 32 <= row0 || fr >= row0 + ER * EPI_GROUPS) continue;
#pragma unroll
      for (int fj = 0; fj < FN; ++fj) {
        const int col = wn * WN + fj * 32 + r32;
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const int r = fr + 8 * (e / 4) + 4 * khalf + (e % 4) - row0;
          stage[r * LD + col] = acc[fi][fj][e] * g.out_scale;
        }
      }
    }
    __syncthreads();
    Epi::template apply<BN, ER>(ep, stage + eg * ER * LD, LD, m_base + row0 + eg * ER, n_base, g.M, g.N, tn, etid);
    __syncthreads();
  }
}

}  // namespace dfl
