// Pipelined 16-bit (fp16 or bf16 operands) MFMA GEMM for gfx950:  C[M, N] = A[M, K] . B[N, K]^T.
//
// Same operand addressing, split-K and LDS-staged epilogues as gemm.h, with a
// deeper memory pipeline: K advances in 128-byte slabs that are copied from
// global memory straight into a ring of STAGES LDS buffers with 16-byte
// global_load_lds (no register staging).  Each thread issues its copies for
// slab k + STAGES - 1 while the MFMAs run on slab k; a per-thread vmcnt wait
// plus a workgroup barrier publishes a slab.  A raw s_barrier is used (not
// __syncthreads, whose release fence would drain every outstanding copy).
//
// LDS layout of one buffer: A rows [0, BM) then B rows [0, BN), 8 chunks of 16
// bytes per row with chunk c of row r stored at slot c ^ swz16(r); the copy
// unit writes lane l of a wave to slot (wave base + l), so each lane fetches
// the global chunk that belongs in its slot.
#pragma once
#include <type_traits>
#include "epilogues.h"
#include "gemm.h"
#include "lds_dma.h"

namespace dfl {

static constexpr int GEMM2_EPI_ROWS = 32;   // epilogue slab: 32 rows x (BN+1) fp32 fit one ring buffer

// SA / SB: ring depths of the A (activation) and B (weight) slabs.  Either both
// rings have the same depth, or A is double-buffered and B runs deeper: weight
// slabs come from HBM with a longer latency than the L2-resident activations.
//
// A64: A rows are addressed with per-lane 64-bit byte offsets (one 64-bit add per
// copy) instead of 32-bit offsets from a wave-uniform base, for A buffers of
// 4 GiB or more (the injection's caller-provided hidden states).
//
// NT: 256 threads (4 waves, 2 x 2) or 512 (8 waves, 2 x 4, half the columns per
// wave): two 8-wave work-groups per CU keep four waves on each SIMD, which
// hides more of each slab's wait (measured on the 544-row products: gate/up
// 128 x 128 tiles 148 -> 134 us, down 192 x 128 with K split in four 84 -> 79 us;
// the narrower QKV and O tilings are as fast or faster with 4 waves).
template <typename T, int BM, int BN, int SA, int SB, class Epi, bool A64 = false, int NT = 256>
__global__ __launch_bounds__(NT) void gemm2_kernel(const GemmArgs g, const typename Epi::Params ep) {
  static_assert(sizeof(T) == 2, "16-bit operands");
  static_assert(NT == 256 || NT == 512, "4 or 8 waves");
  typedef typename Frag<T>::type FragT;
  constexpr int BK = 64;
  constexpr int NW = NT / 64, WGN = NW / 2;                 // waves: 2 along M x WGN along N
  constexpr int RPC = NT / 8;                               // rows per copy round
  constexpr int WM = BM / 2, WN = BN / WGN, FM = WM / 16, FN = WN / 16;
  static_assert(WN % 16 == 0 && BM % RPC == 0 && BN % RPC == 0, "tile shape");
  constexpr int NA = BM / RPC, NB = BN / RPC, NL = NA + NB;
  constexpr int ER = GEMM2_EPI_ROWS;
  static_assert(SA >= 2 && SB >= 2 && SA <= 4 && SB <= 4 && (SA == SB || SA == 2), "ring depths");
  static_assert((SA - 2) * NL < 64 && NB * (SB - 1) < 64, "vmcnt range");
  static_assert(ER * (BN + 1) * 4 <= (SA * BM + SB * BN) * 8 * 16, "epilogue slab must fit the rings");

  // one LDS block: A ring [SA][BM rows] then B ring [SB][BN rows], 8 chunks per row
  __shared__ uint4 smem[(SA * BM + SB * BN) * 8];
  auto smemA = [&](int st) { return smem + st * (BM * 8); };
  auto smemB = [&](int st) { return smem + SA * BM * 8 + st * (BN * 8); };
  // the same stages as LDS byte addresses for the copies (integers: no generic
  // pointer round trip per copy)
  const uint32_t lds0 = lds_addr(smem);
  auto ldsA = [&](int st) { return lds0 + (uint32_t)(st * BM * 128); };
  auto ldsB = [&](int st) { return lds0 + (uint32_t)((SA * BM + st * BN) * 128); };

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform (scalar) index
  const int wm = wave & 1, wn = wave >> 1;
  const int logical = xcd_remap(blockIdx.x, gridDim.x);
  if (logical >= g.tiles_m * g.tiles_n) return;
  const int tm = logical % g.tiles_m, tn = logical / g.tiles_m;
  const int split = blockIdx.y;
  const int m_base = tm * BM, n_base = tn * BN;
  if (g.m_valid && m_base >= *g.m_valid - g.m_valid_base) return;
  const int k_begin = split * g.k_per_split;
  const int k_end = min(g.K, k_begin + g.k_per_split);
  const int nk = max(0, (k_end - k_begin) / BK);

  // this thread's copy slots: rows (i*32 + tid/8) of A and B, logical chunk cchunk.
  // Every copy instruction of a wave covers 8 consecutive rows of one operand, so
  // it takes a wave-uniform base (SGPRs) plus a per-lane 32-bit byte offset that
  // stays fixed for the whole K loop; only the bases advance per slab.
  const int crow = tid >> 3;   // 0 .. RPC-1
  const int cchunk = (tid & 7) ^ swz16(crow);
  typedef typename std::conditional<A64, int64_t, uint32_t>::type AOff;
  AOff a_off[NA];
#pragma unroll
  for (int i = 0; i < NA; ++i) {
    const int m = m_base + i * RPC + crow;
    int64_t s = 0;                      // rows outside the product read row 0 (discarded)
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
    const int r0 = n_base + j * RPC + wave * 8;         // first row of this wave's block (uniform)
    const T* p0 = b_row_ptr<T, BN>(g, r0);
    const bool valid = p0 && r0 + (lane >> 3) < g.N;    // blocks never straddle a segment boundary
    b_base[j] = (const char*)(p0 ? p0 : (const T*)g.b_ptr[0]);
    b_off[j] = (uint32_t)((valid ? (lane >> 3) : 0) * g.b_ld * (int64_t)sizeof(T)) + cchunk * 16;
  }

  // A-segment cursor of the next slab to issue (A slabs are issued in K order);
  // the segment's base pointer is read from the arguments only when the
  // cursor enters a segment
  int a_seg = k_begin / g.a_segk, a_kk = k_begin - a_seg * g.a_segk;
  const char* a_cur = (const char*)g.a_ptr[a_seg < g.a_nseg ? a_seg : 0];
  auto issue_a = [&](uint32_t dst) {
    const char* abase = a_cur + (int64_t)a_kk * sizeof(T);
#pragma unroll
    for (int i = 0; i < NA; ++i) {
      const uint32_t d = dst + (uint32_t)((i * RPC * 8 + wave * 64) * 16);
      if constexpr (A64) copy16_to_lds_m0(abase + a_off[i], d);
      else copy16_to_lds_sv_m0(abase, a_off[i], d);
    }
    a_kk += BK;
    if (a_kk == g.a_segk) {
      ++a_seg;
      a_kk = 0;
      if (a_seg < g.a_nseg) a_cur = (const char*)g.a_ptr[a_seg];
    }
  };
  auto issue_b = [&](int kt, uint32_t dst) {
    const int k0 = k_begin + kt * BK;
#pragma unroll
    for (int j = 0; j < NB; ++j)
      copy16_to_lds_sv_m0(b_base[j] + (int64_t)k0 * sizeof(T), b_off[j], dst + (uint32_t)((j * RPC * 8 + wave * 64) * 16));
  };

  // 4-wave tiles with the residual add: the epilogue's X rows are loaded before
  // the main loop, so their latency hides behind it (the product never reads X)
  constexpr int EG = NT / 256;
  constexpr bool PRE = std::is_same<Epi, EpiResidualAdd>::value && NT == 256 && BM % GEMM2_EPI_ROWS == 0;
  constexpr int NPRE = PRE ? BM / GEMM2_EPI_ROWS : 1;
  typename std::conditional<PRE, EpiResidualAdd::Pre<BN, GEMM2_EPI_ROWS>, int>::type pre[NPRE];
  if constexpr (PRE) {
    if (g.splits == 1) {
#pragma unroll
      for (int ps = 0; ps < NPRE; ++ps)
        EpiResidualAdd::load<BN, GEMM2_EPI_ROWS>(ep, m_base + ps * GEMM2_EPI_ROWS, n_base, g.M, g.N, tid, pre[ps]);
    }
  }

  f32x4 acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  const int grp = lane >> 4, r16 = lane & 15;
  auto compute = [&](const uint4* bufA, const uint4* bufB) {
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      FragT af[FM], bfr[FN];
      const int c = s * 4 + grp;
#pragma unroll
      for (int fi = 0; fi < FM; ++fi) {
        const int row = wm * WM + fi * 16 + r16;
        *(uint4*)&af[fi] = bufA[row * 8 + (c ^ swz16(row))];
      }
#pragma unroll
      for (int fj = 0; fj < FN; ++fj) {
        const int row = wn * WN + fj * 16 + r16;
        *(uint4*)&bfr[fj] = bufB[row * 8 + (c ^ swz16(row))];
      }
#pragma unroll
      for (int fi = 0; fi < FM; ++fi)
#pragma unroll
        for (int fj = 0; fj < FN; ++fj) Frag<T>::mma(acc[fi][fj], af[fi], bfr[fj]);
    }
  };
  // rings: slab kt lives in A stage kt % SA and B stage kt % SB.  Issue order:
  // prologue p = 0 .. max(SA, SB) - 2 gives [A(p) if p < SA-1][B(p) if p < SB-1];
  // iteration kt (after its barrier) gives [A(kt+SA-1)][B(kt+SB-1)] when in range.
#pragma unroll
  for (int p = 0; p < (SA > SB ? SA : SB) - 1; ++p) {
    if (p < SA - 1 && p < nk) issue_a(ldsA(p));
    if (p < SB - 1 && p < nk) issue_b(p, ldsB(p));
  }
  for (int kt = 0; kt < nk; ++kt) {
    // wait until A(kt) and B(kt) have landed: count the copies issued after them
    if constexpr (SA == SB) {
      const int ahead = min(SA - 2, nk - 1 - kt);   // slabs after kt allowed to stay in flight
      if constexpr (SA == 4) {
        if (ahead >= 2) wait_vmcnt<2 * NL>();
        else if (ahead == 1) wait_vmcnt<NL>();
        else wait_vmcnt<0>();
      } else if constexpr (SA == 3) {
        if (ahead >= 1) wait_vmcnt<NL>();
        else wait_vmcnt<0>();
      } else {
        wait_vmcnt<0>();
      }
    } else {
      // SA == 2: A(kt) was issued last (iteration kt-1), followed only by B(kt+SB-2)
      // (at kt = 0 this also waits for B(1..SB-2): conservative)
      if (kt + SB - 2 < nk) wait_vmcnt<NB>();
      else wait_vmcnt<0>();
    }
    lds_barrier();
    if (kt + SA - 1 < nk) issue_a(ldsA((kt + SA - 1) % SA));
    if (kt + SB - 1 < nk) issue_b(kt + SB - 1, ldsB((kt + SB - 1) % SB));
    compute(smemA(kt % SA), smemB(kt % SB));
  }
  wait_vmcnt<0>();
  lds_barrier();

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

  // epilogue: NT/256 slabs of ER rows per pass staged as fp32 [ER][BN + 1], one
  // per 256-thread group (the epilogues are written for 256 threads)
  static_assert(EG * ER * (BN + 1) * 4 <= (SA * BM + SB * BN) * 8 * 16, "epilogue slabs must fit the rings");
  static_assert(BM % (EG * ER) == 0, "whole epilogue passes");
  float* stage = (float*)smem;
  const int eg = tid / 256;
#pragma unroll
  for (int pass = 0; pass < BM / (EG * ER); ++pass) {
    if (m_base + pass * EG * ER >= g.M) break;
#pragma unroll
    for (int fi = 0; fi < FM; ++fi) {
      const int row0 = wm * WM + fi * 16;
      if (row0 < pass * EG * ER || row0 >= (pass + 1) * EG * ER) continue;
#pragma unroll
      for (int fj = 0; fj < FN; ++fj) {
        const int col = wn * WN + fj * 16 + r16;
#pragma unroll
        for (int i = 0; i < 4; ++i)
          stage[(row0 - pass * EG * ER + grp * 4 + i) * (BN + 1) + col] = acc[fi][fj][i] * g.out_scale;
      }
    }
    __syncthreads();
    if constexpr (PRE)
      EpiResidualAdd::add<BN, ER>(ep, stage, BN + 1, m_base + pass * ER, n_base, g.M, g.N, tid, pre[pass]);
    else
      Epi::template apply<BN, ER>(ep, stage + eg * ER * (BN + 1), BN + 1, m_base + (pass * EG + eg) * ER, n_base, g.M,
                                  g.N, tn, tid & 255);
    __syncthreads();
  }
}

}  // namespace dfl
