// Host-side dispatch of the GEMM kernel templates over (operand type, epilogue,
// tile shape).  16-bit products (fp16, or bf16 for the fc) use the pipelined
// gemm2 kernel; fp32 products use the register-staged kernel of gemm.h.  Tile
// shapes (measured on MI355X):
//   16-bit, M > 64 : 128 x 128, 2 LDS stages (64 KB: two 8-wave work-groups per CU)
//   16-bit, M <= 64: 64 x 128, 3 stages
//   16-bit LM head and long-K products: 128 x 128, A 2 stages, B 3 stages
//   fp32           : 128 x 128 or 64 x 128
//   16-bit, many rows (injection fc and K|V) and the vocabulary product: 256 x 256
//   (gemm256.h), for the epilogues listed in Gemm256Epi
#pragma once
#include "gemm2.h"
#include "gemm256.h"
#include "ops.h"

namespace dfl {

// Epilogues the 256 x 256 kernel is instantiated for (the products planned onto it)
template <class Epi> struct Gemm256Epi { static constexpr bool value = false; };
template <> struct Gemm256Epi<EpiStore<float>> { static constexpr bool value = true; };
template <> struct Gemm256Epi<EpiKVInject<f16_t>> { static constexpr bool value = true; };
template <> struct Gemm256Epi<EpiKVInject<bf16_t>> { static constexpr bool value = true; };
template <> struct Gemm256Epi<EpiLMHead> { static constexpr bool value = true; };

template <typename T, class Epi>
static void gemm256_go(const GemmArgs& g, const void* ep, hipStream_t s) {
  const typename Epi::Params& p = *(const typename Epi::Params*)ep;
  dim3 grid(gemm_grid(g.tiles_m * g.tiles_n), 1);
  if constexpr (std::is_same<T, bf16_t>::value) {
    if (g.a_wide) {
      gemm256_kernel<T, Epi, true><<<grid, GEMM256_THREADS, 0, s>>>(g, p);
      return;
    }
  }
  gemm256_kernel<T, Epi><<<grid, GEMM256_THREADS, 0, s>>>(g, p);
}

template <typename T, int BM, int BN, int SA, int SB, class Epi, int NT = 256>
static void gemm2_go(const GemmArgs& g, const void* ep, hipStream_t s) {
  const typename Epi::Params& p = *(const typename Epi::Params*)ep;
  dim3 grid(gemm_grid(g.tiles_m * g.tiles_n), g.splits);
  // 64-bit A offsets only where a caller's buffer may exceed 4 GiB (the injection
  // fc over the caller's bf16 hidden states)
  if constexpr (std::is_same<T, bf16_t>::value) {
    if (g.a_wide) {
      gemm2_kernel<T, BM, BN, SA, SB, Epi, true, NT><<<grid, NT, 0, s>>>(g, p);
      if (g.splits > 1 && !g.keep_partials) gemm_reduce_kernel<BM, BN, Epi><<<reduce_grid<BM>(g), 256, 0, s>>>(g, p);
      return;
    }
  }
  gemm2_kernel<T, BM, BN, SA, SB, Epi, false, NT><<<grid, NT, 0, s>>>(g, p);
  if (g.splits > 1 && !g.keep_partials) gemm_reduce_kernel<BM, BN, Epi><<<reduce_grid<BM>(g), 256, 0, s>>>(g, p);
}

template <int BM, class Epi>
static void gemm1_go(const GemmArgs& g, const void* ep, hipStream_t s) {
  const typename Epi::Params& p = *(const typename Epi::Params*)ep;
  dim3 grid(gemm_grid(g.tiles_m * g.tiles_n), g.splits);
  gemm_kernel<float, BM, 128, Epi><<<grid, 256, 0, s>>>(g, p);
  if (g.splits > 1 && !g.keep_partials) gemm_reduce_kernel<BM, 128, Epi><<<reduce_grid<BM>(g), 256, 0, s>>>(g, p);
}

// Epilogues that work on whole heads or whole 128-column statistics tiles need
// output tiles at least 128 wide.
template <class Epi> struct EpiNeedsWide { static constexpr bool value = false; };
template <typename T> struct EpiNeedsWide<EpiQKV<T>> { static constexpr bool value = true; };
template <typename T> struct EpiNeedsWide<EpiKVInject<T>> { static constexpr bool value = true; };
template <> struct EpiNeedsWide<EpiLMHead> { static constexpr bool value = true; };

template <typename T, class Epi>
static void gemm_cfg(const GemmPlan& pl, const GemmArgs& g, const void* ep, hipStream_t s) {
  if constexpr (sizeof(T) == 2) {
    if constexpr (Gemm256Epi<Epi>::value) {
      if (pl.bm == 256) {
        gemm256_go<T, Epi>(g, ep, s);
        return;
      }
    }
    // the 16-bit tilings (BM x BN, A ring, B ring): exactly the plans that
    // runnable_plan lets through (anything else arrives as 128 x 128)
    if (pl.bm == 64 && pl.bn == 128) gemm2_go<T, 64, 128, 3, 3, Epi>(g, ep, s);
    else if (pl.bm == 192 && pl.bn == 128) gemm2_go<T, 192, 128, 2, 2, Epi, 512>(g, ep, s);
    else if (pl.bm == 128 && pl.bn == 128 && pl.sb == 3) gemm2_go<T, 128, 128, 2, 3, Epi>(g, ep, s);
    else if constexpr (!EpiNeedsWide<Epi>::value) {
      if (pl.bm == 96 && pl.bn == 64) gemm2_go<T, 96, 64, 4, 4, Epi>(g, ep, s);
      else if (pl.bm == 64 && pl.bn == 64) gemm2_go<T, 64, 64, 4, 4, Epi>(g, ep, s);
      else gemm2_go<T, 128, 128, 2, 2, Epi, 512>(g, ep, s);
    } else {
      gemm2_go<T, 128, 128, 2, 2, Epi, 512>(g, ep, s);
    }
  } else {
    if (pl.bm == 64) gemm1_go<64, Epi>(g, ep, s);
    else gemm1_go<128, Epi>(g, ep, s);
  }
}

template <typename T>
static void gemm_dispatch_t(EpiKind kind, const GemmPlan& pl, const GemmArgs& g, const void* ep, hipStream_t s) {
  switch (kind) {
    case EPI_STORE_F32: gemm_cfg<T, EpiStore<float>>(pl, g, ep, s); break;
    case EPI_STORE_T: gemm_cfg<T, EpiStore<T>>(pl, g, ep, s); break;
    case EPI_RESADD: gemm_cfg<T, EpiResidualAdd>(pl, g, ep, s); break;
    case EPI_SWIGLU: gemm_cfg<T, EpiSwiGLU<T>>(pl, g, ep, s); break;
    case EPI_QKV: gemm_cfg<T, EpiQKV<T>>(pl, g, ep, s); break;
    case EPI_KVINJECT: gemm_cfg<T, EpiKVInject<T>>(pl, g, ep, s); break;
    case EPI_LMHEAD: gemm_cfg<T, EpiLMHead>(pl, g, ep, s); break;
    case EPI_STORE_SPLIT: gemm_cfg<T, EpiStoreSplit>(pl, g, ep, s); break;
  }
}

void gemm_dispatch_bf16(EpiKind kind, const GemmPlan& pl, const GemmArgs& g, const void* ep, hipStream_t s);
void gemm_dispatch_f16(EpiKind kind, const GemmPlan& pl, const GemmArgs& g, const void* ep, hipStream_t s);
void gemm_dispatch_f32(EpiKind kind, const GemmPlan& pl, const GemmArgs& g, const void* ep, hipStream_t s);

}  // namespace dfl
