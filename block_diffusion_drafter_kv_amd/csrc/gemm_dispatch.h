// Host-side dispatch of the GEMM kernel template over (epilogue, tile height).
#pragma once
#include "ops.h"

namespace dfl {

template <typename T, int BM, class Epi>
static void gemm_go(const GemmArgs& g, const void* ep, hipStream_t s) {
  const typename Epi::Params& p = *(const typename Epi::Params*)ep;
  dim3 grid(g.tiles_m * g.tiles_n, g.splits);
  gemm_kernel<T, BM, 128, Epi><<<grid, 256, 0, s>>>(g, p);
  if (g.splits > 1) gemm_reduce_kernel<BM, 128, Epi><<<g.tiles_m * g.tiles_n, 256, 0, s>>>(g, p);
}

template <typename T, class Epi>
static void gemm_bm(int bm, const GemmArgs& g, const void* ep, hipStream_t s) {
  if (bm == 64) gemm_go<T, 64, Epi>(g, ep, s);
  else gemm_go<T, 128, Epi>(g, ep, s);
}

template <typename T>
static void gemm_dispatch_t(EpiKind kind, int bm, const GemmArgs& g, const void* ep, hipStream_t s) {
  switch (kind) {
    case EPI_STORE_F32: gemm_bm<T, EpiStore<float>>(bm, g, ep, s); break;
    case EPI_STORE_T: gemm_bm<T, EpiStore<T>>(bm, g, ep, s); break;
    case EPI_RESADD: gemm_bm<T, EpiResidualAdd>(bm, g, ep, s); break;
    case EPI_SWIGLU: gemm_bm<T, EpiSwiGLU<T>>(bm, g, ep, s); break;
    case EPI_QKV: gemm_bm<T, EpiQKV<T>>(bm, g, ep, s); break;
    case EPI_KVINJECT: gemm_bm<T, EpiKVInject<T>>(bm, g, ep, s); break;
    case EPI_LMHEAD: gemm_bm<T, EpiLMHead>(bm, g, ep, s); break;
  }
}

void gemm_dispatch_bf16(EpiKind kind, int bm, const GemmArgs& g, const void* ep, hipStream_t s);
void gemm_dispatch_f32(EpiKind kind, int bm, const GemmArgs& g, const void* ep, hipStream_t s);

}  // namespace dfl
