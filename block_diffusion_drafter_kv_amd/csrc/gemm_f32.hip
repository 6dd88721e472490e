// fp32 GEMM instantiations (fp32 drafters use v_mfma_f32_16x16x4_f32).
#include "gemm_dispatch.h"

namespace dfl {

void gemm_dispatch_f32(EpiKind kind, const GemmPlan& pl, const GemmArgs& g, const void* ep, hipStream_t s) {
  gemm_dispatch_t<float>(kind, pl, g, ep, s);
}

}  // namespace dfl
