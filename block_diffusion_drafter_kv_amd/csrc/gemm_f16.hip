// fp16-operand GEMM instantiations (every product of a bf16 drafter but the fc).
#include "gemm_dispatch.h"

namespace dfl {

void gemm_dispatch_f16(EpiKind kind, const GemmPlan& pl, const GemmArgs& g, const void* ep, hipStream_t s) {
  gemm_dispatch_t<f16_t>(kind, pl, g, ep, s);
}

}  // namespace dfl
