// Skinny-GEMM instantiations for fp8 weights (see gemv_impl.h).
#include "gemv_impl.h"

namespace dspark {

hipError_t launch_gemv_fp8(const GemvArgs& a, const GemvPlan& p, int mode, hipStream_t st) {
  if (mode == GEMV_MARKOV) return hipErrorInvalidValue;
  return dispatch_fmt<DT_FP8>(a, p, mode, st);
}

}  // namespace dspark
