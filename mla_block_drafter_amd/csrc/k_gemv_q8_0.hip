// Skinny-GEMM instantiations for q8_0 weights (see gemv_impl.h).
#include "gemv_impl.h"

namespace dspark {

hipError_t launch_gemv_q8_0(const GemvArgs& a, const GemvPlan& p, int mode, hipStream_t st) {
  if (mode == GEMV_MARKOV) return hipErrorInvalidValue;
  return dispatch_fmt<DT_Q8_0>(a, p, mode, st);
}

}  // namespace dspark
