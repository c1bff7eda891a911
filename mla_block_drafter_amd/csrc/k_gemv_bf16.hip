// Skinny-GEMM instantiations for bf16 weights (see gemv_impl.h).
#include "gemv_impl.h"

namespace dspark {

hipError_t launch_gemv_bf16(const GemvArgs& a, const GemvPlan& p, int mode, hipStream_t st) {
  if (mode == GEMV_MARKOV) return dispatch_markov<DT_BF16>(a, p, st);
  return dispatch_fmt<DT_BF16>(a, p, mode, st);
}

}  // namespace dspark
