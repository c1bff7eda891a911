// Skinny-GEMM instantiations for MXFP4 weights (see gemv_impl.h).
#include "gemv_impl.h"

namespace dspark {

hipError_t launch_gemv_mxfp4(const GemvArgs& a, const GemvPlan& p, int mode, hipStream_t st) {
  if (mode == GEMV_MARKOV || p.ksteps_per_split % 4 || a.w.KB % 4) return hipErrorInvalidValue;
  return dispatch_fmt<DT_MXFP4>(a, p, mode, st);
}

}  // namespace dspark
