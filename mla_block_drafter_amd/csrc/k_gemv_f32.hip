// Skinny-GEMM instantiations for f32 weights (see gemv_impl.h).
#include "gemv_impl.h"

namespace dspark {

hipError_t launch_gemv_f32(const GemvArgs& a, const GemvPlan& p, int mode, hipStream_t st) {
  if (mode == GEMV_MARKOV) return dispatch_markov<DT_F32>(a, p, st);
  return dispatch_fmt<DT_F32>(a, p, mode, st);
}

}  // namespace dspark
