// rq_gemm_f8.hip -- the matrix-core kernel's instances for FP8 E4M3 codes with a matrix scale.
#include "rq_gemm_impl.h"

namespace rq {

hipError_t launch_gemm_fmt_f8(const Problem* const* p, int n, const GemmCfg& c, float* ws, hipStream_t s) {
  return launch_fmt<FMT_F8>(p, n, c, ws, s);
}

}  // namespace rq
