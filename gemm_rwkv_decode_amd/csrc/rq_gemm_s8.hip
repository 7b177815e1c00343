// rq_gemm_s8.hip -- the matrix-core kernel's instances for symmetric 8-bit codes (groups of 16, 32, 64).
#include "rq_gemm_impl.h"

namespace rq {

hipError_t launch_gemm_fmt_s8(const Problem* const* p, int n, const GemmCfg& c, float* ws, hipStream_t s) {
  return launch_fmt<FMT_S8>(p, n, c, ws, s);
}

}  // namespace rq
