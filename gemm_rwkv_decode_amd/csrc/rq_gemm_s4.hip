// rq_gemm_s4.hip -- the matrix-core kernel's instances for symmetric 4-bit codes (groups of 32, 64, 128).
#include "rq_gemm_impl.h"

namespace rq {

hipError_t launch_gemm_fmt_s4(const Problem* const* p, int n, const GemmCfg& c, float* ws, hipStream_t s) {
  return launch_fmt<FMT_S4>(p, n, c, ws, s);
}

}  // namespace rq
