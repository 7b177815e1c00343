// rq_gemm_a5.hip -- the matrix-core kernel's instances for 5-bit asymmetric superblock codes.
#include "rq_gemm_impl.h"

namespace rq {

hipError_t launch_gemm_fmt_a5(const Problem* const* p, int n, const GemmCfg& c, float* ws, hipStream_t s) {
  return launch_fmt<FMT_A5>(p, n, c, ws, s);
}

}  // namespace rq
