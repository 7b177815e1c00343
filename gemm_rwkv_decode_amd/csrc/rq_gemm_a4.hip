// rq_gemm_a4.hip -- the matrix-core kernel's instances for 4-bit asymmetric superblock codes.
#include "rq_gemm_impl.h"

namespace rq {

hipError_t launch_gemm_fmt_a4(const Problem* const* p, int n, const GemmCfg& c, float* ws, hipStream_t s) {
  return launch_fmt<FMT_A4>(p, n, c, ws, s);
}

}  // namespace rq
