// rq_gemm.hip -- y = x W^T on the matrix cores for small batches (M <= 64):
// the dispatch to the per-format instances (rq_gemm_<format>.hip); the plan
// choice is in rq_gemm_plan.h.  The kernel and its design are in
// rq_gemm_impl.h.
#include "rq_gemm_plan.h"

namespace rq {

hipError_t launch_gemm_many(const Problem* const* p, int count, const GemmCfg& c, float* ws,
                            hipStream_t s) {
  if (count > 1 && c.splits > 1) return hipErrorInvalidValue;
  for (int first = 0; first < count; first += MM_BATCH) {
    const int n = count - first < MM_BATCH ? count - first : MM_BATCH;
    const Problem* const* q = p + first;
    hipError_t e;
    switch (q[0]->fmt) {
      case FMT_S4: e = launch_gemm_fmt_s4(q, n, c, ws, s); break;
      case FMT_S8: e = launch_gemm_fmt_s8(q, n, c, ws, s); break;
      case FMT_F8: e = launch_gemm_fmt_f8(q, n, c, ws, s); break;
      case FMT_A5: e = launch_gemm_fmt_a5(q, n, c, ws, s); break;
      case FMT_A6: e = launch_gemm_fmt_a6(q, n, c, ws, s); break;
      default: e = launch_gemm_fmt_a4(q, n, c, ws, s); break;
    }
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

hipError_t launch_gemm(const Problem& p, const GemmCfg& c, float* ws, hipStream_t s) {
  const Problem* one = &p;
  return launch_gemm_many(&one, 1, c, ws, s);
}

}  // namespace rq
