// rq_gemm.hip -- y = x W^T on the matrix cores for small batches (M <= 64):
// plan choice, the split-K reduce, and the dispatch to the per-format
// instances (rq_gemm_<format>.hip).  The kernel and its design are in
// rq_gemm_impl.h.
#include "rq_gemm_plan.h"

namespace rq {

// y[i] = sum over K-ranges s = 0..splits-1 (in order) of ws[s][i], i < count.
__global__ void __launch_bounds__(256)
k_split_reduce(const float* __restrict__ ws, float* __restrict__ y, size_t count,
               int splits) {
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < count;
       i += (size_t)gridDim.x * blockDim.x) {
    float v = 0.0f;
    for (int sp = 0; sp < splits; sp++) v += ws[(size_t)sp * count + i];
    y[i] = v;
  }
}

void launch_split_reduce(const float* ws, float* y, size_t count, int splits, hipStream_t s) {
  size_t rb = (count + 255) / 256;
  if (rb > 1024) rb = 1024;
  hipLaunchKernelGGL(k_split_reduce, dim3((unsigned)rb), dim3(256), 0, s, ws, y, count, splits);
}

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
