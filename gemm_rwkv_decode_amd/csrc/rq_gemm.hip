// rq_gemm.hip -- y = x W^T on the matrix cores for small batches (M <= 64):
// plan choice, the split-K reduce, and the dispatch to the per-format
// instances (rq_gemm_<format>.hip).  The kernel and its design are in
// rq_gemm_impl.h.
#include "rq_gemm_impl.h"

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

// ---------------------------------------------------------------------------
// host side
// ---------------------------------------------------------------------------

static int round_k(int fmt, int mt, int group, int plan) {
  const Plan& q = kPlans[plan];
  return mm_round(fmt, mt, q.wk, group, q.rd);
}

static bool plan_fits(int fmt, int mt, int g, const Plan& q) {
  const int kc = mm_kc(fmt, mt, q.wk, g, q.rd);
  const int round = q.wk * kc;
  const int dx = mm_xdepth(fmt, mt, g, q.wr, q.wk, q.nt, q.rd);
  const int dc = mm_cdepth(fmt, mt, g, q.wr, q.wk, q.nt, q.rd);
  const int rs = mm_byte(fmt) ? round : round / 2;
  const int red = q.wk > 1 ? q.wr * q.wk * 64 * q.nt * mt * 4 * 4 : 0;
  if (kc % g != 0 || kc / g > 8) return false;
  if (q.nt * mt > (64 * (q.wr * q.wk + MM_XP + MM_CP) > 512 ? 4 : 8)) return false;
  if (is_asym(fmt) && (SUPERBLOCK % kc != 0 || round % SUPERBLOCK != 0)) return false;
  if (!is_asym(fmt) && (round / g) % 2 != 0) return false;
  if (rs / 16 < 8 || ((rs / 16) & (rs / 16 - 1)) != 0) return false;
  const int bytes = (dx + 1) * mm_xslot(fmt, mt, g, q.wk, q.rd) +
                    (dc + 1) * mm_cslot(fmt, mt, g, q.wr, q.wk, q.nt, q.rd);
  return dx >= 1 && dc >= 1 && bytes <= LDS_LIMIT && red * 4 <= LDS_LIMIT;
}

// The plan can run this problem: K is a whole number of rounds, a row's
// scales are whole dwords, and the workgroup's layout fits the LDS.
static bool plan_ok(int fmt, int mt, int group, int K, int plan) {
  const int rk = round_k(fmt, mt, group, plan);
  return K % rk == 0 && (K / group) % 2 == 0 && plan_fits(fmt, mt, group, kPlans[plan]);
}

size_t gemm_workspace_floats(const GemmCfg& c, int M, int N) {
  return c.splits > 1 ? (size_t)c.splits * M * N : 0;
}

bool gemm_supports(int fmt, int M, int K, int group) {
  if (fmt == FMT_F8) group = MM_F8_GROUP;
  const int mt = (M + 15) / 16;
  for (int p = 0; p < kNumPlans; p++)
    if (plan_ok(fmt, mt, group, K, p)) return true;
  return false;
}

GemmCfg choose_gemm(int fmt, int M, int N, int K, int group, int blocks48, bool allow_split) {
  if (fmt == FMT_F8) group = MM_F8_GROUP;
  GemmCfg c{};
  c.mt = (M + 15) / 16;
  c.splits = 1;
  const Tuning& tu = tuning();
  // Preference order by row count: with few rows, more K-slices per
  // workgroup keep one workgroup per CU busy; with many rows, 64-row
  // workgroups cut the x staging per row (every workgroup stages all of x,
  // M*K*2 bytes, from L2).  Measured on MI355X for the RWKV-7 shapes, int4
  // g64, weights cold in HBM.
  static const int small_n[] = {1, 0, 6, 3, 8, 4, 5, 7, 2, 9, 10, 11, 12, 13, 14, 15, 16, 17};
  static const int mid_n[] = {3, 8, 4, 1, 0, 6, 5, 7, 2, 9, 10, 11, 12, 13, 14, 15, 16, 17};
  static const int large_n[] = {5, 7, 2, 9, 8, 3, 4, 0, 6, 1, 10, 11, 12, 13, 14, 15, 16, 17};
  // Few rows and long rows (K >= 16384) or a full M-tile stack (M > 48): the
  // x staging of 16-row workgroups dominates, so 64-row workgroups with K
  // split four ways (a second, small kernel adds the partial sums) -- at
  // 4096x16384: 16.2 -> 15.0 us (M=16), 23.0 -> 18.8 us (M=32),
  // 45.8 -> 25.0 us (M=64).
  static const int split_n_m16[] = {7, 5, 9, 2, 8, 3, 4, 0, 6, 1, 10, 11, 12, 13, 14, 15, 16, 17};
  static const int split_n[] = {5, 2, 7, 9, 8, 3, 4, 0, 6, 1, 10, 11, 12, 13, 14, 15, 16, 17};
  const bool split_k = allow_split && N < 8192 && (K >= 16384 || c.mt >= 4);
  const int* order = split_k ? (c.mt == 1 ? split_n_m16 : split_n)
                             : (N >= 16384 ? large_n : (N >= 8192 ? mid_n : small_n));
  c.plan = -1;
  if (tu.gemm_plan > 0 && tu.gemm_plan <= kNumPlans &&
      plan_ok(fmt, c.mt, group, K, tu.gemm_plan - 1))
    c.plan = tu.gemm_plan - 1;
  // 48-row workgroups where they make one wave of 224..256 row blocks (64-row
  // ones leave a quarter of the CUs idle): one 12288x4096 product,
  // 14.1 -> 11.2 us (M=16), 18.3 -> 12.1 us (M=32), 30.1 -> 20.3 us (M=64).
  // Blocks are counted per problem: three 4096-row problems need 258, and
  // the two past one wave nearly double the launch.
  const int b48 = blocks48 > 0 ? blocks48 : (N + 47) / 48;
  if (c.plan < 0 && !split_k && b48 >= 224 && b48 <= 256) {
    const int p48 = c.mt <= 2 ? 17 : 15;
    if (plan_ok(fmt, c.mt, group, K, p48)) c.plan = p48;
  }
  for (int i = 0; i < kNumPlans && c.plan < 0; i++)
    if (plan_ok(fmt, c.mt, group, K, order[i])) c.plan = order[i];
  // Splits divide K into whole rounds and the partial sums stay under 64 MiB.
  // Automatic only in the case above, enough row blocks x K-ranges for 256
  // CUs (at most 4); RQ_GEMM_SPLITS overrides.
  const int rows = kPlans[c.plan].wr * kPlans[c.plan].nt * 16;
  const int blocks = (N + rows - 1) / rows;
  int want = 1;
  if (split_k && rows == 64 && blocks < 256) want = (256 + blocks - 1) / blocks;
  if (want > 4) want = 4;
  if (tu.gemm_splits) want = tu.gemm_splits;
  if (!allow_split) want = 1;
  const int nr = K / round_k(fmt, c.mt, group, c.plan);
  if (want > nr) want = nr;
  if (want < 1) want = 1;
  int sp = want;
  while (sp > 1 && (nr % sp != 0 || (size_t)sp * M * N * 4 > ((size_t)64 << 20))) sp--;
  c.splits = sp;
  return c;
}

hipError_t launch_gemm_many(const Problem* const* p, int count, const GemmCfg& c, float* ws,
                            hipStream_t s) {
  if (count > 1 && c.splits > 1) return hipErrorInvalidValue;
  for (int first = 0; first < count; first += MM_BATCH) {
    const int n = count - first < MM_BATCH ? count - first : MM_BATCH;
    const Problem* const* q = p + first;
    switch (q[0]->fmt) {
      case FMT_S4: launch_gemm_fmt_s4(q, n, c, ws, s); break;
      case FMT_S8: launch_gemm_fmt_s8(q, n, c, ws, s); break;
      case FMT_F8: launch_gemm_fmt_f8(q, n, c, ws, s); break;
      case FMT_A5: launch_gemm_fmt_a5(q, n, c, ws, s); break;
      case FMT_A6: launch_gemm_fmt_a6(q, n, c, ws, s); break;
      default: launch_gemm_fmt_a4(q, n, c, ws, s); break;
    }
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

hipError_t launch_gemm(const Problem& p, const GemmCfg& c, float* ws, hipStream_t s) {
  const Problem* one = &p;
  return launch_gemm_many(&one, 1, c, ws, s);
}

}  // namespace rq
