// rq_gemm_plan.h -- host side of the matrix-core kernel: which workgroup
// arrangement (plan) runs a problem and whether K is split over workgroups.
// Included by rq_gemm.hip (and by a host-only check of the plan table).
#pragma once

#include "rq_gemm_impl.h"

#include <array>
#include <utility>

namespace rq {

static int round_k(int fmt, int mt, int group, int plan) {
  const Plan& q = kPlans[plan];
  return mm_round(fmt, mt, q.wk, group, q.rd);
}

// Whether plan `plan` fits (LDS, registers, copy layout) for the format, M-tile
// count and group: read from the kernel instance's own FITS, so the host and
// the device cannot disagree.
template <int FMT, int MT, int G, int XR, size_t... P>
static constexpr std::array<bool, kNumPlans> fits_row(std::index_sequence<P...>) {
  return {{MmPlan<FMT, MT, G, (int)P, XR>::FITS...}};
}
template <int FMT, int MT, int G, int XR>
static constexpr std::array<bool, kNumPlans> kFits =
    fits_row<FMT, MT, G, XR>(std::make_index_sequence<kNumPlans>{});

template <int FMT, int MT, int XR = 0>
static bool fits_mt(int g, int plan) {
  if constexpr (FMT == FMT_F8) {
    return g == MM_F8_GROUP && kFits<FMT, MT, MM_F8_GROUP, XR>[plan];
  } else if constexpr (is_asym(FMT)) {
    return g == SB_GROUP && kFits<FMT, MT, SB_GROUP, XR>[plan];
  } else if constexpr (FMT == FMT_S8) {
    return g == 16 ? kFits<FMT, MT, 16, XR>[plan]
                   : (g == 32 ? kFits<FMT, MT, 32, XR>[plan]
                              : (g == 64 && kFits<FMT, MT, 64, XR>[plan]));
  } else {
    return g == 32 ? kFits<FMT, MT, 32, XR>[plan]
                   : (g == 64 ? kFits<FMT, MT, 64, XR>[plan]
                              : (g == 128 && kFits<FMT, MT, 128, XR>[plan]));
  }
}

template <int FMT>
static bool fits_fmt(int mt, int g, int plan, int xr) {
  switch (mt) {
    case 1:
      return xr == 4 ? fits_mt<FMT, 1, 4>(g, plan)
                     : (xr == 8 ? fits_mt<FMT, 1, 8>(g, plan) : fits_mt<FMT, 1>(g, plan));
    case 2: return fits_mt<FMT, 2>(g, plan);
    case 3: return fits_mt<FMT, 3>(g, plan);
    case 4: return fits_mt<FMT, 4>(g, plan);
    default: return false;
  }
}

// xr: x rows staged per round (4 or 8 for one M-tile, 0 for 16 * mt)
static bool plan_fits(int fmt, int mt, int g, int plan, int xr = 0) {
  if (plan < 0 || plan >= kNumPlans) return false;
  if (xr != 0 && (mt != 1 || (xr != 4 && xr != 8))) return false;
  switch (fmt) {
    case FMT_S4: return fits_fmt<FMT_S4>(mt, g, plan, xr);
    case FMT_S8: return fits_fmt<FMT_S8>(mt, g, plan, xr);
    case FMT_A4: return fits_fmt<FMT_A4>(mt, g, plan, xr);
    case FMT_A5: return fits_fmt<FMT_A5>(mt, g, plan, xr);
    case FMT_A6: return fits_fmt<FMT_A6>(mt, g, plan, xr);
    case FMT_F8: return fits_fmt<FMT_F8>(mt, g, plan, xr);
    default: return false;
  }
}

// x rows to stage for M activation rows: only as many as the rows present
// when M <= 8 (fewer copies per round; the copies bound the 16-row plans).
static int x_rows(int M) { return M <= 4 ? 4 : (M <= 8 ? 8 : 0); }

// The plan can run this problem: K is a whole number of rounds, a row's
// scales are whole dwords, and the workgroup's layout fits the LDS.
static bool plan_ok(int fmt, int mt, int group, int K, int plan, int xr = 0) {
  const int rk = round_k(fmt, mt, group, plan);
  return K % rk == 0 && (K / group) % 2 == 0 && plan_fits(fmt, mt, group, plan, xr);
}

size_t gemm_workspace_floats(const GemmCfg& c, int M, int N) {
  return c.splits > 1 ? SPLIT_COUNTERS + (size_t)c.splits * M * N : 0;
}

bool gemm_supports(int fmt, int M, int K, int group) {
  if (fmt == FMT_F8) group = MM_F8_GROUP;
  const int mt = (M + 15) / 16;
  for (int p = 0; p < kNumPlans; p++)
    if (plan_ok(fmt, mt, group, K, p, x_rows(M))) return true;
  return false;
}

GemmCfg choose_gemm(int fmt, int M, int N, int K, int group, int blocks48, bool allow_split) {
  if (fmt == FMT_F8) group = MM_F8_GROUP;
  GemmCfg c{};
  c.mt = (M + 15) / 16;
  c.xr = x_rows(M);
  c.splits = 1;
  const Tuning& tu = tuning();
  // Preference order by row count: with few rows, more K-slices per
  // workgroup keep one workgroup per CU busy; with many rows, 64-row
  // workgroups cut the x staging per row (every workgroup stages all of x,
  // M*K*2 bytes, from L2).  Measured on MI355X for the RWKV-7 shapes, int4
  // g64, weights cold in HBM.
  static const int small_n[] = {1, 0, 6, 3, 8, 4, 5, 7, 2, 9, 10, 11, 12, 13, 14, 15, 16, 17, 18, 19, 20, 21, 22, 23, 24, 25, 26};
  static const int mid_n[] = {3, 8, 4, 1, 0, 6, 5, 7, 2, 9, 10, 11, 12, 13, 14, 15, 16, 17, 18, 19, 20, 21, 22, 23, 24, 25, 26};
  static const int large_n[] = {5, 7, 2, 9, 8, 3, 4, 0, 6, 1, 10, 11, 12, 13, 14, 15, 16, 17, 18, 19, 20, 21, 22, 23, 24, 25, 26};
  // Few rows and long rows (K >= 16384) or a full M-tile stack (M > 48): the
  // x staging of 16-row workgroups dominates, so 64-row workgroups with K
  // split four ways (the last wave to finish a tile adds the partial sums) --
  // at 4096x16384: 16.2 -> 13.6 us (M=16), 23.0 -> 15.9 us (M=32),
  // 45.8 -> 23.7 us (M=64).
  static const int split_n_m16[] = {7, 5, 9, 2, 8, 3, 4, 0, 6, 1, 10, 11, 12, 13, 14, 15, 16, 17, 18, 19, 20, 21, 22, 23, 24, 25, 26};
  static const int split_n[] = {5, 2, 7, 9, 8, 3, 4, 0, 6, 1, 10, 11, 12, 13, 14, 15, 16, 17, 18, 19, 20, 21, 22, 23, 24, 25, 26};
  // 12288..16383 rows (the grouped receptance/key/value launch): 64-row
  // workgroups, about 192 of them, halve the x staging of 32-row ones --
  // three 4096x4096 products in one launch: 11.65 -> 9.18 us (M=16, 32 rows
  // with two workgroups per CU), 15.66 -> 11.18 us (M=32, 64 rows as two
  // 16-row tiles per wave), 25.64 -> 17.37 us (M=64)
  static const int wide_m16[] = {21, 7, 5, 3, 8, 4, 1, 0, 6, 2, 9, 10, 11, 12, 13, 14, 15, 16, 17, 18, 19, 20, 22, 23, 24, 25, 26};
  static const int wide_m32[] = {11, 5, 20, 10, 3, 8, 4, 1, 0, 6, 7, 2, 9, 12, 13, 14, 15, 16, 17, 18, 19, 21, 22, 23, 24, 25, 26};
  static const int wide_m64[] = {5, 10, 2, 3, 8, 4, 1, 0, 6, 7, 9, 11, 12, 13, 14, 15, 16, 17, 18, 19, 20, 21, 22, 23, 24, 25, 26};
  // 16384 rows and more at M = 17..32: two 16-row tiles per wave
  // (16384x4096: 13.28 -> 12.69 us)
  static const int large_n_m32[] = {11, 5, 7, 2, 9, 8, 3, 4, 0, 6, 1, 10, 12, 13, 14, 15, 16, 17, 18, 19, 20, 21, 22, 23, 24, 25, 26};
  const bool split_k = allow_split && N < 8192 && (K >= 16384 || c.mt >= 4);
  const int* order;
  if (split_k)
    order = c.mt == 1 ? split_n_m16 : split_n;
  else if (N >= 16384)
    order = c.mt == 2 ? large_n_m32 : large_n;
  else if (N >= 12288)
    order = c.mt == 1 ? wide_m16 : (c.mt == 2 ? wide_m32 : wide_m64);
  else if (N >= 8192)
    order = mid_n;
  else
    order = small_n;
  c.plan = -1;
  if (tu.gemm_plan > 0 && tu.gemm_plan <= kNumPlans &&
      plan_ok(fmt, c.mt, group, K, tu.gemm_plan - 1, c.xr))
    c.plan = tu.gemm_plan - 1;
  // Measured best arrangements for the RWKV-7 matrices of the 1.5B- and
  // 2.9B-shaped workloads (one product, weights cold; sweeps of every plan x
  // split count at M = 4..32), where the rules below miss by more than 5%.
  struct Tuned {
    int fmt, group, mt, N, K, plan, splits;
  };
  static const Tuned tuned[] = {
      // 4-bit asymmetric, width 2560 (FFN key 10240x2560: 14.85 -> 9.31 us at
      // M = 8, 18.19 -> 10.91 us at M = 32)
      {FMT_A4, 32, 1, 2560, 2560, 18, 1},  {FMT_A4, 32, 2, 2560, 2560, 0, 1},
      {FMT_A4, 32, 1, 10240, 2560, 21, 1}, {FMT_A4, 32, 2, 10240, 2560, 17, 1},
      {FMT_A4, 32, 1, 2560, 10240, 19, 1}, {FMT_A4, 32, 2, 2560, 10240, 17, 4},
      // 8-bit group 16, width 2048 (FFN value 2048x8192: 14.3 -> 11.6 us at M = 32)
      {FMT_S8, 16, 1, 2048, 2048, 19, 1},  {FMT_S8, 16, 2, 2048, 2048, 0, 1},
      {FMT_S8, 16, 1, 8192, 2048, 19, 1},  {FMT_S8, 16, 2, 8192, 2048, 21, 1},
      {FMT_S8, 16, 1, 2048, 8192, 19, 4},  {FMT_S8, 16, 2, 2048, 8192, 21, 4},
      // 4-bit group 64, width 2048 (FFN value 2048x8192: 11.1 -> 10.2 us at M = 32)
      {FMT_S4, 64, 1, 2048, 2048, 19, 1},  {FMT_S4, 64, 1, 8192, 2048, 21, 1},
      {FMT_S4, 64, 1, 2048, 8192, 21, 4},  {FMT_S4, 64, 2, 2048, 8192, 3, 4},
  };
  int tuned_splits = 0;
  if (c.plan < 0 && blocks48 == 0) {
    for (const Tuned& t : tuned) {
      if (t.fmt == fmt && t.group == group && t.mt == c.mt && t.N == N && t.K == K &&
          plan_ok(fmt, c.mt, group, K, t.plan, c.xr)) {
        c.plan = t.plan;
        tuned_splits = t.splits;
        break;
      }
    }
  }
  // 48-row workgroups where they make one wave of 224..256 row blocks (64-row
  // ones leave a quarter of the CUs idle): one 12288x4096 product,
  // 14.1 -> 11.2 us (M=16), 18.3 -> 12.1 us (M=32), 30.1 -> 20.3 us (M=64).
  // Blocks are counted per problem: three 4096-row problems need 258, and
  // the two past one wave nearly double the launch.
  const int b48 = blocks48 > 0 ? blocks48 : (N + 47) / 48;
  if (c.plan < 0 && !split_k && b48 >= 224 && b48 <= 256) {
    const int p48 = c.mt <= 2 ? 17 : 15;
    if (plan_ok(fmt, c.mt, group, K, p48, c.xr)) c.plan = p48;
  }
  for (int i = 0; i < kNumPlans && c.plan < 0; i++)
    if (plan_ok(fmt, c.mt, group, K, order[i], c.xr)) c.plan = order[i];
  // Splits divide K into whole rounds and the partial sums stay under 64 MiB.
  // Automatic only in the case above, enough row blocks x K-ranges for 256
  // CUs (at most 4); RQ_GEMM_SPLITS overrides.
  const int rows = kPlans[c.plan].wr * kPlans[c.plan].nt * 16;
  const int blocks = (N + rows - 1) / rows;
  int want = 1;
  if (split_k && rows == 64 && blocks < 256) want = (256 + blocks - 1) / blocks;
  if (want > 4) want = 4;
  if (tuned_splits > 0) want = tuned_splits;
  if (tu.gemm_splits) want = tu.gemm_splits;
  if (want > MM_MAX_SPLITS) want = MM_MAX_SPLITS;
  if (!allow_split) want = 1;
  const int nr = K / round_k(fmt, c.mt, group, c.plan);
  if (want > nr) want = nr;
  if (want < 1) want = 1;
  int sp = want;
  const size_t part_max = GEMM_WS_MAX_BYTES - SPLIT_COUNTERS * sizeof(unsigned);
  while (sp > 1 && (nr % sp != 0 || (size_t)sp * M * N * 4 > part_max)) sp--;
  // one arrival counter per 16-row tile
  if ((N + 15) / 16 > SPLIT_COUNTERS) sp = 1;
  c.splits = sp;
  return c;
}

}  // namespace rq
