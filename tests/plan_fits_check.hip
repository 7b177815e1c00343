// Host-only check of the matrix-core kernel's plan table (built and run by
// tests/test_plan_table.py; no GPU code is executed).
//
// For every format, M-tile count, group size and plan it compares three
// things that must agree:
//   * plan_fits() -- what the host's chooser in rq_gemm.hip accepts;
//   * Mm<...>::FITS -- what the kernel instance accepts (a plan that does not
//     fit is never launched: launch_s returns an error instead);
//   * an independent restatement of the conditions below (LDS bytes of the
//     two rings and of the K-slice reduction, registers, copy layout).
// It prints one line per fitting combination and exits non-zero on the first
// disagreement.
#include "rq_gemm_plan.h"

#include <cstdio>

namespace rq {
// The chooser reads the launch-shape overrides; none here.
const Tuning& tuning() {
  static Tuning t{};
  return t;
}
}  // namespace rq

using namespace rq;

// Restated fit conditions of one (format, M-tiles, group, plan, x rows).
static bool restated_fits(int fmt, int mt, int g, const Plan& q, int xr) {
  const int xrows = xr > 0 ? xr : 16 * mt;  // activation rows staged per round
  const int kc = mm_kc(fmt, mt, q.wk, g, q.rd);
  const int round = q.wk * kc;
  const int rows = 16 * q.nt * q.wr;
  const int waves = q.wr * q.wk;
  const int threads = 64 * (waves + MM_XP + MM_CP);
  const int dx = mm_xdepth(fmt, mt, g, q.wr, q.wk, q.nt, q.rd, q.occ, xr);
  const int dc = mm_cdepth(fmt, mt, g, q.wr, q.wk, q.nt, q.rd, q.occ, xr);
  const int lds = LDS_LIMIT / q.occ;  // two workgroups per CU share its LDS
  const int row_bytes = mm_byte(fmt) ? round : round / 2;  // code bytes per row and round
  const int pieces = row_bytes / 16;
  // binary32 partial tiles of every multiplying wave: 64 lanes x 4 floats per tile
  const long red_bytes = q.wk > 1 ? (long)waves * 64 * q.nt * mt * 4 * 4 : 0;
  if (kc % g != 0 || kc / g < 1 || kc / g > 8) return false;
  if (threads > 1024) return false;  // a workgroup holds at most 16 waves
  if (q.nt * mt * q.occ > (threads > 512 ? 4 : 8)) return false;
  if (is_asym(fmt) && (SUPERBLOCK % kc != 0 || round % SUPERBLOCK != 0)) return false;
  if (!is_asym(fmt) && (round / g) % 2 != 0) return false;
  if (pieces < 8 || (pieces & (pieces - 1)) != 0) return false;
  if ((rows * pieces) % 64 != 0) return false;
  const long ring = (long)(dx + 1) * xrows * (round + 8) * 2 +
                    (long)(dc + 1) * mm_cslot(fmt, mt, g, q.wr, q.wk, q.nt, q.rd);
  return dx >= 1 && dc >= 1 && ring <= lds && red_bytes <= lds;
}

template <int FMT, int MT, int G, int XR = 0, int P = 0>
static int check_plans(const char* name, int* fitting) {
  if constexpr (P >= kNumPlans) {
    return 0;
  } else {
    using S = MmPlan<FMT, MT, G, P, XR>;
    const bool host = plan_fits(FMT, MT, G, P, XR);
    const bool again = restated_fits(FMT, MT, G, kPlans[P], XR);
    if (host != S::FITS || again != S::FITS) {
      printf("MISMATCH %s mt=%d xr=%d g=%d plan=%d: kernel %d host %d restated %d\n", name,
             MT, XR, G, P, (int)S::FITS, (int)host, (int)again);
      return 1;
    }
    if (S::FITS) {
      printf("fits %s mt=%d xr=%d g=%d plan=%d lds=%d red=%d\n", name, MT, XR, G, P,
             S::LDS_BYTES, S::RED * 4);
      ++*fitting;
    }
    return check_plans<FMT, MT, G, XR, P + 1>(name, fitting);
  }
}

template <int FMT, int G>
static int check_groups(const char* name, int* fitting) {
  return check_plans<FMT, 1, G, 4>(name, fitting) + check_plans<FMT, 1, G, 8>(name, fitting) +
         check_plans<FMT, 1, G>(name, fitting) + check_plans<FMT, 2, G>(name, fitting) +
         check_plans<FMT, 3, G>(name, fitting) + check_plans<FMT, 4, G>(name, fitting);
}

int main() {
  int fitting = 0, bad = 0;
  bad += check_groups<FMT_S4, 32>("int4", &fitting);
  bad += check_groups<FMT_S4, 64>("int4", &fitting);
  bad += check_groups<FMT_S4, 128>("int4", &fitting);
  bad += check_groups<FMT_S8, 16>("int8", &fitting);
  bad += check_groups<FMT_S8, 32>("int8", &fitting);
  bad += check_groups<FMT_S8, 64>("int8", &fitting);
  bad += check_groups<FMT_A4, 32>("asym4", &fitting);
  bad += check_groups<FMT_A5, 32>("asym5", &fitting);
  bad += check_groups<FMT_A6, 32>("asym6", &fitting);
  bad += check_groups<FMT_F8, MM_F8_GROUP>("fp8", &fitting);
  // group sizes a format does not have are never accepted
  if (plan_fits(FMT_S4, 1, 16, 0) || plan_fits(FMT_A4, 1, 64, 0) || plan_fits(FMT_F8, 1, 32, 0))
    bad++;
  // nor x-row counts other than 4 and 8 for one M-tile
  if (plan_fits(FMT_S4, 2, 64, 2, 8) || plan_fits(FMT_S4, 1, 64, 2, 12)) bad++;
  printf("plans=%d fitting=%d mismatches=%d\n", kNumPlans, fitting, bad);
  return bad ? 1 : 0;
}
