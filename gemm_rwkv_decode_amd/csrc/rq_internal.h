// rq_internal.h -- host-side launchers shared between the translation units
// of librq.  Arguments have been validated by rq_api.hip before these run.
#pragma once

#include <hip/hip_runtime.h>

namespace rq {

// Launch-shape overrides for measurements and tests, read from the
// environment once (RQ_GEMV_LPR, RQ_GEMV_CPL, RQ_GEMV_NPASS, RQ_GEMM_PLAN,
// RQ_GEMM_SPLITS, RQ_GEMV_KERNEL; 0 = no override) and again on
// rq_tuning_reload().
struct Tuning {
  int gemv_lpr, gemv_cpl, gemv_npass, gemm_plan, gemm_splits;
  // kernel of rq_gemv and rq_gemv_batched: 0 automatic, 1 vector-unit
  // kernel, 2 matrix-core decode kernel (M <= 4), 3 matrix-core small-batch
  // kernel; 2 and 3 fall back to 1 where they cannot take the shape
  int gemv_kernel;
};
const Tuning& tuning();

struct Problem {
  const void* qweight;
  const void* scales;
  const void* zeros;
  const void* x;  // binary16 [M][K]
  float* y;       // [M][N]
  int M, N, K, group;
  int fmt;        // Fmt
};

// Tuning knobs of one GEMV launch (chosen by choose_gemv unless overridden).
struct GemvCfg {
  int lpr;    // lanes per row (power of two, 8..64); 0 = generic kernel
  int cpl;    // 16-byte chunks per lane per row (1 or 2)
  int npass;  // row passes per workgroup (rows per workgroup = npass*64/lpr)
  int mt;     // activation rows per launch (1, 2, 4, 8)
};

// Problems per GEMV launch of a batch.
constexpr int GEMV_BATCH = 16;

// N is the largest row count of the problems sharing the launch.
GemvCfg choose_gemv(int fmt, int M, int N, int K);
hipError_t launch_gemv(const Problem& p, const GemvCfg& c, hipStream_t s);
// count problems sharing fmt, K, group and M
hipError_t launch_gemv_many(const Problem* const* p, int count, const GemvCfg& c,
                            hipStream_t s);

// Matrix-core kernel for M = 1..4 (rq_mv.hip): problems sharing fmt, K,
// group and M, up to MV_BATCH per launch.
constexpr int MV_BATCH = 16;
bool mv_supports(int fmt, int M, int K, int group);
hipError_t launch_mv_many(const Problem* const* p, int count, hipStream_t s);

struct GemmCfg {
  int mt;      // 16-row M-tiles (1..4)
  int plan;    // workgroup arrangement (index into the kernel's plan table)
  int splits;  // K split across workgroups
  int xr;      // x rows staged per round: 4 or 8 for M <= 4 or 8, else 0 (16 * mt)
};

// The matrix-core kernel needs K to be a whole number of its rounds.
bool gemm_supports(int fmt, int M, int K, int group);
// N: rows of all problems of the launch; blocks48: their 48-row blocks, each
// problem rounded up (0: one problem of N rows).  allow_split = false keeps K
// whole (no workspace) and picks the plan for that.
GemmCfg choose_gemm(int fmt, int M, int N, int K, int group, int blocks48 = 0,
                    bool allow_split = true);
// ws: workspace of gemm_workspace_floats() floats (unused when splits == 1):
// SPLIT_COUNTERS arrival counters, zero between launches, then the partial
// sums.
hipError_t launch_gemm(const Problem& p, const GemmCfg& c, float* ws, hipStream_t s);
// count problems sharing fmt, M, K and group, MM_BATCH per launch (splits must
// be 1 when count > 1)
constexpr int MM_BATCH = 8;
hipError_t launch_gemm_many(const Problem* const* p, int count, const GemmCfg& c, float* ws,
                            hipStream_t s);
size_t gemm_workspace_floats(const GemmCfg& c, int M, int N);
// Split-K arrival counters at the front of a workspace: one per 16-row tile,
// so K is split only for N <= 16 * SPLIT_COUNTERS.
constexpr int SPLIT_COUNTERS = 16384;
// Largest split-K workspace choose_gemm asks for: the counters and at most
// GEMM_WS_MAX_BYTES - 64 KiB of partial sums (splits * M * N floats).
constexpr size_t GEMM_WS_MAX_BYTES = (size_t)64 << 20;

hipError_t launch_dequant(const void* qweight, const void* scales, const void* zeros,
                          void* out, int N, int K, int group, int fmt, int out_kind,
                          hipStream_t s);

}  // namespace rq
