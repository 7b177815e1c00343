// rq_api.hip -- the C interface of librq (declared in include/rq.h): argument
// validation on the host, format dispatch, launch on the caller's stream.
#include <hip/hip_runtime.h>

#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#include <map>
#include <mutex>
#include <utility>

#include "rq.h"
#include "rq_common.h"
#include "rq_internal.h"
#include "rq_probe.h"

namespace rq {

static Tuning g_tuning;
static std::once_flag g_tuning_once;

static int env_or_zero(const char* name) {
  const char* v = getenv(name);
  return v ? atoi(v) : 0;
}

static void read_tuning() {
  g_tuning = Tuning{env_or_zero("RQ_GEMV_LPR"), env_or_zero("RQ_GEMV_CPL"),
                    env_or_zero("RQ_GEMV_NPASS"), env_or_zero("RQ_GEMM_PLAN"),
                    env_or_zero("RQ_GEMM_SPLITS"), env_or_zero("RQ_GEMV_KERNEL")};
}

const Tuning& tuning() {
  std::call_once(g_tuning_once, read_tuning);
  return g_tuning;
}

}  // namespace rq

namespace {

using rq::FMT_A4;
using rq::FMT_A5;
using rq::FMT_A6;
using rq::FMT_F8;
using rq::FMT_S4;
using rq::FMT_S8;

// (layout, bits, group) -> format id, or -1 if unsupported.
int format_of(int layout, int bits, int group) {
  if (layout == RQ_LAYOUT_SYM && bits == 4 && (group == 32 || group == 64 || group == 128))
    return FMT_S4;
  if (layout == RQ_LAYOUT_SYM && bits == 8 && (group == 16 || group == 32 || group == 64))
    return FMT_S8;
  if (layout == RQ_LAYOUT_ASYM_SB && bits == 4 && group == 32) return FMT_A4;
  if (layout == RQ_LAYOUT_ASYM_SB && bits == 5 && group == 32) return FMT_A5;
  if (layout == RQ_LAYOUT_ASYM_SB && bits == 6 && group == 32) return FMT_A6;
  if (layout == RQ_LAYOUT_FP8_TENSOR && bits == 8 && group == 0) return FMT_F8;
  return -1;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

struct Range {
  uintptr_t lo, hi;  // [lo, hi)
};

Range range_of(const void* p, size_t bytes) {
  const uintptr_t a = reinterpret_cast<uintptr_t>(p);
  return Range{a, a + bytes};
}

bool overlaps(Range a, Range b) { return a.lo < b.hi && b.lo < a.hi; }

size_t code_bytes(int N, int K, int bits) { return (size_t)N * K * bits / 8; }
size_t scale_bytes(int N, int K, int group, int layout) {
  if (layout == RQ_LAYOUT_FP8_TENSOR) return 4;  // one binary32
  return layout == RQ_LAYOUT_ASYM_SB ? (size_t)N * (K / 256) * 8
                                     : (size_t)N * (K / group) * 2;
}

// Sizes every kernel takes: whole groups, rows of whole 16-byte chunks,
// operands addressed with 32-bit offsets, whole superblocks.
rq_status check_shape(int N, int K, int bits, int group, int layout) {
  if (N < 1 || K < 1) return RQ_ERR_SHAPE;
  if (group > 0 && (K < group || K % group != 0)) return RQ_ERR_SHAPE;
  if (((size_t)K * bits / 8) % 16 != 0) return RQ_ERR_SHAPE;
  if (code_bytes(N, K, bits) >= ((size_t)1 << 31)) return RQ_ERR_SHAPE;
  if (layout == RQ_LAYOUT_ASYM_SB && K % 256 != 0) return RQ_ERR_SHAPE;
  return RQ_OK;
}

// Shared checks of the weight description.  Returns RQ_OK and the format id.
rq_status check_weights(const void* qweight, const void* scales, const void* zeros, int N,
                        int K, int bits, int group, int layout, int* fmt) {
  if (!qweight || !scales) return RQ_ERR_NULL;
  if (layout != RQ_LAYOUT_SYM && layout != RQ_LAYOUT_ASYM_SB && layout != RQ_LAYOUT_FP8_TENSOR)
    return RQ_ERR_UNSUPPORTED;
  const int f = format_of(layout, bits, group);
  if (f < 0) return RQ_ERR_UNSUPPORTED;
  if (layout == RQ_LAYOUT_ASYM_SB && !zeros) return RQ_ERR_NULL;
  if (layout != RQ_LAYOUT_ASYM_SB && zeros) return RQ_ERR_UNSUPPORTED;
  if (check_shape(N, K, bits, group, layout) != RQ_OK) return RQ_ERR_SHAPE;
  if (!aligned16(qweight) || !aligned16(scales) || (zeros && !aligned16(zeros)))
    return RQ_ERR_ALIGN;
  *fmt = f;
  return RQ_OK;
}

rq_status check_output(const void* out, size_t out_bytes, const void* qweight,
                       const void* scales, const void* zeros, const void* x, int N, int K,
                       int bits, int group, int layout, int M) {
  const Range o = range_of(out, out_bytes);
  if (overlaps(o, range_of(qweight, code_bytes(N, K, bits)))) return RQ_ERR_ALIAS;
  if (overlaps(o, range_of(scales, scale_bytes(N, K, group, layout)))) return RQ_ERR_ALIAS;
  if (zeros && overlaps(o, range_of(zeros, scale_bytes(N, K, group, layout))))
    return RQ_ERR_ALIAS;
  if (x && overlaps(o, range_of(x, (size_t)M * K * 2))) return RQ_ERR_ALIAS;
  return RQ_OK;
}

// The current device must be a gfx950; checked once per device (the result
// is shared; each thread also remembers the last device that passed).
rq_status check_device(int* dev_out) {
  static std::mutex mu;
  static int arch_state[64];  // 0 unknown, 1 ok, 2 unusable
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) {
    (void)hipGetLastError();
    return RQ_ERR_DEVICE;
  }
  thread_local int last_ok_dev = -1;
  if (dev == last_ok_dev) {
    *dev_out = dev;
    return RQ_OK;
  }
  std::lock_guard<std::mutex> lk(mu);
  if (arch_state[dev] == 0) {
    hipDeviceProp_t prop;
    if (hipGetDeviceProperties(&prop, dev) != hipSuccess) {
      (void)hipGetLastError();
      return RQ_ERR_DEVICE;
    }
    arch_state[dev] = (strncmp(prop.gcnArchName, "gfx950", 6) == 0) ? 1 : 2;
  }
  if (arch_state[dev] != 1) return RQ_ERR_DEVICE;
  last_ok_dev = dev;
  *dev_out = dev;
  return RQ_OK;
}

// Split-K scratch of rq_gemm_smallm_noalloc: a fixed device array (each GPU
// the library runs on holds its own copy until the process ends), so that
// entry point never allocates.  It holds the split-K arrival counters (zero
// at load, and every launch leaves them zero) and partial sums for every
// split the automatic choice makes (at most 4 K-ranges x 64 rows x 8191
// outputs of binary32).
constexpr size_t SCRATCH_BYTES = (size_t)RQ_NOALLOC_SCRATCH_BYTES;
static __device__ __align__(256) float scratch[SCRATCH_BYTES / sizeof(float)];

// The device address of this GPU's `scratch`, looked up once per device with
// that device current (host code must never pass the array's own name: on the
// host it is only a stand-in).  NULL if the lookup fails.
float* device_scratch(int dev) {
  static std::mutex mu;
  static float* addr[64];
  static bool looked[64];
  std::lock_guard<std::mutex> lk(mu);
  if (!looked[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess) {
      (void)hipGetLastError();
      return nullptr;
    }
    addr[dev] = static_cast<float*>(p);
    looked[dev] = true;
  }
  return addr[dev];
}

rq_status check_product(const void* qweight, const void* scales, const void* zeros,
                        const void* x, float* y, int M, int N, int K, int bits, int group,
                        int layout, int* fmt) {
  if (!x || !y) return RQ_ERR_NULL;
  rq_status st = check_weights(qweight, scales, zeros, N, K, bits, group, layout, fmt);
  if (st != RQ_OK) return st;
  if (M < 1 || M > RQ_MAX_M) return RQ_ERR_SHAPE;
  if ((size_t)M * K * 2 >= ((size_t)1 << 31) || (size_t)M * N * 4 >= ((size_t)1 << 31))
    return RQ_ERR_SHAPE;
  if (!aligned16(x) || !aligned16(y)) return RQ_ERR_ALIGN;
  return check_output(y, (size_t)M * N * 4, qweight, scales, zeros, x, N, K, bits, group,
                      layout, M);
}

enum Kernel { KERN_VECTOR, KERN_DECODE_MFMA, KERN_SMALLM_MFMA };

// The kernel rq_gemv and rq_gemv_batched use for M activation rows (N: rows of
// the launch).  Measured on MI355X, weights cold in HBM, int4 g64 / int8 g16 /
// asym4 / FP8 / 5- and 6-bit codes at widths 2048..4096 and K up to 16384:
//  * M >= 3: the small-batch matrix-core kernel (4 or 8 x rows staged for
//    M <= 4 or 8, else 16 per M-tile) beats the vector-unit passes of eight
//    rows by up to 11x (int4 4096x4096 M = 8: 11.5 -> 5.3 us; 2560x10240
//    asymmetric M = 8: 65.7 -> 11.0 us) and, at M = 3..4, the decode kernel
//    (int8 8192x2048 M = 4: 7.5 -> 6.8 us; asymmetric 2560x2560 M = 4:
//    6.1 -> 5.2 us; 5-bit 16384x4096 M = 4: 20.2 -> 19.5 us), except for
//    the measured shapes below, where the decode kernel or the vector units
//    win at M = 3..4 (these calls keep K whole, so few, long rows or many
//    short ones leave the small-batch kernel with too little work per
//    workgroup).
//  * M <= 2: the vector-unit kernel, unless none of its tuned launch shapes
//    splits the row (the generic kernel: FP8 4096x16384 at M = 2 takes
//    52.1 us there, 18.0 us on the small-batch kernel).  Then the decode
//    kernel for int4 and asymmetric 4-bit (2048x65536 at M = 1: 32.3 and
//    43.2 us, against 36.4 and 58.7 us on the small-batch kernel), the
//    small-batch kernel otherwise (int8 4096x32768 at M = 1: 37.0 against
//    42.9 us).
// *gc receives the vector-unit launch shape when that kernel is chosen.  The
// common decode case (M <= 2, a tuned vector-unit shape) returns after one
// launch-shape search, so stream-mode callers pay little host time per call.
// RWKV-7 matrices where, at M = 3..4, another kernel beats the small-batch
// kernel with K kept whole (one product, weights cold, launches replayed from
// a graph).  N is the launch's row count, so a grouped launch of several
// problems does not match.
//  * the matrix-core decode kernel: 4-bit asymmetric 10240x2560, the
//    2.9B-shaped FFN key (10.36-10.39 -> 8.74-8.97 us);
//  * the vector units in one pass of 4 rows: int4 g64 2048x8192, the
//    1.5B-shaped FFN value (decode kernel 7.19-7.39, small-batch 9.34-9.43,
//    vector units 6.36-6.76 us; the 24-layer step at M = 4 0.581-0.584 ->
//    0.563 ms).  (int8 g16 2048x2048, 5.1 -> 4.7 us alone, left the int8
//    step no faster: 0.755-0.759 -> 0.763 ms.)
struct MvShape {
  int fmt, group, N, K;
};
constexpr MvShape kDecodeWins[] = {{FMT_A4, 32, 10240, 2560}};
constexpr MvShape kVectorWins[] = {{FMT_S4, 64, 2048, 8192}};

template <size_t n>
bool listed(const MvShape (&tab)[n], int fmt, int M, int N, int K, int group) {
  if (M < 3 || M > 4) return false;
  for (const MvShape& s : tab)
    if (s.fmt == fmt && s.group == group && s.N == N && s.K == K) return true;
  return false;
}

Kernel pick_kernel(int fmt, int M, int N, int K, int group, rq::GemvCfg* gc) {
  int t = rq::tuning().gemv_kernel;
  if (t < 0 || t > 3) t = 0;  // unknown override values: the automatic choice
  if (t == 1 || (t == 0 && M <= 2)) {
    *gc = rq::choose_gemv(fmt, M, N, K);
    if (t == 1 || gc->lpr != 0) return KERN_VECTOR;
  }
  const bool mv = rq::mv_supports(fmt, M, K, group);
  const bool mm = rq::gemm_supports(fmt, M, K, group);
  Kernel k;
  if (t == 2) {
    k = mv ? KERN_DECODE_MFMA : KERN_VECTOR;
  } else if (t == 3) {
    k = mm ? KERN_SMALLM_MFMA : KERN_VECTOR;
  } else if (M >= 3) {
    if (listed(kVectorWins, fmt, M, N, K, group)) {
      *gc = rq::choose_gemv(fmt, M, N, K);
      if (gc->lpr != 0) return KERN_VECTOR;
    }
    if (mv && listed(kDecodeWins, fmt, M, N, K, group)) return KERN_DECODE_MFMA;
    k = mm ? KERN_SMALLM_MFMA : (mv ? KERN_DECODE_MFMA : KERN_VECTOR);
  } else {  // M <= 2 on the generic vector-unit kernel
    if (mv && (fmt == FMT_S4 || fmt == FMT_A4 || !mm)) return KERN_DECODE_MFMA;
    k = mm ? KERN_SMALLM_MFMA : KERN_VECTOR;
  }
  if (k == KERN_VECTOR) *gc = rq::choose_gemv(fmt, M, N, K);
  return k;
}

}  // namespace

extern "C" {

rq_status rq_dequant(const void* qweight, const void* scales, const void* zeros,
                     void* out, int N, int K, int bits, int group, int layout,
                     int out_kind, void* stream) {
  if (!out) return RQ_ERR_NULL;
  int fmt = -1;
  rq_status st = check_weights(qweight, scales, zeros, N, K, bits, group, layout, &fmt);
  if (st != RQ_OK) return st;
  if (out_kind != RQ_OUT_F32 && out_kind != RQ_OUT_CODES_I8) return RQ_ERR_UNSUPPORTED;
  if (out_kind == RQ_OUT_CODES_I8 && fmt == FMT_F8) return RQ_ERR_UNSUPPORTED;
  if (!aligned16(out)) return RQ_ERR_ALIGN;
  const size_t ob = (size_t)N * K * (out_kind == RQ_OUT_F32 ? 4 : 1);
  st = check_output(out, ob, qweight, scales, zeros, nullptr, N, K, bits, group, layout, 0);
  if (st != RQ_OK) return st;
  int dev;
  st = check_device(&dev);
  if (st != RQ_OK) return st;
  const hipError_t e = rq::launch_dequant(qweight, scales, zeros, out, N, K, group, fmt,
                                          out_kind, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? RQ_OK : RQ_ERR_LAUNCH;
}

rq_status rq_gemv(const void* qweight, const void* scales, const void* zeros,
                  const void* x, float* y, int M, int N, int K, int bits, int group,
                  int layout, void* stream) {
  int fmt = -1;
  rq_status st =
      check_product(qweight, scales, zeros, x, y, M, N, K, bits, group, layout, &fmt);
  if (st != RQ_OK) return st;
  int dev;
  st = check_device(&dev);
  if (st != RQ_OK) return st;
  rq::Problem p{qweight, scales, zeros, x, y, M, N, K, group, fmt};
  const rq::Problem* one = &p;
  const hipStream_t s = static_cast<hipStream_t>(stream);
  hipError_t e;
  rq::GemvCfg gc{};
  switch (pick_kernel(fmt, M, N, K, group, &gc)) {
    case KERN_DECODE_MFMA: e = rq::launch_mv_many(&one, 1, s); break;
    case KERN_SMALLM_MFMA:
      // K kept whole: this entry point never allocates
      e = rq::launch_gemm(p, rq::choose_gemm(fmt, M, N, K, group, 0, false), nullptr, s);
      break;
    default: e = rq::launch_gemv(p, gc, s); break;
  }
  return e == hipSuccess ? RQ_OK : RQ_ERR_LAUNCH;
}

rq_status rq_gemv_batched(const rq_problem* problems, int count, int M, int bits,
                          int group, int layout, void* stream) {
  if (!problems) return RQ_ERR_NULL;
  if (count < 1 || count > RQ_MAX_BATCH) return RQ_ERR_SHAPE;
  int fmt = -1;
  for (int i = 0; i < count; i++) {
    const rq_problem& q = problems[i];
    rq_status st = check_product(q.qweight, q.scales, q.zeros, q.x, q.y, M, q.N, q.K, bits,
                                 group, layout, &fmt);
    if (st != RQ_OK) return st;
  }
  // outputs against the other problems' inputs and outputs
  for (int i = 0; i < count; i++) {
    const rq_problem& a = problems[i];
    for (int j = 0; j < count; j++) {
      if (j == i) continue;
      const rq_problem& b = problems[j];
      rq_status st = check_output(a.y, (size_t)M * a.N * 4, b.qweight, b.scales, b.zeros,
                                  b.x, b.N, b.K, bits, group, layout, M);
      if (st != RQ_OK) return st;
      if (overlaps(range_of(a.y, (size_t)M * a.N * 4), range_of(b.y, (size_t)M * b.N * 4)))
        return RQ_ERR_ALIAS;
    }
  }
  int dev;
  rq_status st = check_device(&dev);
  if (st != RQ_OK) return st;
  // group by K (launch shapes depend on K), keeping the caller's order within
  rq::Problem pb[RQ_MAX_BATCH];
  const rq::Problem* order[RQ_MAX_BATCH];
  bool done[RQ_MAX_BATCH] = {false};
  for (int i = 0; i < count; i++) {
    const rq_problem& q = problems[i];
    pb[i] = rq::Problem{q.qweight, q.scales, q.zeros, q.x, q.y, M, q.N, q.K, group, fmt};
  }
  const hipStream_t s = static_cast<hipStream_t>(stream);
  for (int i = 0; i < count; i++) {
    if (done[i]) continue;
    int n = 0, rows = 0, blocks48 = 0;
    for (int j = i; j < count; j++) {
      if (!done[j] && pb[j].K == pb[i].K) {
        order[n++] = &pb[j];
        rows += pb[j].N;
        blocks48 += (pb[j].N + 47) / 48;
        done[j] = true;
      }
    }
    hipError_t e;
    rq::GemvCfg gc{};
    switch (pick_kernel(fmt, M, rows, pb[i].K, group, &gc)) {
      case KERN_SMALLM_MFMA:
        e = rq::launch_gemm_many(
            order, n, rq::choose_gemm(fmt, M, rows, pb[i].K, group, blocks48, false), nullptr,
            s);
        break;
      case KERN_DECODE_MFMA: e = rq::launch_mv_many(order, n, s); break;
      default: e = rq::launch_gemv_many(order, n, gc, s); break;
    }
    if (e != hipSuccess) return RQ_ERR_LAUNCH;
  }
  return RQ_OK;
}

// The arrangement rq_gemm_smallm_ws would launch and the workspace bytes it
// needs (0 when K is kept whole).
rq::GemmCfg smallm_cfg(int fmt, int M, int N, int K, int group, size_t* need) {
  const rq::GemmCfg c = rq::choose_gemm(fmt, M, N, K, group);
  *need = rq::gemm_workspace_floats(c, M, N) * sizeof(float);
  return c;
}

rq_status rq_gemm_smallm(const void* qweight, const void* scales, const void* zeros,
                         const void* x, float* y, int M, int N, int K, int bits,
                         int group, int layout, void* stream) {
  // no workspace: K kept whole
  return rq_gemm_smallm_ws(qweight, scales, zeros, x, y, M, N, K, bits, group, layout,
                           nullptr, 0, stream);
}

rq_status rq_gemm_smallm_workspace_size(int M, int N, int K, int bits, int group, int layout,
                                        size_t* bytes) {
  if (!bytes) return RQ_ERR_NULL;
  *bytes = 0;
  const int fmt = format_of(layout, bits, group);
  if (fmt < 0) return RQ_ERR_UNSUPPORTED;
  if (M < 1 || M > RQ_MAX_M || check_shape(N, K, bits, group, layout) != RQ_OK)
    return RQ_ERR_SHAPE;
  if (rq::gemm_supports(fmt, M, K, group)) smallm_cfg(fmt, M, N, K, group, bytes);
  return RQ_OK;
}

rq_status rq_gemm_smallm_ws(const void* qweight, const void* scales, const void* zeros,
                            const void* x, float* y, int M, int N, int K, int bits,
                            int group, int layout, void* workspace, size_t workspace_bytes,
                            void* stream) {
  int fmt = -1;
  rq_status st =
      check_product(qweight, scales, zeros, x, y, M, N, K, bits, group, layout, &fmt);
  if (st != RQ_OK) return st;
  const bool has_ws = workspace != nullptr;
  if (has_ws && !aligned16(workspace)) return RQ_ERR_ALIGN;
  // host-only choice first, so a workspace that is too small or overlaps an
  // operand enqueues nothing
  const bool mfma = rq::gemm_supports(fmt, M, K, group);
  size_t need = 0;
  rq::GemmCfg c{};
  if (mfma) c = smallm_cfg(fmt, M, N, K, group, &need);
  float* ws = nullptr;
  if (need > 0) {
    if (!has_ws) {
      c = rq::choose_gemm(fmt, M, N, K, group, 0, false);  // K kept whole
    } else {
      if (workspace_bytes < need) return RQ_ERR_SCRATCH;
      // the bytes this call uses against every input and the output
      st = check_output(workspace, need, qweight, scales, zeros, x, N, K, bits, group, layout,
                        M);
      if (st != RQ_OK) return st;
      if (overlaps(range_of(workspace, need), range_of(y, (size_t)M * N * 4)))
        return RQ_ERR_ALIAS;
      ws = static_cast<float*>(workspace);
    }
  }
  int dev;
  st = check_device(&dev);
  if (st != RQ_OK) return st;
  const hipStream_t s = static_cast<hipStream_t>(stream);
  rq::Problem p{qweight, scales, zeros, x, y, M, N, K, group, fmt};
  if (!mfma) {
    // K is not a whole number of the matrix-core kernel's chunks
    const rq::GemvCfg gc = rq::choose_gemv(fmt, M, N, K);
    return rq::launch_gemv(p, gc, s) == hipSuccess ? RQ_OK : RQ_ERR_LAUNCH;
  }
  const hipError_t e = rq::launch_gemm(p, c, ws, s);
  return e == hipSuccess ? RQ_OK : RQ_ERR_LAUNCH;
}

rq_status rq_gemm_smallm_noalloc(const void* qweight, const void* scales, const void* zeros,
                                 const void* x, float* y, int M, int N, int K, int bits,
                                 int group, int layout, void* stream) {
  int fmt = -1;
  rq_status st =
      check_product(qweight, scales, zeros, x, y, M, N, K, bits, group, layout, &fmt);
  if (st != RQ_OK) return st;
  int dev;
  st = check_device(&dev);
  if (st != RQ_OK) return st;
  const hipStream_t s = static_cast<hipStream_t>(stream);
  rq::Problem p{qweight, scales, zeros, x, y, M, N, K, group, fmt};
  if (!rq::gemm_supports(fmt, M, K, group)) {
    const rq::GemvCfg c = rq::choose_gemv(fmt, M, N, K);
    return rq::launch_gemv(p, c, s) == hipSuccess ? RQ_OK : RQ_ERR_LAUNCH;
  }
  // the arrangement rq_gemm_smallm_ws chooses, partial sums in `scratch`
  const rq::GemmCfg c = rq::choose_gemm(fmt, M, N, K, group);
  float* ws = nullptr;
  if (c.splits > 1) {
    if (rq::gemm_workspace_floats(c, M, N) * sizeof(float) > SCRATCH_BYTES)
      return RQ_ERR_SCRATCH;
    ws = device_scratch(dev);
    if (!ws) return RQ_ERR_DEVICE;
  }
  const hipError_t e = rq::launch_gemm(p, c, ws, s);
  return e == hipSuccess ? RQ_OK : RQ_ERR_LAUNCH;
}

const char* rq_status_string(int status) {
  switch (status) {
    case RQ_OK: return "success";
    case RQ_ERR_NULL: return "a required pointer is NULL";
    case RQ_ERR_SHAPE: return "M, N, K or group violate the shape rules";
    case RQ_ERR_UNSUPPORTED: return "unsupported layout, bits, group or output kind";
    case RQ_ERR_ALIGN: return "a pointer is not 16-byte aligned";
    case RQ_ERR_LAUNCH: return "the kernel launch failed";
    case RQ_ERR_ALIAS: return "an output overlaps an input";
    case RQ_ERR_DEVICE: return "no usable gfx950 device";
    case RQ_ERR_SCRATCH: return "the call needs more scratch or workspace than it was given";
    default: return "unknown status";
  }
}

int rq_version(void) { return (1 << 16) | 1; }

int rq_gemm_config(int M, int N, int K, int bits, int group, int layout, int allow_split,
                   int* plan, int* splits) {
  if (!plan || !splits) return RQ_ERR_NULL;
  const int fmt = format_of(layout, bits, group);
  if (fmt < 0) return RQ_ERR_UNSUPPORTED;
  if (M < 1 || M > RQ_MAX_M || N < 1 || K < 1) return RQ_ERR_SHAPE;
  if (group > 0 && K % group != 0) return RQ_ERR_SHAPE;
  if (!rq::gemm_supports(fmt, M, K, group)) return RQ_ERR_UNSUPPORTED;
  const rq::GemmCfg c = rq::choose_gemm(fmt, M, N, K, group, 0, allow_split != 0);
  *plan = c.plan + 1;
  *splits = c.splits;
  return RQ_OK;
}

int rq_gemv_config(int M, int N, int K, int bits, int group, int layout, int* kernel,
                   int* lpr, int* cpl, int* npass) {
  if (!kernel || !lpr || !cpl || !npass) return RQ_ERR_NULL;
  const int fmt = format_of(layout, bits, group);
  if (fmt < 0) return RQ_ERR_UNSUPPORTED;
  if (M < 1 || M > RQ_MAX_M || check_shape(N, K, bits, group, layout) != RQ_OK)
    return RQ_ERR_SHAPE;
  rq::GemvCfg gc{};
  const Kernel k = pick_kernel(fmt, M, N, K, group, &gc);
  *kernel = (int)k;
  *lpr = k == KERN_VECTOR ? gc.lpr : 0;
  *cpl = k == KERN_VECTOR ? gc.cpl : 0;
  *npass = k == KERN_VECTOR ? gc.npass : 0;
  return RQ_OK;
}

int rq_tuning_reload(void) {
  rq::tuning();  // make sure the one-time read has happened
  rq::read_tuning();
  return RQ_OK;
}

}  // extern "C"
