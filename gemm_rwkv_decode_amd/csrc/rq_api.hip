// rq_api.hip -- the C interface of librq (declared in include/rq.h): argument
// validation on the host, format dispatch, launch on the caller's stream.
#include <hip/hip_runtime.h>

#include <stdint.h>
#include <string.h>

#include <map>
#include <mutex>
#include <utility>

#include "rq.h"
#include "rq_common.h"
#include "rq_internal.h"

namespace {

using rq::FMT_A4;
using rq::FMT_S4;
using rq::FMT_S8;

// (layout, bits, group) -> format id, or -1 if unsupported.
int format_of(int layout, int bits, int group) {
  if (layout == RQ_LAYOUT_SYM && bits == 4 && (group == 32 || group == 64 || group == 128))
    return FMT_S4;
  if (layout == RQ_LAYOUT_SYM && bits == 8 && (group == 16 || group == 32 || group == 64))
    return FMT_S8;
  if (layout == RQ_LAYOUT_ASYM_SB && bits == 4 && group == 32) return FMT_A4;
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
  return layout == RQ_LAYOUT_ASYM_SB ? (size_t)N * (K / 256) * 8
                                     : (size_t)N * (K / group) * 2;
}

// Shared checks of the weight description.  Returns RQ_OK and the format id.
rq_status check_weights(const void* qweight, const void* scales, const void* zeros, int N,
                        int K, int bits, int group, int layout, int* fmt) {
  if (!qweight || !scales) return RQ_ERR_NULL;
  if (layout != RQ_LAYOUT_SYM && layout != RQ_LAYOUT_ASYM_SB) return RQ_ERR_UNSUPPORTED;
  const int f = format_of(layout, bits, group);
  if (f < 0) return RQ_ERR_UNSUPPORTED;
  if (layout == RQ_LAYOUT_ASYM_SB && !zeros) return RQ_ERR_NULL;
  if (layout == RQ_LAYOUT_SYM && zeros) return RQ_ERR_UNSUPPORTED;
  if (N < 1 || K < group || K % group != 0) return RQ_ERR_SHAPE;
  if (((size_t)K * bits / 8) % 16 != 0) return RQ_ERR_SHAPE;
  if (layout == RQ_LAYOUT_ASYM_SB && K % 256 != 0) return RQ_ERR_SHAPE;
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

// The current device must be a gfx950; checked once per device.
rq_status check_device(int* dev_out) {
  static std::mutex mu;
  static int verdict[64];  // 0 unknown, 1 ok, 2 unusable
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) {
    (void)hipGetLastError();
    return RQ_ERR_DEVICE;
  }
  std::lock_guard<std::mutex> lk(mu);
  if (verdict[dev] == 0) {
    hipDeviceProp_t prop;
    if (hipGetDeviceProperties(&prop, dev) != hipSuccess) {
      (void)hipGetLastError();
      return RQ_ERR_DEVICE;
    }
    verdict[dev] = (strncmp(prop.gcnArchName, "gfx950", 6) == 0) ? 1 : 2;
  }
  if (verdict[dev] != 1) return RQ_ERR_DEVICE;
  *dev_out = dev;
  return RQ_OK;
}

// Split-K workspace: one per (device, stream), grown on demand, never freed.
struct Workspace {
  float* partial = nullptr;
  size_t floats = 0;
  unsigned* counters = nullptr;
  size_t ncounters = 0;
};

rq_status get_workspace(int dev, hipStream_t stream, size_t floats, size_t ncounters,
                        Workspace* out) {
  static std::mutex mu;
  static std::map<std::pair<int, hipStream_t>, Workspace> cache;
  std::lock_guard<std::mutex> lk(mu);
  Workspace& w = cache[std::make_pair(dev, stream)];
  if (w.floats >= floats && w.ncounters >= ncounters) {
    *out = w;
    return RQ_OK;
  }
  hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
  if (stream && hipStreamIsCapturing(stream, &cs) == hipSuccess &&
      cs != hipStreamCaptureStatusNone)
    return RQ_ERR_DEVICE;  // cannot allocate while a graph is being captured
  const size_t want_f = floats > ((size_t)4 << 20) ? floats : ((size_t)4 << 20);
  const size_t want_c = ncounters > 65536 ? ncounters : 65536;
  if (hipDeviceSynchronize() != hipSuccess) return RQ_ERR_DEVICE;
  if (w.partial) (void)hipFree(w.partial);
  if (w.counters) (void)hipFree(w.counters);
  w = Workspace{};
  float* p = nullptr;
  unsigned* c = nullptr;
  if (hipMalloc(&p, want_f * sizeof(float)) != hipSuccess) {
    (void)hipGetLastError();
    return RQ_ERR_DEVICE;
  }
  if (hipMalloc(&c, want_c * sizeof(unsigned)) != hipSuccess ||
      hipMemset(c, 0, want_c * sizeof(unsigned)) != hipSuccess ||
      hipDeviceSynchronize() != hipSuccess) {
    (void)hipGetLastError();
    (void)hipFree(p);
    if (c) (void)hipFree(c);
    return RQ_ERR_DEVICE;
  }
  w.partial = p;
  w.floats = want_f;
  w.counters = c;
  w.ncounters = want_c;
  *out = w;
  return RQ_OK;
}

rq_status check_product(const void* qweight, const void* scales, const void* zeros,
                        const void* x, float* y, int M, int N, int K, int bits, int group,
                        int layout, int* fmt) {
  if (!x || !y) return RQ_ERR_NULL;
  rq_status st = check_weights(qweight, scales, zeros, N, K, bits, group, layout, fmt);
  if (st != RQ_OK) return st;
  if (M < 1 || M > RQ_MAX_M) return RQ_ERR_SHAPE;
  if (!aligned16(x) || !aligned16(y)) return RQ_ERR_ALIGN;
  return check_output(y, (size_t)M * N * 4, qweight, scales, zeros, x, N, K, bits, group,
                      layout, M);
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
  const rq::GemvCfg c = rq::choose_gemv(fmt, M, N, K);
  const hipError_t e = rq::launch_gemv(p, c, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? RQ_OK : RQ_ERR_LAUNCH;
}

rq_status rq_gemm_smallm(const void* qweight, const void* scales, const void* zeros,
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
  if (!rq::gemm_supports(fmt, M, K)) {
    // K is not a whole number of the matrix-core kernel's chunks
    const rq::GemvCfg c = rq::choose_gemv(fmt, M, N, K);
    return rq::launch_gemv(p, c, s) == hipSuccess ? RQ_OK : RQ_ERR_LAUNCH;
  }
  const rq::GemmCfg c = rq::choose_gemm(fmt, M, N, K, group);
  Workspace w;
  if (c.splits > 1) {
    st = get_workspace(dev, s, rq::gemm_workspace_floats(c, M, N),
                       (size_t)rq::gemm_counters(c, N), &w);
    if (st != RQ_OK) return st;
  }
  const hipError_t e = rq::launch_gemm(p, c, w.partial, w.counters, s);
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
    case RQ_ERR_DEVICE: return "no usable gfx950 device or workspace";
    default: return "unknown status";
  }
}

int rq_version(void) { return (1 << 16) | 0; }

}  // extern "C"
