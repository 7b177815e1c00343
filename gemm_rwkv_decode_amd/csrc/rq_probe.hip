// rq_probe.hip -- measurement kernels declared in include/rq_probe.h.
#include <hip/hip_runtime.h>

#include <stdint.h>

#include "rq.h"
#include "rq_common.h"
#include "rq_probe.h"

namespace {

using rq::u32;
using rq::u32x4;

constexpr int UNR = 8;  // 16-byte loads in flight per lane

__global__ void __launch_bounds__(1024)
k_probe_read(const u32x4* __restrict__ src, size_t n16, unsigned* __restrict__ sink) {
  const size_t stride = (size_t)gridDim.x * blockDim.x;
  size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  u32 acc = 0;
  for (; i + (UNR - 1) * stride < n16; i += UNR * stride) {
    u32x4 v[UNR];
#pragma unroll
    for (int u = 0; u < UNR; u++) v[u] = __builtin_nontemporal_load(src + i + u * stride);
#pragma unroll
    for (int u = 0; u < UNR; u++) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
  }
  for (; i < n16; i += stride) {
    const u32x4 v = __builtin_nontemporal_load(src + i);
    acc ^= v.x ^ v.y ^ v.z ^ v.w;
  }
  // fold the block's lanes into one word
  for (int off = 32; off >= 1; off >>= 1) acc ^= __shfl_xor(acc, off, 64);
  __shared__ unsigned part[16];
  if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = acc;
  __syncthreads();
  if (threadIdx.x == 0) {
    unsigned a = 0;
    for (int w = 0; w < (int)(blockDim.x >> 6); w++) a ^= part[w];
    sink[blockIdx.x] = a;
  }
}

__global__ void __launch_bounds__(256)
k_probe_copy(const u32x4* __restrict__ src, u32x4* __restrict__ dst, size_t n16) {
  const size_t stride = (size_t)gridDim.x * blockDim.x;
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n16; i += stride)
    dst[i] = src[i];
}

__global__ void k_probe_empty() {}

bool ok16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

}  // namespace

extern "C" {

int rq_probe_read(const void* src, size_t bytes, unsigned* sink, int blocks, int threads,
                  void* stream) {
  if (!src || !sink) return RQ_ERR_NULL;
  if (bytes == 0 || bytes % 16) return RQ_ERR_SHAPE;
  if (!ok16(src)) return RQ_ERR_ALIGN;
  if (blocks <= 0) blocks = 2048;
  if (threads <= 0) threads = 256;
  if (threads % 64 || threads > 1024) return RQ_ERR_SHAPE;
  hipLaunchKernelGGL(k_probe_read, dim3(blocks), dim3(threads), 0,
                     static_cast<hipStream_t>(stream), static_cast<const u32x4*>(src),
                     bytes / 16, sink);
  return hipGetLastError() == hipSuccess ? RQ_OK : RQ_ERR_LAUNCH;
}

int rq_probe_copy(const void* src, void* dst, size_t bytes, void* stream) {
  if (!src || !dst) return RQ_ERR_NULL;
  if (bytes == 0 || bytes % 16) return RQ_ERR_SHAPE;
  if (!ok16(src) || !ok16(dst)) return RQ_ERR_ALIGN;
  const uintptr_t a = reinterpret_cast<uintptr_t>(src), b = reinterpret_cast<uintptr_t>(dst);
  if (a < b + bytes && b < a + bytes) return RQ_ERR_ALIAS;
  size_t n16 = bytes / 16;
  size_t blocks = (n16 + 255) / 256;
  if (blocks > 8192) blocks = 8192;
  hipLaunchKernelGGL(k_probe_copy, dim3((unsigned)blocks), dim3(256), 0,
                     static_cast<hipStream_t>(stream), static_cast<const u32x4*>(src),
                     static_cast<u32x4*>(dst), n16);
  return hipGetLastError() == hipSuccess ? RQ_OK : RQ_ERR_LAUNCH;
}

int rq_probe_empty(void* stream) {
  hipLaunchKernelGGL(k_probe_empty, dim3(1), dim3(64), 0, static_cast<hipStream_t>(stream));
  return hipGetLastError() == hipSuccess ? RQ_OK : RQ_ERR_LAUNCH;
}

}  // extern "C"
