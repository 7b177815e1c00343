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

// ---------------------------------------------------------------------------
// Cross-workgroup signalling.  flags[0] is a monotonic arrival counter,
// flags[1] an abort flag, flags[64 + 64*b ...] block b's 64-dword data slot.
// Device-scope ("agent") relaxed atomic stores and loads are the coherent
// accesses of the memory model (global stores/loads with sc1 on gfx950);
// a release fence additionally writes back the L2 (buffer_wbl2) and an acquire
// invalidates it (buffer_inv).
// ---------------------------------------------------------------------------
constexpr int SYNC_SLOT = 64;

__device__ __forceinline__ void store_agent(unsigned* p, unsigned v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ unsigned load_agent(const unsigned* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// mode 0: data stores, __threadfence(), one arrival per workgroup.
// mode 1: device-scope data stores, a wait until they are acknowledged, one
//         relaxed arrival per workgroup (no cache write-back).
__global__ void __launch_bounds__(256) k_probe_signal(unsigned* flags, int mode) {
  unsigned* slot = flags + SYNC_SLOT + SYNC_SLOT * blockIdx.x;
  const int t = threadIdx.x;
  if (mode == 0) {
    if (t < SYNC_SLOT) slot[t] = blockIdx.x;
    __threadfence();
    __syncthreads();
  } else {
    if (t < SYNC_SLOT) store_agent(slot + t, blockIdx.x);
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
  }
  if (t == 0) __hip_atomic_fetch_add(flags, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// `rounds` grid-wide barriers; every workgroup must be resident (cooperative
// launch).  In round r each workgroup writes r + 1 into its slot, arrives, waits
// until all have arrived, then reads its neighbour's slot and counts values
// other than r + 1 into bad[blockIdx].  mode 2: device-scope stores and loads,
// arrival after the stores are acknowledged; mode 3: plain stores, release
// arrival, acquire wait.  Every wait is bounded: after `spin` polls the
// workgroup raises the abort flag, and every workgroup stops at the next poll.
__global__ void __launch_bounds__(256)
k_probe_barrier(unsigned* flags, int mode, int rounds, int spin, unsigned* bad) {
  const int t = threadIdx.x;
  const unsigned G = gridDim.x;
  unsigned* slot = flags + SYNC_SLOT + SYNC_SLOT * blockIdx.x;
  const unsigned* peer = flags + SYNC_SLOT + SYNC_SLOT * ((blockIdx.x + 1) % G);
  unsigned nbad = 0;
  __shared__ int stop;
  if (t == 0) stop = 0;
  __syncthreads();
  for (int r = 0; r < rounds; r++) {
    if (t < SYNC_SLOT) {
      if (mode == 2) store_agent(slot + t, (unsigned)r + 1);
      else slot[t] = (unsigned)r + 1;
    }
    if (mode == 2) __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    if (t == 0) {
      if (mode == 2)
        __hip_atomic_fetch_add(flags, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      else
        __hip_atomic_fetch_add(flags, 1u, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
      // two arrivals per workgroup and round: after the first of round r
      // the count reaches (2r + 1) G
      const unsigned want = (unsigned)(2 * r + 1) * G;
      int n = 0;
      for (;;) {
        const unsigned c = mode == 2
            ? load_agent(flags)
            : __hip_atomic_load(flags, __ATOMIC_ACQUIRE, __HIP_MEMORY_SCOPE_AGENT);
        if (c >= want) break;
        if (load_agent(flags + 1) != 0u || ++n >= spin) {
          store_agent(flags + 1, 1u);
          stop = 1;
          break;
        }
        __builtin_amdgcn_s_sleep(1);
      }
    }
    __syncthreads();
    if (stop) break;
    if (t < SYNC_SLOT) {
      const unsigned v = mode == 2 ? load_agent(peer + t) : peer[t];
      nbad += (v != (unsigned)r + 1);
    }
    // nobody overwrites a slot before its reader is done with it
    __syncthreads();
    if (t == 0) {
      if (mode == 2)
        __hip_atomic_fetch_add(flags, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      else
        __hip_atomic_fetch_add(flags, 1u, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
      const unsigned want = (unsigned)(2 * r + 2) * G;
      int n = 0;
      for (;;) {
        const unsigned c = load_agent(flags);
        if (c >= want) break;
        if (load_agent(flags + 1) != 0u || ++n >= spin) {
          store_agent(flags + 1, 1u);
          stop = 1;
          break;
        }
        __builtin_amdgcn_s_sleep(1);
      }
    }
    __syncthreads();
    if (stop) break;
  }
  for (int o = 32; o >= 1; o >>= 1) nbad += __shfl_xor(nbad, o, 64);
  __shared__ unsigned wb[4];
  if ((t & 63) == 0) wb[t >> 6] = nbad;
  __syncthreads();
  if (t == 0) bad[blockIdx.x] = wb[0] + wb[1] + wb[2] + wb[3] + (stop ? 0x10000u : 0u);
}

// Dense fp16 matrix-core rate: every wave runs `iters` x 8 independent
// v_mfma_f32_16x16x32_f16 (eight accumulator chains), then folds its
// accumulators into sink so nothing is dropped.
__global__ void __launch_bounds__(256) k_probe_mfma(int iters, float* sink) {
  typedef _Float16 h8 __attribute__((ext_vector_type(8)));
  typedef float f4 __attribute__((ext_vector_type(4)));
  const int lane = threadIdx.x & 63;
  h8 a, b;
  for (int i = 0; i < 8; i++) {
    a[i] = (_Float16)((lane + i) & 3);
    b[i] = (_Float16)((lane * 3 + i) & 3);
  }
  f4 c[8];
#pragma unroll
  for (int j = 0; j < 8; j++) c[j] = f4{0, 0, 0, 0};
  for (int it = 0; it < iters; it++) {
#pragma unroll
    for (int j = 0; j < 8; j++) c[j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c[j], 0, 0, 0);
  }
  float s = 0.0f;
#pragma unroll
  for (int j = 0; j < 8; j++) s += c[j][0] + c[j][1] + c[j][2] + c[j][3];
  if (s == 1234.5f) sink[blockIdx.x] = s;  // practically never true; keeps the work live
}

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

int rq_probe_signal(unsigned* flags, int mode, int blocks, void* stream) {
  if (!flags) return RQ_ERR_NULL;
  if ((mode != 0 && mode != 1) || blocks < 1 || blocks > 65536) return RQ_ERR_SHAPE;
  hipLaunchKernelGGL(k_probe_signal, dim3(blocks), dim3(256), 0,
                     static_cast<hipStream_t>(stream), flags, mode);
  return hipGetLastError() == hipSuccess ? RQ_OK : RQ_ERR_LAUNCH;
}

int rq_probe_barrier(unsigned* flags, int mode, int blocks, int rounds, int spin,
                     unsigned* bad, void* stream) {
  if (!flags || !bad) return RQ_ERR_NULL;
  if ((mode != 2 && mode != 3) || blocks < 1 || rounds < 1 || spin < 1) return RQ_ERR_SHAPE;
  void* args[] = {&flags, &mode, &rounds, &spin, &bad};
  // cooperative: the runtime refuses the launch unless every workgroup can be
  // resident at once, which the waits need
  const hipError_t e = hipLaunchCooperativeKernel(
      reinterpret_cast<const void*>(k_probe_barrier), dim3(blocks), dim3(256), args, 0,
      static_cast<hipStream_t>(stream));
  if (e != hipSuccess) {
    (void)hipGetLastError();
    return RQ_ERR_LAUNCH;
  }
  return RQ_OK;
}

int rq_probe_mfma(int blocks, int iters, float* sink, void* stream) {
  if (!sink) return RQ_ERR_NULL;
  if (blocks < 1 || iters < 1) return RQ_ERR_SHAPE;
  hipLaunchKernelGGL(k_probe_mfma, dim3(blocks), dim3(256), 0,
                     static_cast<hipStream_t>(stream), iters, sink);
  return hipGetLastError() == hipSuccess ? RQ_OK : RQ_ERR_LAUNCH;
}

int rq_probe_empty(void* stream) {
  hipLaunchKernelGGL(k_probe_empty, dim3(1), dim3(64), 0, static_cast<hipStream_t>(stream));
  return hipGetLastError() == hipSuccess ? RQ_OK : RQ_ERR_LAUNCH;
}

}  // extern "C"
