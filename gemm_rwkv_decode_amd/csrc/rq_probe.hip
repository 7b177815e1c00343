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

// Layout of the barrier probe's flags buffer (dwords): arrival counters
// (one per 128-byte line), the abort flag, one arrival word per workgroup
// (contiguous), then the 64-dword data slots.
constexpr int BAR_CTR_LINE = 32;
constexpr int BAR_NCTR = 32;
constexpr int BAR_ABORT = BAR_CTR_LINE * BAR_NCTR;
constexpr int BAR_WGFLAG = BAR_ABORT + 64;

__device__ __forceinline__ unsigned wave_sum(unsigned v) {
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}

// One barrier phase for workgroup b of G: arrive (after this workgroup's
// writes), then wait until every workgroup has arrived `phase` times.  Wave 0
// does the arriving and polling; the others wait at the workgroup barrier.
// Returns false if the wait gave up (after `spin` polls) or another
// workgroup did.
//   mode 2: one counter, relaxed device-scope atomics, coherent writes;
//   mode 3: one counter, release arrival and acquire polls;
//   mode 4: 32 counters on separate lines (workgroup b arrives on b mod 32),
//           the poll sums them with one load per lane;
//   mode 5: no atomics: workgroup b stores `phase` in its own word, the poll
//           reads all words (G/64 loads per lane) and checks them all.
__device__ bool bar_phase(unsigned* flags, int mode, unsigned phase, int spin) {
  const int t = threadIdx.x;
  const unsigned G = gridDim.x, b = blockIdx.x;
  __shared__ int ok;
  if (t < 64) {
    const int lane = t;
    if (lane == 0) {
      if (mode == 2) {
        __hip_atomic_fetch_add(flags, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      } else if (mode == 3) {
        __hip_atomic_fetch_add(flags, 1u, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
      } else if (mode == 4) {
        __hip_atomic_fetch_add(flags + (b % BAR_NCTR) * BAR_CTR_LINE, 1u, __ATOMIC_RELAXED,
                               __HIP_MEMORY_SCOPE_AGENT);
      } else {
        store_agent(flags + BAR_WGFLAG + b, phase);
      }
    }
    int n = 0;
    bool done = false, gave_up = false;
    while (!done) {
      if (mode == 2 || mode == 3) {
        const unsigned c = mode == 2 ? load_agent(flags)
                                     : __hip_atomic_load(flags, __ATOMIC_ACQUIRE,
                                                         __HIP_MEMORY_SCOPE_AGENT);
        done = c >= phase * G;
      } else if (mode == 4) {
        const unsigned c = lane < BAR_NCTR ? load_agent(flags + lane * BAR_CTR_LINE) : 0u;
        done = wave_sum(c) >= phase * G;
      } else {
        bool all = true;
        for (unsigned w = lane; w < G; w += 64) all &= load_agent(flags + BAR_WGFLAG + w) >= phase;
        done = __all(all);
      }
      if (done) break;
      if (load_agent(flags + BAR_ABORT) != 0u || ++n >= spin) {
        if (lane == 0) store_agent(flags + BAR_ABORT, 1u);
        gave_up = true;
        break;
      }
      __builtin_amdgcn_s_sleep(1);
    }
    if (lane == 0) ok = gave_up ? 0 : 1;
  }
  __syncthreads();
  return ok != 0;
}

// `rounds` grid-wide barriers; every workgroup must be resident (cooperative
// launch).  In round r each workgroup writes r + 1 into its 64-dword slot,
// passes a barrier, reads its neighbour's slot and counts values other than
// r + 1 into bad[blockIdx], then passes a second barrier before the slot is
// rewritten.  Writes and reads of the slots are device-scope coherent (mode 3:
// plain, ordered by the release/acquire of the barrier); a write is awaited
// before the arrival.  Every wait is bounded: after `spin` polls a workgroup
// raises the abort flag, and every workgroup stops at its next poll.
__global__ void __launch_bounds__(256)
k_probe_barrier(unsigned* flags, int mode, int rounds, int spin, unsigned* bad) {
  const int t = threadIdx.x;
  const unsigned G = gridDim.x;
  const unsigned gpad = (G + 63) / 64 * 64;
  unsigned* slots = flags + BAR_WGFLAG + gpad;
  unsigned* slot = slots + SYNC_SLOT * blockIdx.x;
  const unsigned* peer = slots + SYNC_SLOT * ((blockIdx.x + 1) % G);
  unsigned nbad = 0;
  bool stopped = false;
  for (int r = 0; r < rounds && !stopped; r++) {
    if (t < SYNC_SLOT) {
      if (mode == 3) slot[t] = (unsigned)r + 1;
      else store_agent(slot + t, (unsigned)r + 1);
    }
    if (mode != 3) __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    if (!bar_phase(flags, mode, 2u * r + 1u, spin)) {
      stopped = true;
      break;
    }
    if (t < SYNC_SLOT) {
      const unsigned v = mode == 3 ? peer[t] : load_agent(peer + t);
      nbad += (v != (unsigned)r + 1);
    }
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();  // nobody rewrites a slot before its reader is done
    if (!bar_phase(flags, mode, 2u * r + 2u, spin)) stopped = true;
  }
  for (int o = 32; o >= 1; o >>= 1) nbad += __shfl_xor(nbad, o, 64);
  __shared__ unsigned wb[4];
  if ((t & 63) == 0) wb[t >> 6] = nbad;
  __syncthreads();
  if (t == 0) bad[blockIdx.x] = wb[0] + wb[1] + wb[2] + wb[3] + (stopped ? 0x10000u : 0u);
}

// Dense fp16 matrix-core rate: every wave runs `iters` x 8 independent
// v_mfma_f32_16x16x32_f16 (shape 0: eight accumulator chains, 16384 flops
// each) or iters x 4 v_mfma_f32_32x32x16_f16 (shape 1: four chains, 32768
// flops each), then folds its accumulators so nothing is dropped.
__global__ void __launch_bounds__(256) k_probe_mfma(int iters, int shape, float* sink) {
  typedef _Float16 h8 __attribute__((ext_vector_type(8)));
  typedef float f4 __attribute__((ext_vector_type(4)));
  const int lane = threadIdx.x & 63;
  h8 a, b;
  for (int i = 0; i < 8; i++) {
    a[i] = (_Float16)((lane + i) & 3);
    b[i] = (_Float16)((lane * 3 + i) & 3);
  }
  float s = 0.0f;
  if (shape == 0) {
    f4 c[8];
#pragma unroll
    for (int j = 0; j < 8; j++) c[j] = f4{0, 0, 0, 0};
    for (int it = 0; it < iters; it++) {
#pragma unroll
      for (int j = 0; j < 8; j++)
        c[j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c[j], 0, 0, 0);
    }
#pragma unroll
    for (int j = 0; j < 8; j++) s += c[j][0] + c[j][1] + c[j][2] + c[j][3];
  } else {
    // v_mfma_f32_32x32x16_f16: the same 16384 flops... x2 (32768), four chains
    typedef float f16v __attribute__((ext_vector_type(16)));
    f16v c[4];
#pragma unroll
    for (int j = 0; j < 4; j++)
#pragma unroll
      for (int i = 0; i < 16; i++) c[j][i] = 0.0f;
    for (int it = 0; it < iters; it++) {
#pragma unroll
      for (int j = 0; j < 4; j++)
        c[j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c[j], 0, 0, 0);
    }
#pragma unroll
    for (int j = 0; j < 4; j++)
#pragma unroll
      for (int i = 0; i < 16; i++) s += c[j][i];
  }
  if (s == 1234.5f) sink[blockIdx.x] = s;  // practically never true; keeps the work live
}

// Vector-unit issue cost of one instruction kind: every lane runs `iters` x 64
// instructions of kind OP over eight independent registers.  Inline assembly,
// so that exactly the named instruction is timed; the values are never used
// beyond the final fold.
constexpr int VALU_KINDS = 17;
template <int OP>
__global__ void __launch_bounds__(512) k_probe_valu(int iters, unsigned* sink) {
  const u32 lane = threadIdx.x;
  u32 a[8];
#pragma unroll
  for (int i = 0; i < 8; i++) a[i] = lane * 2654435761u + (u32)i * 0x3C003C00u;
  const u32 b = 0x3BFF3BFFu ^ lane, c = 0x00010001u + lane;
  for (int it = 0; it < iters; it++) {
#pragma unroll
    for (int r = 0; r < 8; r++)
#pragma unroll
      for (int i = 0; i < 8; i++) {
        if constexpr (OP == 0) asm volatile("v_and_b32 %0, %0, %1" : "+v"(a[i]) : "v"(b));
        if constexpr (OP == 1) asm volatile("v_lshrrev_b32 %0, 3, %0" : "+v"(a[i]));
        if constexpr (OP == 2) asm volatile("v_perm_b32 %0, %0, %1, %2" : "+v"(a[i]) : "v"(b), "v"(c));
        if constexpr (OP == 3)
          asm volatile("v_bitop3_b32 %0, %0, %1, %2 bitop3:0x6c" : "+v"(a[i]) : "v"(b), "v"(c));
        if constexpr (OP == 4) asm volatile("v_pk_fma_f16 %0, %0, %1, %2" : "+v"(a[i]) : "v"(b), "v"(c));
        if constexpr (OP == 5) asm volatile("v_pk_add_f16 %0, %0, %1" : "+v"(a[i]) : "v"(b));
        if constexpr (OP == 6) asm volatile("v_dot2c_f32_f16 %0, %1, %2" : "+v"(a[i]) : "v"(b), "v"(c));
        if constexpr (OP == 7)
          asm volatile("v_fma_mix_f32 %0, %1, %0, %2 op_sel_hi:[1,0,0]" : "+v"(a[i]) : "v"(b), "v"(c));
        if constexpr (OP == 8) asm volatile("v_fma_f32 %0, %0, %1, %2" : "+v"(a[i]) : "v"(b), "v"(c));
        if constexpr (OP == 9) asm volatile("v_cvt_f32_f16 %0, %0" : "+v"(a[i]));
        if constexpr (OP == 10) asm volatile("v_add_u32 %0, %0, %1" : "+v"(a[i]) : "v"(b));
        if constexpr (OP == 11) asm volatile("v_add_f32 %0, %0, %1" : "+v"(a[i]) : "v"(b));
        if constexpr (OP == 12) asm volatile("v_mul_f32 %0, %0, %1" : "+v"(a[i]) : "v"(b));
        if constexpr (OP == 13)
          asm volatile("v_mov_b32_dpp %0, %0 row_shr:1 row_mask:0xf bank_mask:0xf" : "+v"(a[i]));
        if constexpr (OP == 14)
          asm volatile("v_add_f32_dpp %0, %0, %0 row_shr:1 row_mask:0xf bank_mask:0xf"
                       : "+v"(a[i]));
        if constexpr (OP == 15) asm volatile("v_lshl_or_b32 %0, %0, 4, %1" : "+v"(a[i]) : "v"(b));
        if constexpr (OP == 16)
          asm volatile("v_and_or_b32 %0, %0, %1, %2" : "+v"(a[i]) : "v"(b), "v"(c));
      }
  }
  u32 f = 0;
#pragma unroll
  for (int i = 0; i < 8; i++) f ^= a[i];
  if (f == 0x12345679u) sink[blockIdx.x] = f;  // practically never true
}

template <int OP>
hipError_t launch_valu(int op, int blocks, int iters, unsigned* sink, hipStream_t s) {
  if constexpr (OP >= VALU_KINDS) {
    return hipErrorInvalidValue;
  } else {
    if (op != OP) return launch_valu<OP + 1>(op, blocks, iters, sink, s);
    hipLaunchKernelGGL(k_probe_valu<OP>, dim3(blocks), dim3(512), 0, s, iters, sink);
    return hipGetLastError();
  }
}

// Vector work beside the matrix pipe.  Each wave runs `iters` rounds; a round
// is eight independent v_mfma_f32_16x16x32_f16 and/or PER vector operations
// per MFMA (KIND 0: binary16 pair FMAs, 1: integer bit operations, 2: binary32
// FMAs, on eight independent registers).  MODE 0: MFMAs only; 1: vector work
// only; 2: both in every wave, each MFMA followed by its share of the vector
// work; 3: the MFMAs in waves 0-3 and the vector work in waves 4-7 of the
// 512-thread workgroup (which share the four SIMDs when waves are spread over
// them in turn).
template <int MODE, int KIND, int PER>
__global__ void __launch_bounds__(512) k_probe_overlap(int iters, float* sink) {
  typedef _Float16 h8 __attribute__((ext_vector_type(8)));
  typedef _Float16 h2v __attribute__((ext_vector_type(2)));
  typedef float f4 __attribute__((ext_vector_type(4)));
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const h8 a = (h8)(_Float16)(0.001f * lane), b = (h8)(_Float16)(0.002f * lane);
  f4 c[8];
  h2v v[8];
  u32 u[8];
  float w[8];
#pragma unroll
  for (int i = 0; i < 8; i++) {
    c[i] = f4{0, 0, 0, 0};
    v[i] = h2v{(_Float16)(0.5f + lane * 1e-3f * i), (_Float16)0.25f};
    u[i] = (u32)lane * 2654435761u + (u32)i;
    w[i] = 0.5f + lane * 1e-3f * i;
  }
  const h2v m = {(_Float16)0.999f, (_Float16)0.999f}, ad = {(_Float16)0.001f, (_Float16)0.001f};
  const bool do_m = MODE == 0 || MODE == 2 || (MODE == 3 && wave < 4);
  const bool do_v = MODE == 1 || MODE == 2 || (MODE == 3 && wave >= 4);
  auto vop = [&](int j) {
    if constexpr (KIND == 0) v[j & 7] = __builtin_elementwise_fma(v[j & 7], m, ad);
    else if constexpr (KIND == 1) u[j & 7] = ((u[j & 7] & 0x0F0F0F0Fu) ^ 0x64646464u) | (u[j & 7] >> 3);
    else w[j & 7] = __builtin_fmaf(w[j & 7], 0.999f, 0.001f);
  };
  for (int it = 0; it < iters; it++) {
    if (do_m && do_v) {
#pragma unroll
      for (int i = 0; i < 8; i++) {
        c[i] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c[i], 0, 0, 0);
#pragma unroll
        for (int j = 0; j < PER; j++) vop(j);
      }
#pragma unroll
      for (int i = 0; i < 8; i++) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // one MFMA
        __builtin_amdgcn_sched_group_barrier(0x002, PER, 0);  // then vector work
      }
    } else if (do_m) {
#pragma unroll
      for (int i = 0; i < 8; i++) c[i] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c[i], 0, 0, 0);
    } else if (do_v) {
#pragma unroll
      for (int i = 0; i < 8; i++)
#pragma unroll
        for (int j = 0; j < PER; j++) vop(j);
    }
    __builtin_amdgcn_sched_barrier(0);
  }
  float s = 0;
#pragma unroll
  for (int i = 0; i < 8; i++) s += c[i][0] + c[i][3] + (float)v[i][0] + (float)(u[i] & 7u) + w[i];
  if (s == 1234.5f) sink[blockIdx.x] = s;  // practically never true
}

template <int MODE, int KIND>
hipError_t launch_overlap_k(int per, int blocks, int iters, float* sink, hipStream_t s) {
  switch (per) {
    case 4: hipLaunchKernelGGL((k_probe_overlap<MODE, KIND, 4>), dim3(blocks), dim3(512), 0, s, iters, sink); break;
    case 8: hipLaunchKernelGGL((k_probe_overlap<MODE, KIND, 8>), dim3(blocks), dim3(512), 0, s, iters, sink); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}
template <int MODE>
hipError_t launch_overlap_m(int kind, int per, int blocks, int iters, float* sink, hipStream_t s) {
  switch (kind) {
    case 0: return launch_overlap_k<MODE, 0>(per, blocks, iters, sink, s);
    case 1: return launch_overlap_k<MODE, 1>(per, blocks, iters, sink, s);
    case 2: return launch_overlap_k<MODE, 2>(per, blocks, iters, sink, s);
    default: return hipErrorInvalidValue;
  }
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
  if (mode < 2 || mode > 5 || blocks < 1 || blocks > 4096 || rounds < 1 || spin < 1)
    return RQ_ERR_SHAPE;
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

int rq_probe_mfma(int blocks, int iters, int shape, float* sink, void* stream) {
  if (!sink) return RQ_ERR_NULL;
  if (blocks < 1 || iters < 1 || (shape != 0 && shape != 1)) return RQ_ERR_SHAPE;
  hipLaunchKernelGGL(k_probe_mfma, dim3(blocks), dim3(256), 0,
                     static_cast<hipStream_t>(stream), iters, shape, sink);
  return hipGetLastError() == hipSuccess ? RQ_OK : RQ_ERR_LAUNCH;
}

int rq_probe_valu(int op, int blocks, int iters, unsigned* sink, void* stream) {
  if (!sink) return RQ_ERR_NULL;
  if (op < 0 || op >= VALU_KINDS || blocks < 1 || iters < 1) return RQ_ERR_SHAPE;
  return launch_valu<0>(op, blocks, iters, sink, static_cast<hipStream_t>(stream)) == hipSuccess
             ? RQ_OK
             : RQ_ERR_LAUNCH;
}

int rq_probe_overlap(int mode, int kind, int per, int blocks, int iters, float* sink,
                     void* stream) {
  if (!sink) return RQ_ERR_NULL;
  if (mode < 0 || mode > 3 || kind < 0 || kind > 2 || (per != 4 && per != 8) || blocks < 1 ||
      iters < 1)
    return RQ_ERR_SHAPE;
  const hipStream_t s = static_cast<hipStream_t>(stream);
  hipError_t e;
  switch (mode) {
    case 0: e = launch_overlap_m<0>(kind, per, blocks, iters, sink, s); break;
    case 1: e = launch_overlap_m<1>(kind, per, blocks, iters, sink, s); break;
    case 2: e = launch_overlap_m<2>(kind, per, blocks, iters, sink, s); break;
    default: e = launch_overlap_m<3>(kind, per, blocks, iters, sink, s); break;
  }
  return e == hipSuccess ? RQ_OK : RQ_ERR_LAUNCH;
}

int rq_probe_empty(void* stream) {
  hipLaunchKernelGGL(k_probe_empty, dim3(1), dim3(64), 0, static_cast<hipStream_t>(stream));
  return hipGetLastError() == hipSuccess ? RQ_OK : RQ_ERR_LAUNCH;
}

}  // extern "C"
