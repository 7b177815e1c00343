/*
 * rq_probe.h -- measurement kernels that bound what any kernel of librq can
 * reach on the device: a streaming read (the achievable HBM read rate for a
 * given size and launch shape), a copy (the reference for the memory traffic
 * counters: it moves exactly `bytes` in and `bytes` out) and an empty kernel
 * (the launch floor).  They serve the roofline figures reported next to the
 * products of include/rq.h; they compute nothing of the method.
 *
 * Pointers are device memory owned by the caller, 16-byte aligned; `bytes`
 * must be a multiple of 16.  Work is enqueued on `stream` (a hipStream_t,
 * NULL = null stream).  Return values are rq_status codes (include/rq.h).
 */
#ifndef RQ_PROBE_H
#define RQ_PROBE_H

#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Read `bytes` from src once (16-byte nontemporal loads, grid-stride, eight
 * loads in flight per lane).  sink[blockIdx] receives an XOR of what the block
 * read, so the loads cannot be dropped; sink needs `blocks` entries.
 * blocks <= 0 or threads <= 0 choose defaults (2048 blocks of 256). */
int rq_probe_read(const void* src, size_t bytes, unsigned* sink, int blocks,
                  int threads, void* stream);

/* dst[i] = src[i] for `bytes` bytes (ranges must not overlap). */
int rq_probe_copy(const void* src, void* dst, size_t bytes, void* stream);

/* One workgroup of 64 threads that does nothing. */
int rq_probe_empty(void* stream);

/* Re-read the launch-shape override variables (RQ_GEMV_LPR, RQ_GEMV_CPL,
 * RQ_GEMV_NPASS, RQ_GEMM_PLAN (1-based index of a workgroup arrangement of
 * the matrix-core kernel), RQ_GEMM_SPLITS, RQ_GEMV_KERNEL (the kernel of
 * rq_gemv and rq_gemv_batched at any M: 1 = vector-unit kernel, 2 = matrix-core
 * decode kernel where M <= 4 and K holds at least eight of its chunks,
 * 3 = small-batch matrix-core kernel where K suits it; 2 and 3 fall back to
 * the vector-unit kernel elsewhere); unset or 0 = the library's own
 * choice).  They are read once, at the first call, otherwise.  For tuning
 * sweeps and tests; not thread-safe against concurrent products. */
int rq_tuning_reload(void);

#ifdef __cplusplus
}
#endif

#endif /* RQ_PROBE_H */
