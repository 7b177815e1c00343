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

/* Cross-workgroup signalling cost.  `blocks` workgroups of 256 threads each
 * write a 64-dword slot of `flags` and then count themselves in flags[0]:
 * mode 0 with __threadfence() between the writes and the count (a device-scope
 * release, which writes back the L2); mode 1 with device-scope coherent writes
 * whose completion is awaited instead (no write-back).  flags: device memory
 * of at least 64 * (blocks + 1) dwords, zeroed by the caller. */
int rq_probe_signal(unsigned* flags, int mode, int blocks, void* stream);

/* `rounds` grid-wide barriers among `blocks` (at most 4096) co-resident
 * workgroups (a cooperative launch: RQ_ERR_LAUNCH if they cannot all be
 * resident).  Each round every workgroup writes its 64-dword data slot,
 * passes a barrier, reads its neighbour's slot, and passes a second barrier;
 * bad[b] (blocks entries) receives the number of stale values workgroup b
 * read, plus 0x10000 if a wait gave up.  Arrival schemes: mode 2, one counter
 * with relaxed device-scope atomics and coherent slot writes awaited before
 * arriving; mode 3, one counter with release arrivals and acquire polls and
 * plain slot writes; mode 4, as 2 with 32 counters on separate cache lines;
 * mode 5, as 2 with no atomics (one arrival word per workgroup, polled all at
 * once).  Every wait gives up after `spin` polls (about 1 us each) and then
 * stops every workgroup, so the kernel always ends.  flags: at least
 * 2048 + 65 * blocks dwords, zeroed by the caller. */
int rq_probe_barrier(unsigned* flags, int mode, int blocks, int rounds, int spin,
                     unsigned* bad, void* stream);

/* Dense fp16 matrix-core rate: `blocks` workgroups of four waves, each wave
 * issuing 8 x 16384 flops per iteration for `iters` iterations: shape 0, eight
 * independent chains of v_mfma_f32_16x16x32_f16; shape 1, four chains of
 * v_mfma_f32_32x32x16_f16.  sink: `blocks` floats (practically never
 * written). */
int rq_probe_mfma(int blocks, int iters, int shape, float* sink, void* stream);

/* Vector-unit issue cost of one instruction kind: `blocks` workgroups of 512
 * threads, every lane running `iters` x 64 instructions of kind `op` over
 * eight independent registers.  Kinds: 0 v_and_b32, 1 v_lshrrev_b32,
 * 2 v_perm_b32, 3 v_bitop3_b32, 4 v_pk_fma_f16, 5 v_pk_add_f16,
 * 6 v_dot2c_f32_f16, 7 v_fma_mix_f32, 8 v_fma_f32, 9 v_cvt_f32_f16,
 * 10 v_add_u32, 11 v_add_f32, 12 v_mul_f32, 13 v_mov_b32 with a DPP row
 * shift, 14 v_add_f32 with a DPP row shift, 15 v_lshl_or_b32,
 * 16 v_and_or_b32.  sink: `blocks` entries (practically never written). */
int rq_probe_valu(int op, int blocks, int iters, unsigned* sink, void* stream);

/* Vector work beside the matrix pipe: every wave of `blocks` 512-thread
 * workgroups runs `iters` rounds of eight independent
 * v_mfma_f32_16x16x32_f16 and/or `per` (4 or 8) vector operations per MFMA
 * of kind `kind` (0 binary16 pair FMAs, 1 integer bit operations, 2 binary32
 * FMAs).  mode 0: MFMAs only; 1: vector work only; 2: both in every wave,
 * each MFMA followed by its share; 3: MFMAs in waves 0-3, vector work in
 * waves 4-7 of each workgroup.  Comparing the four durations shows whether
 * the two kinds of work overlap in time.  sink: `blocks` floats. */
int rq_probe_overlap(int mode, int kind, int per, int blocks, int iters, float* sink,
                     void* stream);

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

/* The workgroup arrangement of the small-batch matrix-core kernel for one
 * product: *plan receives its 1-based index (the numbering RQ_GEMM_PLAN
 * uses), *splits the number of K-ranges split across workgroups.
 * allow_split = 0 asks for the arrangement rq_gemv and rq_gemv_batched use
 * (K kept whole), nonzero for rq_gemm_smallm's own choice (which keeps K whole
 * too when it has no workspace).  Overrides in effect are applied, so a test
 * can see whether a forced plan was taken.  Host-only; no GPU needed.
 * Returns RQ_ERR_UNSUPPORTED when the matrix-core kernel cannot take the shape
 * (rq_gemm_smallm then runs the vector-unit kernel). */
int rq_gemm_config(int M, int N, int K, int bits, int group, int layout, int allow_split,
                   int* plan, int* splits);

/* The kernel rq_gemv runs for one product of M activation rows: *kernel
 * receives 0 for the vector-unit kernel, 1 for the matrix-core decode kernel,
 * 2 for the small-batch matrix-core kernel.  For the vector-unit kernel,
 * *lpr receives the lanes per weight row (0 = the generic kernel, which
 * splits no row), *cpl the 16-byte chunks per lane per row and *npass the
 * rows each lane streams; all three are 0 for the other kernels.  Overrides
 * in effect are applied.  Host-only; no GPU needed.  Returns
 * RQ_ERR_UNSUPPORTED for an unknown format, RQ_ERR_SHAPE for sizes rq_gemv
 * rejects. */
int rq_gemv_config(int M, int N, int K, int bits, int group, int layout, int* kernel,
                   int* lpr, int* cpl, int* npass);

#ifdef __cplusplus
}
#endif

#endif /* RQ_PROBE_H */
