/*
 * rq.h -- C interface of librq: group-wise low-bit weight dequantization and
 * dequantize-and-multiply (GEMV / small-M GEMM) on AMD Instinct MI355X (gfx950).
 *
 * The operation.  A weight matrix W with N rows (outputs) and K columns
 * (inputs) is stored as packed integer codes q[n][k] plus per-group scale
 * material; rows are [out][in], as the FFN key (16384x4096) and FFN value
 * (4096x16384) of a width-4096 RWKV-7 model are listed on the package page
 * "RWKV-7 FP8 Quantized Inference" (section "Operator Optimization Details").
 * Five storage formats are supported:
 *
 *   RQ_LAYOUT_SYM, bits = 4, group in {32, 64, 128}
 *       The 4-bit symmetric format with one scale per group of consecutive
 *       weights of a row; group 64 is the format of the model card
 *       "RWKV-7 G1 1.5B -- int4 GPTQ for rwkv-sglang" (opening paragraph,
 *       section "Format & loading").  qweight: uint8 [N][K/2], two codes per
 *       byte, the even k in bits 0-3, each code a 4-bit two's complement
 *       integer (-8..7).  scales: IEEE binary16 [N][K/group].  w = s * q.
 *   RQ_LAYOUT_SYM, bits = 8, group in {16, 32, 64}
 *       The 8-bit symmetric projection format of the REDUCTION preset (group
 *       16) in the news article "rwkv-quant: keeping one matrix in bf16 ..."
 *       (section "Two presets and six sizes").  qweight: int8 [N][K] two's
 *       complement.  scales: binary16 [N][K/group].  w = s * q.
 *   RQ_LAYOUT_ASYM_SB, bits = 4, group = 32
 *       The 4-bit asymmetric superblock projection format of the COMPRESSION
 *       preset (same article and section): each 32-wide group has its own
 *       scale and shift.  qweight: uint8 [N][K/2], unsigned codes 0..15, even
 *       k in bits 0-3.  A superblock is 256 consecutive k of one row (eight
 *       groups).  scales: [N][K/256] records of 8 bytes: binary16 d in bytes
 *       0-1 (little endian), then eight 6-bit unsigned sub-scales sc_j packed
 *       LSB-first in the 48-bit little-endian field of bytes 2-7 (sc_j at bits
 *       6j..6j+5).  zeros: records of the same shape holding m and the
 *       sub-mins mn_j.  With j = (k mod 256)/32:
 *       w = (d * sc_j) * q - (m * mn_j).
 *   RQ_LAYOUT_ASYM_SB, bits = 5 or 6, group = 32
 *       The same superblock layout with 5- or 6-bit unsigned codes (0..31,
 *       0..63): the FFN key and head in 5 bits (COMPRESSION) and the FFN in
 *       6 bits (REDUCTION), same article and section; the pages give the
 *       widths only, the storage below is ours.  qweight holds two planes: the
 *       low 4 bits of every code exactly as the 4-bit layout stores them
 *       ([N][K/2]), then the high bits, [N][K*(bits-4)/8] bytes: per row, per
 *       32-code chunk, 1 (5-bit) or 2 (6-bit) little-endian dwords.  Code
 *       8i + j of a chunk (i = 0..3, j = 0..7), with base = (j >= 4 ? 16 : 0)
 *       + (j even ? 4 : 8) and g = (j mod 4)/2, keeps bit 4 at bit
 *       base + (g == 0 ? i - 4 : i + 4) of the dword (5-bit), or bits 4 and 5
 *       at bits base + s and base + 1 + s of dword i/2 with s = -4, -2, 4, 6
 *       for (i mod 2, g) = (0,0), (0,1), (1,0), (1,1) (6-bit).
 *   RQ_LAYOUT_FP8_TENSOR, bits = 8, group = 0
 *       FP8 E4M3 weights with one binary32 scale for the whole matrix, the
 *       format of the package page "RWKV-7 FP8 Quantized Inference" (sections
 *       "Core Approach: Full FP8, No Residuals" and "Quantization Principle";
 *       the scale is fp32 per section "Quantization Metadata Format"), used
 *       here as weight-only quantization (binary16 activations).  qweight:
 *       uint8 [N][K], each byte an OCP E4M3 value (bias 7, 3 fraction bits,
 *       subnormals, no infinities, S.1111.111 = NaN, largest finite 448).
 *       scales: one float (binary32).  zeros: NULL.  w = fp8 * scale.
 *
 * Every dequantized weight is the binary32 value nearest (ties to even) the
 * exact value of its formula; for these formats that value is the same however
 * the products are grouped, so there is exactly one right answer.
 *
 * Pointers.  Every pointer is device memory owned by the caller and must be
 * 16-byte aligned.  Each operand (packed codes, scales, x, y) must be smaller
 * than 2 GiB (RQ_ERR_SHAPE otherwise).  The library never allocates or frees
 * device memory, does not retain caller memory between calls (a workspace
 * is passed in: rq_gemm_smallm_ws), never copies to the host and never
 * synchronizes: work is
 * enqueued on `stream`
 * (a hipStream_t; NULL means the null stream) and the call returns after the
 * enqueue.  Outputs must not overlap any input.
 *
 * Errors.  Arguments are validated on the host before any HIP call, so a call
 * that returns an error other than RQ_ERR_LAUNCH or RQ_ERR_DEVICE has
 * enqueued nothing.  A kernel fault is reported by the caller's next
 * synchronization, as for any asynchronous HIP work.  No exception crosses
 * this interface and nothing is printed.
 */
#ifndef RQ_H
#define RQ_H

#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    RQ_OK = 0,
    RQ_ERR_NULL = 1,        /* a required pointer is NULL                       */
    RQ_ERR_SHAPE = 2,       /* M, N, K or group violate the shape rules         */
    RQ_ERR_UNSUPPORTED = 3, /* (layout, bits, group, out_kind) not supported    */
    RQ_ERR_ALIGN = 4,       /* a pointer is not 16-byte aligned                 */
    RQ_ERR_LAUNCH = 5,      /* the kernel launch was rejected by the runtime    */
    RQ_ERR_ALIAS = 6,       /* an output range overlaps an input range          */
    RQ_ERR_DEVICE = 7,      /* no usable gfx950 device                           */
    RQ_ERR_SCRATCH = 8      /* the split-K partial sums would not fit the
                               caller's workspace (rq_gemm_smallm_ws) or the
                               fixed array (rq_gemm_smallm_noalloc)              */
} rq_status;

typedef enum { RQ_LAYOUT_SYM = 0, RQ_LAYOUT_ASYM_SB = 1, RQ_LAYOUT_FP8_TENSOR = 2 } rq_layout;

typedef enum {
    RQ_OUT_F32 = 0,     /* binary32 weights [N][K]                               */
    RQ_OUT_CODES_I8 = 1 /* the integer codes as int8 [N][K]: -8..7 (4-bit sym),
                           -128..127 (8-bit), 0..15 (asymmetric)                 */
} rq_out_kind;

/* Largest M accepted by rq_gemv, rq_gemv_batched and rq_gemm_smallm. */
#define RQ_MAX_M 64

/* Largest number of problems in one rq_gemv_batched call. */
#define RQ_MAX_BATCH 64

/* One product y = x W^T of rq_gemv_batched (pointers as for rq_gemv). */
typedef struct {
    const void* qweight;
    const void* scales;
    const void* zeros;
    const void* x; /* binary16 [M][K] */
    float* y;      /* float [M][N], overwritten */
    int N;
    int K;
} rq_problem;

/*
 * rq_dequant -- unpack the codes of W, or dequantize W to binary32.
 * Defines the dequantization of the formats above (the model card's accuracy
 * paragraph reports that the serving kernel reproduces the offline dequant bit
 * for bit; this call is that offline dequant).
 *   out: RQ_OUT_F32 -> float [N][K]; RQ_OUT_CODES_I8 -> int8 [N][K] (not for
 *   RQ_LAYOUT_FP8_TENSOR, whose codes are not integers: RQ_ERR_UNSUPPORTED).
 *   zeros: NULL for RQ_LAYOUT_SYM and RQ_LAYOUT_FP8_TENSOR, required for
 *   RQ_LAYOUT_ASYM_SB.
 * Shape rules: N >= 1, K >= 1, K % group == 0 (group > 0), K*bits/8 % 16 == 0,
 * and for the asymmetric layout K % 256 == 0.
 */
rq_status rq_dequant(const void* qweight, const void* scales, const void* zeros,
                     void* out, int N, int K, int bits, int group, int layout,
                     int out_kind, void* stream);

/*
 * rq_gemv -- y[m][n] = sum_k x[m][k] * w[n][k] for 1 <= M <= RQ_MAX_M, where w
 * is the dequantized weight above (the weight-only decode product whose speed
 * the model card reports against fp16, section "Speed").
 *   x: binary16 [M][K] row-major.  y: float [M][N] row-major, overwritten.
 * Each output is within 1e-3 * sum_k |x[m][k] * w[n][k]| of the exact value
 * (fp32 accumulation).  The kernel is chosen per M, format and shape:
 * vector units at M <= 2 (a matrix-core kernel where K is too long for their
 * tuned launch shapes); from M = 3 on the small-batch matrix-core kernel of
 * rq_gemm_smallm (4 or 8 activation rows staged for M <= 4 or 8, else M
 * padded to a multiple of 16), or the matrix-core decode kernel where the
 * former does not take K and for one measured RWKV-7 shape at M = 3..4
 * (4-bit asymmetric 10240x2560); the vector units, in passes of up to 8
 * rows, wherever K suits neither and for one measured shape at M = 3..4
 * (int4 g64 2048x8192).  The small-batch kernel runs here with K whole:
 * this entry point never allocates or synchronizes.
 * Shape rules as for rq_dequant, plus 1 <= M <= RQ_MAX_M.
 */
rq_status rq_gemv(const void* qweight, const void* scales, const void* zeros,
                  const void* x, float* y, int M, int N, int K, int bits,
                  int group, int layout, void* stream);

/*
 * rq_gemv_batched -- `count` independent products, issued as few kernel
 * launches as possible: problems with the same K share one launch (up to 16
 * per launch on the vector-unit and decode kernels, up to 8 on the
 * small-batch matrix-core kernel).  Each group takes the kernel rq_gemv
 * would take for M, its K and its total row count; K is never split.
 * This is the grouped
 * form of the decode step's independent projections -- the package page
 * "RWKV-7 FP8 Quantized Inference" (section "Operator Optimization Details")
 * computes the receptance, key and value projections of a layer in a single
 * kernel.  All problems share M, bits, group and layout; N, K and the
 * pointers are per problem.  `problems` is a host array the call reads before
 * it returns.  No output may overlap another output or any input.
 * Errors as for rq_gemv; a failed call enqueues nothing.
 */
rq_status rq_gemv_batched(const rq_problem* problems, int count, int M, int bits,
                          int group, int layout, void* stream);

/*
 * rq_gemm_smallm -- the same product and contract as rq_gemv, computed on the
 * matrix cores (fp16 MFMA on exact integer or FP8 codes, fp32 per-group
 * scaling; FP8 sums are scaled once by the matrix scale).  This is the
 * batched-decode member of the kernel family the model card "RWKV-7 G1 1.5B --
 * int4 GPTQ for rwkv-sglang" names in its "Speed" line (a small-M GEMM next
 * to the GEMV, credited with beating fp16 at every batch up to 32).  Every
 * layout and code width, 5- and 6-bit codes included.
 * Tuned for 16 <= M <= 64 (batched decode); for M <= 4 or 8 only 4 or 8
 * activation rows are staged per round, otherwise M is padded to a multiple
 * of 16; it beats the vector units from M = 3 on.
 * This entry point keeps K whole: it has no workspace, and the library never
 * allocates, frees or synchronizes.  rq_gemm_smallm_ws below is the same call
 * with a caller-owned workspace, through which K may be split.
 */
rq_status rq_gemm_smallm(const void* qweight, const void* scales, const void* zeros,
                         const void* x, float* y, int M, int N, int K, int bits,
                         int group, int layout, void* stream);

/* The most workspace rq_gemm_smallm_ws ever uses (split-K arrival counters
 * and partial sums); a workspace of this size suits every call. */
#define RQ_GEMM_WORKSPACE_MAX_BYTES (64 << 20)

/*
 * rq_gemm_smallm_workspace_size -- *bytes = the workspace rq_gemm_smallm_ws
 * uses at these arguments: 0 where K is kept whole, at most
 * RQ_GEMM_WORKSPACE_MAX_BYTES.  Host-only (no device call); shape rules and
 * errors as for rq_gemm_smallm.
 */
rq_status rq_gemm_smallm_workspace_size(int M, int N, int K, int bits, int group,
                                        int layout, size_t* bytes);

/*
 * rq_gemm_smallm_ws -- rq_gemm_smallm with a workspace owned by the caller.
 * For long rows at small row counts the kernel splits K across workgroups
 * (more rows share each staged copy of x); the partial sums then go through
 * `workspace`, and the last workgroup to finish a 16-row tile adds them in a
 * fixed order, so results are deterministic.
 *   workspace: device memory, 16-byte aligned, of workspace_bytes bytes; the
 *   bytes the call uses (the size rq_gemm_smallm_workspace_size reports) must
 *   overlap no input and not y (RQ_ERR_ALIAS).  Its first 64 KiB (the arrival counters)
 *   must be zero before its first use; every call leaves them zero again, and
 *   the rest needs no clearing.  NULL keeps K whole (then workspace_bytes is
 *   ignored).
 * Errors as for rq_gemm_smallm, plus RQ_ERR_SCRATCH when a non-NULL workspace
 * is smaller than rq_gemm_smallm_workspace_size reports (nothing enqueued).
 * Calls that share one workspace must not overlap in time (calls on one
 * stream are ordered; graphs holding the same workspace must not be replayed
 * concurrently).  The library never allocates, frees or synchronizes.
 */
rq_status rq_gemm_smallm_ws(const void* qweight, const void* scales, const void* zeros,
                            const void* x, float* y, int M, int N, int K, int bits,
                            int group, int layout, void* workspace, size_t workspace_bytes,
                            void* stream);

/* Bytes of the fixed device array behind rq_gemm_smallm_noalloc. */
#define RQ_NOALLOC_SCRATCH_BYTES ((8 << 20) + (64 << 10))

/*
 * rq_gemm_smallm_noalloc -- rq_gemm_smallm for callers that cannot allocate
 * device memory (code under graph capture, tight serving loops, harnesses
 * that forbid allocation): the arguments of rq_gemm_smallm and the kernels,
 * arrangement, K split and results (bit for bit) of rq_gemm_smallm_ws with an
 * ample workspace, but the split-K arrival counters and
 * partial sums go to a fixed device array of RQ_NOALLOC_SCRATCH_BYTES that
 * the library holds on each GPU it runs on until the process ends.  The call
 * never allocates, frees or synchronizes.  The array covers every split the
 * automatic choice makes; a call whose partial sums would exceed it (only
 * with a forced split count) returns RQ_ERR_SCRATCH and enqueues nothing.
 * Every partial sum is written before it is read and every launch leaves the
 * counters at zero, so nothing needs clearing between calls, but all calls
 * on one GPU share the array: calls that may overlap in time on one GPU (on
 * different streams, or graphs replayed concurrently) race on it.
 */
rq_status rq_gemm_smallm_noalloc(const void* qweight, const void* scales, const void* zeros,
                                 const void* x, float* y, int M, int N, int K, int bits,
                                 int group, int layout, void* stream);

/* A static, NUL-terminated English description of a status value. */
const char* rq_status_string(int status);

/* Interface version: (major << 16) | minor. */
int rq_version(void);

#ifdef __cplusplus
}
#endif

#endif /* RQ_H */
