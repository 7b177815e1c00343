/*
 * rq_oracle.h -- host-only interface of the CPU oracle (test infrastructure).
 *
 * Every pointer is host memory owned by the caller.  Functions return 0 on
 * success and 1 on a bad argument.  Nothing here is used by the GPU library.
 * Layout values: 0 = symmetric, 1 = asymmetric superblock (groups of 32,
 * superblocks of 256), 2 = FP8 E4M3 codes with one binary32 scale for the
 * matrix (bits 8, group 0).  Binary16 values are passed as their raw uint16
 * bits.
 */
#ifndef RQ_ORACLE_H
#define RQ_ORACLE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

double rqo_half_to_double(uint16_t h);
double rqo_fp8_to_double(uint8_t b);
int rqo_code_at(const uint8_t* qweight, int N, int K, int bits, int layout,
                int n, int k);
int rqo_unpack_codes(const uint8_t* qweight, int N, int K, int bits, int layout,
                     int8_t* codes);
int rqo_pack_codes(const int8_t* codes, int N, int K, int bits, int layout,
                   uint8_t* qweight);
int rqo_pack_record(uint16_t base_bits, const uint8_t sub[8], uint8_t out[8]);
int rqo_unpack_record(const uint8_t rec[8], uint16_t* base_bits, uint8_t sub[8]);
int rqo_dequant(const uint8_t* qweight, const void* scales, const void* zeros,
                int N, int K, int bits, int group, int layout, float* out);
int rqo_gemv_ref(const uint8_t* qweight, const void* scales, const void* zeros,
                 const uint16_t* x, int M, int N, int K, int bits, int group,
                 int layout, int n0, int n1, double* y_ref, double* bound);
long rqo_check(const float* y, const double* y_ref, const double* bound,
               long count, double rtol, long* first_bad, double* worst);
int rqo_version(void);

#ifdef __cplusplus
}
#endif

#endif
