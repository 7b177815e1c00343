/*
 * rq_oracle.cpp -- plain, slow, single-threaded CPU oracle for group-wise
 * low-bit weight dequantization and the dequantize-and-multiply matvec.
 *
 * THIS IS TEST INFRASTRUCTURE.  Only the test suite, the smoke check and the
 * CPU-baseline leg of the benchmark may load it.  The GPU library never links,
 * includes or calls anything in this directory, and this file includes nothing
 * from the GPU library: the two share no code, headers, tables or helpers.
 *
 * What it computes, and which passage fixes each step:
 *
 *   Formats.
 *   - 4-bit symmetric codes with one scale per 64 consecutive weights of a
 *     row, stored as a packed code tensor plus a scale tensor (model card
 *     "RWKV-7 G1 1.5B -- int4 GPTQ for rwkv-sglang", opening paragraph and
 *     section "Format & loading").
 *   - 8-bit symmetric codes with one scale per 16 weights: the projection
 *     format of the REDUCTION preset (news article "rwkv-quant: keeping one
 *     matrix in bf16 ...", section "Two presets and six sizes").
 *   - 4-bit asymmetric codes in superblocks of 32-wide groups, each group
 *     with its own scale and shift: the projection format of the COMPRESSION
 *     preset (same article and section).
 *   - 5- and 6-bit codes: the same presets keep the FFN in 6 bits (REDUCTION)
 *     and the FFN key and the head in 5 bits (COMPRESSION) (same section).
 *   - 8-bit floating-point codes, FP8 E4M3 ("float8_e4m3fn"), one binary32
 *     scale for the whole matrix: w = fp8 * scale (package page "RWKV-7 FP8
 *     Quantized Inference", sections "Core Approach: Full FP8, No Residuals"
 *     and "Quantization Principle"; the scale dtype is fp32 per the metadata
 *     table of section "Quantization Metadata Format").
 *   - Weight matrices are stored [out][in]: the FFN key of a width-4096 model
 *     is 16384x4096 and the FFN value 4096x16384 (package page
 *     "RWKV-7 FP8 Quantized Inference", section "Operator Optimization
 *     Details", tile table).  So W is [N][K] and y = x * W^T.
 *
 *   Readings taken where the pages are silent (each is listed with its reason
 *   in the design notes of the repository):
 *   - two 4-bit codes per byte, the even k in the low nibble;
 *   - symmetric 4-bit codes are 4-bit two's complement (-8..7), 8-bit codes
 *     are int8 two's complement; asymmetric 4-bit codes are unsigned (0..15);
 *   - symmetric scales are IEEE binary16, one per group, row-major [N][K/g];
 *   - an asymmetric superblock is 256 consecutive k of one row holding eight
 *     32-wide groups; its scale record is 8 bytes: a binary16 superblock scale
 *     d (bytes 0-1, little endian) and eight 6-bit unsigned sub-scales sc_j in
 *     a 48-bit little-endian field (bytes 2-7, sc_j at bits 6j..6j+5).  The
 *     zero record has the same shape with the superblock min m and sub-mins
 *     mn_j.  The weight is w = (d*sc_j)*q - (m*mn_j);
 *   - 5- and 6-bit codes use the asymmetric superblock layout above (the
 *     layout the pages attach to their sub-8-bit codes), unsigned
 *     0..2^bits-1.  qweight holds two planes: the low 4 bits of every code
 *     exactly as the 4-bit layout stores them ([N][K/2]), then the high
 *     bits, [N][K*(bits-4)/8] bytes, in the order given at hi_bit_position
 *     below (the pages give only the widths; this order is ours);
 *   - dequantized weights are binary32, correctly rounded from the exact
 *     value; the model card's accuracy paragraph reports that its kernel
 *     reproduces the offline dequantization bit for bit, so the dequantized
 *     weights have one right answer;
 *   - FP8 E4M3 is the OCP encoding: exponent bias 7, 3 fraction bits,
 *     subnormals, no infinities, S.1111.111 is NaN (max finite 448, the value
 *     the page's per-tensor scale divides by).  The weight is the binary32
 *     product fp8 * scale, rounded once (both factors are exact binary64s and
 *     their product has at most 4 + 24 significant bits);
 *   - the matvec accumulates x*w in binary64, in k order, and also returns
 *     bound = sum_k |x*w|, against which results are judged:
 *     |y - y_ref| <= rtol * bound.
 *
 * Every function is written for a reader to check by eye; none is tuned.
 */
#include "rq_oracle.h"

#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

/* Layout and status values of the interface the oracle checks. */
enum { LAYOUT_SYM = 0, LAYOUT_ASYM_SB = 1, LAYOUT_FP8_TENSOR = 2 };
enum { OK = 0, BAD_ARG = 1 };

static const int SUPERBLOCK = 256; /* k per asymmetric superblock  */
static const int SB_GROUP = 32;    /* k per asymmetric group         */
static const int RECORD_BYTES = 8; /* bytes per superblock record    */

/* ------------------------------------------------------------------------ */
/* IEEE 754 binary16 -> binary64, exact.                                     */
/* A binary16 has 1 sign bit, 5 exponent bits (bias 15) and 10 fraction bits. */
/* Normal:    (-1)^s * (1024 + f) * 2^(e - 25)                              */
/* Subnormal: (-1)^s * f * 2^-24                                            */
/* ------------------------------------------------------------------------ */
double rqo_half_to_double(uint16_t h) {
    int s = (h >> 15) & 1;
    int e = (h >> 10) & 0x1F;
    int f = h & 0x3FF;
    double v;
    if (e == 0) {
        v = ldexp((double)f, -24);
    } else if (e == 31) {
        v = (f == 0) ? INFINITY : NAN;
    } else {
        v = ldexp((double)(1024 + f), e - 25);
    }
    return s ? -v : v;
}

/* ------------------------------------------------------------------------ */
/* OCP FP8 E4M3 -> binary64, exact.                                          */
/* 1 sign bit, 4 exponent bits (bias 7), 3 fraction bits; no infinities.     */
/* Normal:    (-1)^s * (8 + f) * 2^(e - 10)                                  */
/* Subnormal: (-1)^s * f * 2^-9                                             */
/* e = 15 with f = 7 is NaN.                                                */
/* ------------------------------------------------------------------------ */
double rqo_fp8_to_double(uint8_t b) {
    int s = (b >> 7) & 1;
    int e = (b >> 3) & 0x0F;
    int f = b & 0x07;
    double v;
    if (e == 15 && f == 7) {
        v = NAN;
    } else if (e == 0) {
        v = ldexp((double)f, -9);
    } else {
        v = ldexp((double)(8 + f), e - 10);
    }
    return s ? -v : v;
}

/* ------------------------------------------------------------------------ */
/* High bits of 5- and 6-bit codes.  A row's high plane is a run of 32-code  */
/* chunks (chunk c holds codes 32c..32c+31) of 4 bytes (5-bit) or 8 bytes    */
/* (6-bit), read as little-endian 32-bit words.  In a chunk, code 8i + j     */
/* (i = 0..3, j = 0..7) has                                                  */
/*   base = (j >= 4 ? 16 : 0) + (j even ? 4 : 8),   g = (j mod 4) / 2;       */
/*   5-bit: bit 4 of the code in word 0 at bit base + (g == 0 ? i - 4 : i + 4); */
/*   6-bit: bits 4 and 5 in word i/2 at bits base + s and base + 1 + s, with */
/*          s = -4, -2, 4, 6 for (i mod 2, g) = (0,0), (0,1), (1,0), (1,1).  */
/* Returns the bit position of code bit 4 + b; *word gets the word index.    */
/* ------------------------------------------------------------------------ */
static int hi_bit_position(int bits, int c, int b, int* word) {
    int i = c / 8, j = c % 8, g = (j % 4) / 2;
    int base = (j >= 4 ? 16 : 0) + (j % 2 == 0 ? 4 : 8);
    if (bits == 5) {
        *word = 0;
        return base + (g == 0 ? i - 4 : i + 4);
    }
    static const int s6[2][2] = {{-4, -2}, {4, 6}};
    *word = i / 2;
    return base + b + s6[i % 2][g];
}

/* Byte offset of row n's high plane within qweight. */
static size_t hi_plane_row(int N, int K, int bits, int n) {
    return (size_t)N * (K / 2) + (size_t)n * ((size_t)K * (bits - 4) / 8);
}

/* ------------------------------------------------------------------------ */
/* Code decode: the integer code q[n][k].                                    */
/* ------------------------------------------------------------------------ */
int rqo_code_at(const uint8_t* qweight, int N, int K, int bits, int layout,
                int n, int k) {
    if (bits == 5 || bits == 6) {
        /* low 4 bits as in the 4-bit layout, high bits from the second plane */
        int q = rqo_code_at(qweight, N, K, 4, LAYOUT_ASYM_SB, n, k);
        const uint8_t* chunk = qweight + hi_plane_row(N, K, bits, n) +
                               (size_t)(k / 32) * 4 * (bits - 4);
        for (int b = 0; b < bits - 4; b++) {
            int word;
            int pos = hi_bit_position(bits, k % 32, b, &word);
            const uint8_t* w = chunk + 4 * word;
            uint32_t v = (uint32_t)w[0] | ((uint32_t)w[1] << 8) |
                         ((uint32_t)w[2] << 16) | ((uint32_t)w[3] << 24);
            q |= (int)((v >> pos) & 1u) << (4 + b);
        }
        return q;
    }
    if (bits == 8) {
        /* one int8 two's-complement code per byte */
        return (int)(int8_t)qweight[(size_t)n * K + k];
    }
    /* two codes per byte, the even k in bits 0-3 and the odd k in bits 4-7 */
    uint8_t byte = qweight[(size_t)n * (K / 2) + k / 2];
    int nibble = (k % 2 == 0) ? (byte & 0x0F) : (byte >> 4);
    if (layout == LAYOUT_SYM) {
        /* 4-bit two's complement: 0..7 -> 0..7, 8..15 -> -8..-1 */
        return (nibble >= 8) ? nibble - 16 : nibble;
    }
    return nibble; /* asymmetric: unsigned 0..15 */
}

static int valid_format(int bits, int group, int layout) {
    if (layout == LAYOUT_SYM) return (bits == 4 || bits == 8) && group > 0;
    if (layout == LAYOUT_ASYM_SB)
        return (bits == 4 || bits == 5 || bits == 6) && group == SB_GROUP;
    if (layout == LAYOUT_FP8_TENSOR) return bits == 8 && group == 0;
    return 0;
}

static int valid_shape(int N, int K, int bits, int group, int layout) {
    if (N < 1 || K < 1 || !valid_format(bits, group, layout)) return 0;
    if (group > 0 && K % group != 0) return 0;
    if (bits == 4 && K % 2 != 0) return 0;
    if (layout == LAYOUT_ASYM_SB && K % SUPERBLOCK != 0) return 0;
    return 1;
}

int rqo_unpack_codes(const uint8_t* qweight, int N, int K, int bits, int layout,
                     int8_t* codes) {
    if (!qweight || !codes) return BAD_ARG;
    if (N < 1 || K < 1 || !(bits == 4 || bits == 5 || bits == 6 || bits == 8)) return BAD_ARG;
    if (bits == 4 && K % 2 != 0) return BAD_ARG;
    if ((bits == 5 || bits == 6) && (layout != LAYOUT_ASYM_SB || K % 32 != 0)) return BAD_ARG;
    if (layout == LAYOUT_ASYM_SB && bits == 8) return BAD_ARG;
    if (layout == LAYOUT_FP8_TENSOR) return BAD_ARG; /* codes are not integers */
    for (int n = 0; n < N; n++)
        for (int k = 0; k < K; k++)
            codes[(size_t)n * K + k] =
                (int8_t)rqo_code_at(qweight, N, K, bits, layout, n, k);
    return OK;
}

int rqo_pack_codes(const int8_t* codes, int N, int K, int bits, int layout,
                   uint8_t* qweight) {
    if (!qweight || !codes) return BAD_ARG;
    if (N < 1 || K < 1 || !(bits == 4 || bits == 5 || bits == 6 || bits == 8)) return BAD_ARG;
    if (bits == 4 && K % 2 != 0) return BAD_ARG;
    if ((bits == 5 || bits == 6) && (layout != LAYOUT_ASYM_SB || K % 32 != 0)) return BAD_ARG;
    if (layout == LAYOUT_ASYM_SB && bits == 8) return BAD_ARG;
    if (layout == LAYOUT_FP8_TENSOR) return BAD_ARG; /* codes are not integers */
    if (bits == 5 || bits == 6) {
        /* low nibbles as in the 4-bit layout, then the high plane */
        memset(qweight, 0, (size_t)N * K * bits / 8);
        for (int n = 0; n < N; n++) {
            for (int k = 0; k < K; k++) {
                int c = codes[(size_t)n * K + k];
                if (c < 0 || c >= (1 << bits)) return BAD_ARG;
                qweight[(size_t)n * (K / 2) + k / 2] |=
                    (uint8_t)((c & 0x0F) << (4 * (k % 2)));
                uint8_t* chunk = qweight + hi_plane_row(N, K, bits, n) +
                                 (size_t)(k / 32) * 4 * (bits - 4);
                for (int b = 0; b < bits - 4; b++) {
                    int word;
                    int pos = hi_bit_position(bits, k % 32, b, &word);
                    if ((c >> (4 + b)) & 1)
                        chunk[4 * word + pos / 8] |= (uint8_t)(1u << (pos % 8));
                }
            }
        }
        return OK;
    }
    if (bits == 8) {
        for (size_t i = 0; i < (size_t)N * K; i++) qweight[i] = (uint8_t)codes[i];
        return OK;
    }
    for (int n = 0; n < N; n++) {
        for (int k = 0; k < K; k += 2) {
            int c0 = codes[(size_t)n * K + k];
            int c1 = codes[(size_t)n * K + k + 1];
            int lo_min = (layout == LAYOUT_SYM) ? -8 : 0;
            int lo_max = (layout == LAYOUT_SYM) ? 7 : 15;
            if (c0 < lo_min || c0 > lo_max || c1 < lo_min || c1 > lo_max)
                return BAD_ARG;
            /* the low 4 bits of a two's-complement int are its nibble */
            int nib0 = c0 & 0x0F;
            int nib1 = c1 & 0x0F;
            qweight[(size_t)n * (K / 2) + k / 2] = (uint8_t)(nib0 | (nib1 << 4));
        }
    }
    return OK;
}

/* ------------------------------------------------------------------------ */
/* Asymmetric superblock record: {binary16 base; eight 6-bit sub-codes}.      */
/* ------------------------------------------------------------------------ */
int rqo_pack_record(uint16_t base_bits, const uint8_t sub[8], uint8_t out[8]) {
    if (!sub || !out) return BAD_ARG;
    uint64_t field = 0;
    for (int j = 0; j < 8; j++) {
        if (sub[j] > 63) return BAD_ARG;
        field |= (uint64_t)sub[j] << (6 * j);
    }
    out[0] = (uint8_t)(base_bits & 0xFF);
    out[1] = (uint8_t)(base_bits >> 8);
    for (int i = 0; i < 6; i++) out[2 + i] = (uint8_t)((field >> (8 * i)) & 0xFF);
    return OK;
}

int rqo_unpack_record(const uint8_t rec[8], uint16_t* base_bits, uint8_t sub[8]) {
    if (!rec || !base_bits || !sub) return BAD_ARG;
    *base_bits = (uint16_t)(rec[0] | (rec[1] << 8));
    uint64_t field = 0;
    for (int i = 0; i < 6; i++) field |= (uint64_t)rec[2 + i] << (8 * i);
    for (int j = 0; j < 8; j++) sub[j] = (uint8_t)((field >> (6 * j)) & 0x3F);
    return OK;
}

/* ------------------------------------------------------------------------ */
/* Scale s and shift t that apply to weight (n, k), as exact binary64 values. */
/* SYM:  s = scales[n][k/group] (binary16), t = 0.                           */
/* ASYM: b = k/256, j = (k%256)/32; s = d*sc_j, t = m*mn_j.                  */
/* FP8:  s = scales[0] (binary32, the whole matrix), t = 0.                  */
/* ------------------------------------------------------------------------ */
static void scale_shift_at(const void* scales, const void* zeros, int K,
                           int group, int layout, int n, int k, double* s,
                           double* t) {
    if (layout == LAYOUT_FP8_TENSOR) {
        *s = (double)((const float*)scales)[0];
        *t = 0.0;
        return;
    }
    if (layout == LAYOUT_SYM) {
        const uint16_t* sc = (const uint16_t*)scales;
        *s = rqo_half_to_double(sc[(size_t)n * (K / group) + k / group]);
        *t = 0.0;
        return;
    }
    int b = k / SUPERBLOCK;
    int j = (k % SUPERBLOCK) / SB_GROUP;
    size_t rec_index = (size_t)n * (K / SUPERBLOCK) + b;
    const uint8_t* srec = (const uint8_t*)scales + rec_index * RECORD_BYTES;
    const uint8_t* zrec = (const uint8_t*)zeros + rec_index * RECORD_BYTES;
    uint16_t d_bits, m_bits;
    uint8_t sc[8], mn[8];
    rqo_unpack_record(srec, &d_bits, sc);
    rqo_unpack_record(zrec, &m_bits, mn);
    *s = rqo_half_to_double(d_bits) * (double)sc[j];
    *t = rqo_half_to_double(m_bits) * (double)mn[j];
}

/* w[n][k] as the binary32 nearest the exact value s*q - t (ties to even).
 * For every binary16 s, t and the code ranges here, s*q - t is an exact
 * binary64 (at most 50 significant bits), so one conversion rounds once.
 * For FP8 codes q is the code's value and s the binary32 matrix scale
 * (product: at most 28 significant bits, exact in binary64). */
static float weight_at(const uint8_t* qweight, const void* scales,
                       const void* zeros, int N, int K, int bits, int group,
                       int layout, int n, int k) {
    double s, t;
    scale_shift_at(scales, zeros, K, group, layout, n, k, &s, &t);
    double q = (layout == LAYOUT_FP8_TENSOR)
                   ? rqo_fp8_to_double(qweight[(size_t)n * K + k])
                   : (double)rqo_code_at(qweight, N, K, bits, layout, n, k);
    double exact = s * q - t;
    return (float)exact;
}

int rqo_dequant(const uint8_t* qweight, const void* scales, const void* zeros,
                int N, int K, int bits, int group, int layout, float* out) {
    if (!qweight || !scales || !out) return BAD_ARG;
    if (layout == LAYOUT_ASYM_SB && !zeros) return BAD_ARG;
    if (!valid_shape(N, K, bits, group, layout)) return BAD_ARG;
    for (int n = 0; n < N; n++)
        for (int k = 0; k < K; k++)
            out[(size_t)n * K + k] = weight_at(qweight, scales, zeros, N, K,
                                               bits, group, layout, n, k);
    return OK;
}

/* ------------------------------------------------------------------------ */
/* Matvec over rows [n0, n1):                                               */
/*   y_ref[m][n] = sum_k x[m][k] * w[n][k]      (binary64, k ascending)      */
/*   bound[m][n] = sum_k |x[m][k] * w[n][k]|                                  */
/* x is binary16 [M][K]; y_ref and bound are [M][N]; only rows n0..n1-1 are   */
/* written.                                                                 */
/* ------------------------------------------------------------------------ */
int rqo_gemv_ref(const uint8_t* qweight, const void* scales, const void* zeros,
                 const uint16_t* x, int M, int N, int K, int bits, int group,
                 int layout, int n0, int n1, double* y_ref, double* bound) {
    if (!qweight || !scales || !x || !y_ref || !bound) return BAD_ARG;
    if (layout == LAYOUT_ASYM_SB && !zeros) return BAD_ARG;
    if (!valid_shape(N, K, bits, group, layout) || M < 1) return BAD_ARG;
    if (n0 < 0 || n1 > N || n0 > n1) return BAD_ARG;

    double* xd = (double*)malloc(sizeof(double) * (size_t)M * K);
    float* wrow = (float*)malloc(sizeof(float) * (size_t)K);
    if (!xd || !wrow) {
        free(xd);
        free(wrow);
        return BAD_ARG;
    }
    for (size_t i = 0; i < (size_t)M * K; i++) xd[i] = rqo_half_to_double(x[i]);

    for (int n = n0; n < n1; n++) {
        for (int k = 0; k < K; k++)
            wrow[k] = weight_at(qweight, scales, zeros, N, K, bits, group,
                                layout, n, k);
        for (int m = 0; m < M; m++) {
            double acc = 0.0, mag = 0.0;
            for (int k = 0; k < K; k++) {
                double p = xd[(size_t)m * K + k] * (double)wrow[k];
                acc += p;
                mag += fabs(p);
            }
            y_ref[(size_t)m * N + n] = acc;
            bound[(size_t)m * N + n] = mag;
        }
    }
    free(xd);
    free(wrow);
    return OK;
}

/* ------------------------------------------------------------------------ */
/* Pass criterion: |y - y_ref| <= rtol * bound for every element; where      */
/* bound is 0, y must be +0 or -0; a NaN or an infinity fails.               */
/* Returns the number of failing elements; *first_bad gets the first failing */
/* index (or -1) and *worst the largest |y - y_ref| / bound seen (0 where    */
/* bound is 0 and y is zero).                                                */
/* ------------------------------------------------------------------------ */
long rqo_check(const float* y, const double* y_ref, const double* bound,
               long count, double rtol, long* first_bad, double* worst) {
    long bad = 0;
    double w = 0.0;
    long first = -1;
    for (long i = 0; i < count; i++) {
        double yi = (double)y[i];
        int ok;
        double ratio;
        if (isnan(yi) || isinf(yi)) {
            ok = 0;
            ratio = INFINITY;
        } else if (bound[i] == 0.0) {
            ok = (yi == 0.0);
            ratio = ok ? 0.0 : INFINITY;
        } else {
            double err = fabs(yi - y_ref[i]);
            ratio = err / bound[i];
            ok = (err <= rtol * bound[i]);
        }
        if (ratio > w) w = ratio;
        if (!ok) {
            if (first < 0) first = i;
            bad++;
        }
    }
    if (first_bad) *first_bad = first;
    if (worst) *worst = w;
    return bad;
}

int rqo_version(void) { return 1; }
