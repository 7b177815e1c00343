// rq_common.h -- device helpers shared by the librq kernels (gfx950 only).
//
// Internal to librq.  Formats and readings are stated in include/rq.h.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace rq {

typedef uint32_t u32;
typedef _Float16 h2 __attribute__((ext_vector_type(2)));
typedef _Float16 h4 __attribute__((ext_vector_type(4)));
typedef _Float16 h8 __attribute__((ext_vector_type(8)));
typedef float f4 __attribute__((ext_vector_type(4)));
typedef u32 u32x2 __attribute__((ext_vector_type(2)));
typedef u32 u32x4 __attribute__((ext_vector_type(4)));

// Format ids of the kernels (a function of layout and bits).
enum Fmt { FMT_S4 = 0, FMT_S8 = 1, FMT_A4 = 2, FMT_F8 = 3, FMT_A5 = 4, FMT_A6 = 5 };

// Asymmetric superblock layouts: 4-, 5- and 6-bit unsigned codes.
constexpr bool is_asym(int fmt) { return fmt == FMT_A4 || fmt == FMT_A5 || fmt == FMT_A6; }
// Bits of a code above its low nibble (they live in the high-bit plane).
constexpr int hi_bits(int fmt) { return fmt == FMT_A5 ? 1 : (fmt == FMT_A6 ? 2 : 0); }

constexpr int SUPERBLOCK = 256;  // k per asymmetric superblock
constexpr int SB_GROUP = 32;     // k per asymmetric group

// Codes in one 16-byte chunk of a row.
template <int FMT>
struct Chunk {
  static constexpr int codes = (FMT == FMT_S8 || FMT == FMT_F8) ? 16 : 32;
};

__device__ __forceinline__ h2 as_h2(u32 v) { return __builtin_bit_cast(h2, v); }
__device__ __forceinline__ u32 as_u32(h2 v) { return __builtin_bit_cast(u32, v); }

// Streaming (read-once) 16-byte load of packed codes.
__device__ __forceinline__ u32x4 load_stream16(const void* p) {
  return __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
}
__device__ __forceinline__ u32x2 load_stream8(const void* p) {
  return __builtin_nontemporal_load(reinterpret_cast<const u32x2*>(p));
}
__device__ __forceinline__ u32 load_stream4(const void* p) {
  return __builtin_nontemporal_load(reinterpret_cast<const u32*>(p));
}

// ---------------------------------------------------------------------------
// Exact code -> binary16 conversion.
//
// A 4-bit value u placed in the low mantissa bits of 0x6400 (= 1024.0) gives
// the binary16 number 1024 + u; in bits 4-7 it gives 1024 + 16u.  Both are
// exact, and so are (1024 + u) - c and (1024 + 16u)/16 - c for the small
// integer c used below, so every code reaches fp16 without rounding.
// ---------------------------------------------------------------------------

// One dword of 4-bit codes, k = 0..7 in nibbles 0..7 (even k low).  Returns
// the pairs (q0,q4) (q1,q5) (q2,q6) (q3,q7) as binary16.  SIGNED selects 4-bit
// two's complement codes (-8..7); otherwise codes are unsigned (0..15).
template <bool SIGNED>
__device__ __forceinline__ void unpack4(u32 d, h2 q[4]) {
  // (d & mask) ^ key: the AND keeps one nibble per half-word, the XOR both
  // flips the two's-complement sign bit (q -> q + 8) and sets the exponent
  // bits of 1024.0 (they lie outside the mask) -- one three-input bit op.
  const u32 lo = 0x000F000Fu, hi = 0x00F000F0u;
  const u32 key_lo = SIGNED ? 0x64086408u : 0x64006400u;
  const u32 key_hi = SIGNED ? 0x64806480u : 0x64006400u;
  const u32 d2 = d >> 8;
  const u32 t0 = (d & lo) ^ key_lo;   // 1024 + u0, 1024 + u4
  const u32 t1 = (d & hi) ^ key_hi;   // 1024 + 16 u1, 1024 + 16 u5
  const u32 t2 = (d2 & lo) ^ key_lo;  // 1024 + u2, 1024 + u6
  const u32 t3 = (d2 & hi) ^ key_hi;  // 1024 + 16 u3, 1024 + 16 u7
  const _Float16 b0 = SIGNED ? (_Float16)-1032.0f : (_Float16)-1024.0f;
  const _Float16 b1 = SIGNED ? (_Float16)-72.0f : (_Float16)-64.0f;
  const h2 bias0 = {b0, b0};
  const h2 bias1 = {b1, b1};
  const h2 sixteenth = {(_Float16)0.0625f, (_Float16)0.0625f};
  q[0] = as_h2(t0) + bias0;
  q[1] = __builtin_elementwise_fma(as_h2(t1), sixteenth, bias1);
  q[2] = as_h2(t2) + bias0;
  q[3] = __builtin_elementwise_fma(as_h2(t3), sixteenth, bias1);
}

// 5- and 6-bit codes.  The low nibbles are stored as 4-bit codes; the high
// bits of each 32-code chunk (one 16-byte chunk of nibbles) are one dword
// (5-bit) or two (6-bit) of the high-bit plane, in an order chosen so that a
// rotation puts the bits of nibble dword i (codes 8i..8i+7) next to the
// nibbles where unpack4 places them: for the pairs (q0,q4) (q1,q5) at bits
// 4 and 20 (8 and 24) of hlo, for (q2,q6) (q3,q7) likewise in hhi.  In the
// stored plane, code 8i + j has base = (j >= 4 ? 16 : 0) + (j even ? 4 : 8)
// and g = (j mod 4) / 2; 5-bit: bit base + (g == 0 ? i - 4 : i + 4) of the
// chunk's dword; 6-bit: bits base + s and base + 1 + s of dword i / 2, with
// s = -4, -2, 4, 6 for (i mod 2, g) = (0,0), (0,1), (1,0), (1,1).
__device__ __forceinline__ u32 rotr(u32 x, int s) { return __builtin_amdgcn_alignbit(x, x, s); }

template <int HB>
__device__ __forceinline__ void hi_words(const u32* w, int i, u32* hlo, u32* hhi) {
  if constexpr (HB == 1) {
    *hlo = rotr(w[0], (i + 28) & 31);  // shift i - 4
    *hhi = rotr(w[0], i + 4);
  } else {
    const u32 p = w[i >> 1];
    *hlo = rotr(p, (i & 1) ? 4 : 28);  // -4 or 4
    *hhi = rotr(p, (i & 1) ? 6 : 30);  // -2 or 6
  }
}

// One dword of nibbles of unsigned 5-/6-bit codes with their high bits in
// hlo/hhi (hi_words).  Pairs as unpack4: (q0,q4) (q1,q5) (q2,q6) (q3,q7).  The
// high bits join the nibble inside the binary16 mantissa: 1024 + q, or
// 1024 + 16 q for the nibbles held in bits 4-7, both exact for q < 64.
template <int HB>
__device__ __forceinline__ void unpack4h(u32 d, u32 hlo, u32 hhi, h2 q[4]) {
  const u32 lo = 0x000F000Fu, hi = 0x00F000F0u, key = 0x64006400u;
  const u32 m0 = HB == 1 ? 0x00100010u : 0x00300030u;
  const u32 m1 = HB == 1 ? 0x01000100u : 0x03000300u;
  const u32 d2 = d >> 8;
  const u32 t0 = ((d & lo) | key) | (hlo & m0);
  const u32 t1 = ((d & hi) | key) | (hlo & m1);
  const u32 t2 = ((d2 & lo) | key) | (hhi & m0);
  const u32 t3 = ((d2 & hi) | key) | (hhi & m1);
  const h2 bias0 = {(_Float16)-1024.0f, (_Float16)-1024.0f};
  const h2 bias1 = {(_Float16)-64.0f, (_Float16)-64.0f};
  const h2 sixteenth = {(_Float16)0.0625f, (_Float16)0.0625f};
  q[0] = as_h2(t0) + bias0;
  q[1] = __builtin_elementwise_fma(as_h2(t1), sixteenth, bias1);
  q[2] = as_h2(t2) + bias0;
  q[3] = __builtin_elementwise_fma(as_h2(t3), sixteenth, bias1);
}

// The same dword, pairs in k order: (q0,q1) (q2,q3) (q4,q5) (q6,q7).  A byte
// perm copies byte j of d into both half-words next to the exponent byte of
// 1024.0; the AND keeps the low nibble in the low half and the high nibble in
// the high half (there worth 16u), the XOR flips the sign bits; one packed
// FMA scales the high half by 1/16 and removes both offsets.
template <bool SIGNED>
__device__ __forceinline__ void unpack4n(u32 d, h2 q[4]) {
  const u32 flip = SIGNED ? 0x00800008u : 0u;
  const _Float16 b0 = SIGNED ? (_Float16)-1032.0f : (_Float16)-1024.0f;
  const _Float16 b1 = SIGNED ? (_Float16)-72.0f : (_Float16)-64.0f;
  const h2 mul = {(_Float16)1.0f, (_Float16)0.0625f};
  const h2 add = {b0, b1};
#pragma unroll
  for (int j = 0; j < 4; j++) {
    // bytes (high to low): 0x64, d.byte j, 0x64, d.byte j
    const u32 w = __builtin_amdgcn_perm(0x64646464u, d, 0x04000400u | (j << 16) | j);
    const u32 t = (w & 0xFFF0FF0Fu) ^ flip;  // 1024 + u_lo | 1024 + 16 u_hi
    q[j] = __builtin_elementwise_fma(as_h2(t), mul, add);
  }
}

// One dword of int8 codes, k = 0..3 in bytes 0..3.  Returns (q0,q1) (q2,q3).
// A byte u = q + 128 placed in the low 8 mantissa bits of 0x6400 is 1024 + u.
__device__ __forceinline__ void unpack8(u32 d, h2 q[2]) {
  d ^= 0x80808080u;  // two's complement byte -> q + 128
  const u32 t0 = __builtin_amdgcn_perm(0x64646464u, d, 0x04010400u);  // u0 | u1
  const u32 t1 = __builtin_amdgcn_perm(0x64646464u, d, 0x04030402u);  // u2 | u3
  const h2 bias = {(_Float16)-1152.0f, (_Float16)-1152.0f};
  q[0] = as_h2(t0) + bias;
  q[1] = as_h2(t1) + bias;
}

// One dword of FP8 E4M3 codes, k = 0..3 in bytes 0..3.  Returns (q0,q1)
// (q2,q3) in binary16, exactly: every E4M3 value, subnormals included, is a
// binary16 (the conversion's scale operand is 1).
__device__ __forceinline__ void unpack_fp8(u32 d, h2 q[2]) {
  q[0] = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(d, 1.0f, false);
  q[1] = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(d, 1.0f, true);
}

// Activation pairs matching unpack4: from the 8 halves x0..x7 held in four
// dwords w0=(x0,x1) w1=(x2,x3) w2=(x4,x5) w3=(x6,x7) build
// (x0,x4) (x1,x5) (x2,x6) (x3,x7).
__device__ __forceinline__ void pair_x4(u32 w0, u32 w1, u32 w2, u32 w3, h2 p[4]) {
  p[0] = as_h2(__builtin_amdgcn_perm(w2, w0, 0x05040100u));
  p[1] = as_h2(__builtin_amdgcn_perm(w2, w0, 0x07060302u));
  p[2] = as_h2(__builtin_amdgcn_perm(w3, w1, 0x05040100u));
  p[3] = as_h2(__builtin_amdgcn_perm(w3, w1, 0x07060302u));
}

// 64-byte spans of a row in the MFMA B layout.  The four lane quarters of a
// row (l/16 = h) each need G/4 consecutive codes of every group, which for
// groups under 64 bytes is less than one 16-byte load.  So a row is read in
// 64-byte spans, one 16-byte piece per quarter -- quarter h takes piece
// span_piece<SG>(h) -- and the pieces are exchanged across the quarters once
// they have arrived: v_permlane16_swap exchanges a register of lane rows 1
// and 3 with one of rows 0 and 2, v_permlane32_swap one of rows 2, 3 with
// one of rows 0, 1.  SG is the number of groups in a span (64 / group bytes).
template <int SG>
__device__ __forceinline__ int span_piece(int h) {
  return SG == 2 ? ((h & 1) << 1 | (h >> 1)) : h;
}
__device__ __forceinline__ void lane_swap16(u32& x, u32& y) {
  const auto r = __builtin_amdgcn_permlane16_swap(x, y, false, false);
  x = r[0];
  y = r[1];
}
__device__ __forceinline__ void lane_swap32(u32& x, u32& y) {
  const auto r = __builtin_amdgcn_permlane32_swap(x, y, false, false);
  x = r[0];
  y = r[1];
}
// A span's four dwords v[0..3] as loaded -> v[j*DPG + s] = dword s of this
// quarter's share of group j of the span (DPG = 4 / SG dwords).
//  SG = 1: the quarter's piece is its share already.
//  SG = 2: quarters 0..3 hold pieces 0, 2, 1, 3 (group 0 = pieces 0-1, group 1
//          = pieces 2-3); one exchange between quarters 0<->1 and 2<->3 gives
//          quarter h dwords 2h, 2h+1 of each group.
//  SG = 4: quarter u holds group u; a 4x4 transpose across the quarters gives
//          quarter h dword h of each group.
template <int SG>
__device__ __forceinline__ void span_fix(u32* v) {
  if constexpr (SG == 2) {
    lane_swap16(v[0], v[2]);
    lane_swap16(v[1], v[3]);
  } else if constexpr (SG == 4) {
    lane_swap16(v[0], v[1]);
    lane_swap16(v[2], v[3]);
    lane_swap32(v[0], v[2]);
    lane_swap32(v[1], v[3]);
  }
}

// Exact binary16 -> binary32 of the low / high half of a dword.
__device__ __forceinline__ float half_lo(u32 v) {
  return (float)__builtin_bit_cast(_Float16, (uint16_t)(v & 0xFFFFu));
}
__device__ __forceinline__ float half_hi(u32 v) {
  return (float)__builtin_bit_cast(_Float16, (uint16_t)(v >> 16));
}

// Asymmetric superblock record {binary16 base; 48-bit field of eight 6-bit
// sub-codes} held in two dwords r.x (bytes 0-3) and r.y (bytes 4-7).
// Returns base * sub_j, exact in binary32 (11 + 6 significant bits).
__device__ __forceinline__ float record_value(u32x2 r, int j) {
  const uint64_t all = ((uint64_t)r.y << 32) | r.x;
  const u32 sub = (u32)(all >> (16 + 6 * j)) & 0x3Fu;
  return half_lo(r.x) * (float)sub;
}

// Sum over the LPR consecutive lanes of a row group (LPR a power of two <=
// 64); every lane of the group receives the total.  Within a row of 16 lanes
// the exchanges are DPP moves (quad swaps, half-row and row mirrors); wider
// groups finish with cross-row shuffles.
template <int CTRL>
__device__ __forceinline__ float dpp_mov(float v) {
  return __builtin_bit_cast(
      float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, 0xF, 0xF, false));
}

template <int LPR>
__device__ __forceinline__ float group_sum(float v) {
  if constexpr (LPR >= 2) v += dpp_mov<0xB1>(v);   // quad_perm(1,0,3,2): lane ^ 1
  if constexpr (LPR >= 4) v += dpp_mov<0x4E>(v);   // quad_perm(2,3,0,1): lane ^ 2
  if constexpr (LPR >= 8) v += dpp_mov<0x141>(v);  // row_half_mirror: i <-> 7 - i
  if constexpr (LPR >= 16) v += dpp_mov<0x140>(v); // row_mirror: i <-> 15 - i
  if constexpr (LPR >= 32) v += __shfl_xor(v, 16, 64);
  if constexpr (LPR >= 64) v += __shfl_xor(v, 32, 64);
  return v;
}

}  // namespace rq
