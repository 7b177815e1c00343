// rq_dequant.hip -- unpack or dequantize packed weights to [N][K].
//
// Bound by the output write (4 bytes per weight for binary32 against 0.53 to
// 1.125 bytes read), so each thread handles one octet of 8 consecutive codes
// and writes 32 contiguous bytes; consecutive threads handle consecutive
// octets, so the two store instructions of a wave fill a contiguous 2 KiB.
//
// Arithmetic: symmetric w = s * q is exact in binary32 (at most 11 + 8
// significant bits).  Asymmetric s_j = d * sc_j and t_j = m * mn_j are exact
// (at most 17 bits) and w = fma(s_j, q, -t_j) rounds the exact s_j*q - t_j
// once, to nearest even -- the correctly rounded value of the formula.  FP8:
// the code converts exactly to binary32 and w = code * scale rounds once.
#include "rq_common.h"
#include "rq_internal.h"

namespace rq {

template <int FMT, bool CODES>
__global__ void __launch_bounds__(256)
k_dequant(const uint8_t* __restrict__ qw, const void* __restrict__ scales,
          const void* __restrict__ zeros, void* __restrict__ out, int N, int K,
          int group, long long octets) {
  const int oct_per_row = K / 8;
  for (long long o = (long long)blockIdx.x * blockDim.x + threadIdx.x; o < octets;
       o += (long long)gridDim.x * blockDim.x) {
    const int n = (int)(o / oct_per_row);
    const int k0 = (int)(o % oct_per_row) * 8;
    if constexpr (FMT == FMT_F8) {
      const u32x2 d = *reinterpret_cast<const u32x2*>(qw + (size_t)n * K + k0);
      const float s = *static_cast<const float*>(scales);
      typedef float f2 __attribute__((ext_vector_type(2)));
      const f2 a = __builtin_amdgcn_cvt_pk_f32_fp8(d.x, false);
      const f2 b = __builtin_amdgcn_cvt_pk_f32_fp8(d.x, true);
      const f2 c = __builtin_amdgcn_cvt_pk_f32_fp8(d.y, false);
      const f2 e = __builtin_amdgcn_cvt_pk_f32_fp8(d.y, true);
      f4* dst = reinterpret_cast<f4*>(static_cast<float*>(out) + (size_t)n * K + k0);
      dst[0] = f4{a.x * s, a.y * s, b.x * s, b.y * s};
      dst[1] = f4{c.x * s, c.y * s, e.x * s, e.y * s};
      continue;
    }
    int q[8];
    if (FMT == FMT_S8) {
      const u32x2 d = *reinterpret_cast<const u32x2*>(qw + (size_t)n * K + k0);
#pragma unroll
      for (int i = 0; i < 4; i++) {
        q[i] = (int)(int8_t)((d.x >> (8 * i)) & 0xFF);
        q[4 + i] = (int)(int8_t)((d.y >> (8 * i)) & 0xFF);
      }
    } else {
      const u32 d = *reinterpret_cast<const u32*>(qw + (size_t)n * (K / 2) + k0 / 2);
#pragma unroll
      for (int i = 0; i < 8; i++) {
        const int nib = (int)((d >> (4 * i)) & 0xF);
        q[i] = (FMT == FMT_S4) ? ((nib ^ 8) - 8) : nib;
      }
      if constexpr (hi_bits(FMT) > 0) {
        // this octet is nibble dword i of its 32-code chunk; the chunk's high
        // bits are 1 (5-bit) or 2 (6-bit) dwords of the plane after the nibbles
        constexpr int HB = hi_bits(FMT);
        const int ci = (k0 % 32) / 8;
        const u32* hp = reinterpret_cast<const u32*>(
            qw + (size_t)N * (K / 2) + (size_t)n * (K / 8 * HB) + (size_t)(k0 / 32) * 4 * HB);
        const u32 w = hp[HB == 1 ? 0 : ci / 2];
#pragma unroll
        for (int j = 0; j < 8; j++) {
          const int g = (j % 4) / 2;
          const int base = (j >= 4 ? 16 : 0) + (j % 2 == 0 ? 4 : 8);
          int pos;
          if (HB == 1) pos = base + (g == 0 ? ci - 4 : ci + 4);
          else pos = base + ((ci % 2 == 0) ? (g == 0 ? -4 : -2) : (g == 0 ? 4 : 6));
          q[j] |= (int)((w >> pos) & (HB == 1 ? 1u : 3u)) << 4;
        }
      }
    }
    if (CODES) {
      u32x2 v;
      v.x = (u32)(q[0] & 0xFF) | ((u32)(q[1] & 0xFF) << 8) | ((u32)(q[2] & 0xFF) << 16) |
            ((u32)(q[3] & 0xFF) << 24);
      v.y = (u32)(q[4] & 0xFF) | ((u32)(q[5] & 0xFF) << 8) | ((u32)(q[6] & 0xFF) << 16) |
            ((u32)(q[7] & 0xFF) << 24);
      *reinterpret_cast<u32x2*>(static_cast<int8_t*>(out) + (size_t)n * K + k0) = v;
      continue;
    }
    float w[8];
    if (is_asym(FMT)) {
      const size_t rec = (size_t)n * (K / SUPERBLOCK) + k0 / SUPERBLOCK;
      const int j = (k0 % SUPERBLOCK) / SB_GROUP;
      const u32x2 sr = reinterpret_cast<const u32x2*>(scales)[rec];
      const u32x2 zr = reinterpret_cast<const u32x2*>(zeros)[rec];
      const float s = record_value(sr, j);
      const float t = record_value(zr, j);
#pragma unroll
      for (int i = 0; i < 8; i++) w[i] = __builtin_fmaf(s, (float)q[i], -t);
    } else {
      const uint16_t sb =
          static_cast<const uint16_t*>(scales)[(size_t)n * (K / group) + k0 / group];
      const float s = (float)__builtin_bit_cast(_Float16, sb);
#pragma unroll
      for (int i = 0; i < 8; i++) w[i] = s * (float)q[i];
    }
    f4* dst = reinterpret_cast<f4*>(static_cast<float*>(out) + (size_t)n * K + k0);
    dst[0] = f4{w[0], w[1], w[2], w[3]};
    dst[1] = f4{w[4], w[5], w[6], w[7]};
  }
}

hipError_t launch_dequant(const void* qweight, const void* scales, const void* zeros,
                          void* out, int N, int K, int group, int fmt, int out_kind,
                          hipStream_t s) {
  const long long octets = (long long)N * K / 8;
  const int threads = 256;
  long long blocks = (octets + threads - 1) / threads;
  if (blocks > 256 * 16) blocks = 256 * 16;
  const uint8_t* q = static_cast<const uint8_t*>(qweight);
  const bool codes = (out_kind == 1);
#define RQ_DQ(F, C)                                                                  \
  hipLaunchKernelGGL((k_dequant<F, C>), dim3((unsigned)blocks), dim3(threads), 0, s, \
                     q, scales, zeros, out, N, K, group, octets)
  if (fmt == FMT_S4) {
    if (codes) RQ_DQ(FMT_S4, true); else RQ_DQ(FMT_S4, false);
  } else if (fmt == FMT_S8) {
    if (codes) RQ_DQ(FMT_S8, true); else RQ_DQ(FMT_S8, false);
  } else if (fmt == FMT_F8) {
    RQ_DQ(FMT_F8, false);  // codes output is rejected by the caller
  } else if (fmt == FMT_A5) {
    if (codes) RQ_DQ(FMT_A5, true); else RQ_DQ(FMT_A5, false);
  } else if (fmt == FMT_A6) {
    if (codes) RQ_DQ(FMT_A6, true); else RQ_DQ(FMT_A6, false);
  } else {
    if (codes) RQ_DQ(FMT_A4, true); else RQ_DQ(FMT_A4, false);
  }
#undef RQ_DQ
  return hipGetLastError();
}

}  // namespace rq
