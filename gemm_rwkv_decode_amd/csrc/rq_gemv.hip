// rq_gemv.hip -- y = x W^T on the vector ALUs, tuned for the decode shape
// (M = 1) and small M (<= 8 rows per launch).
//
// Work split (one workgroup = SK waves = one block of rows):
//   * every wave owns one K-slice of the block's rows (split-K inside the
//     workgroup); the K-slices are combined through LDS at the end, in wave
//     order, so the result does not depend on timing;
//   * inside a wave, LPR consecutive lanes share a row and 64/LPR rows are in
//     flight at once; a lane owns CPL 16-byte chunks of its row's slice, chosen
//     so that the LPR lanes of a row read one contiguous run of LPR*16 bytes;
//   * the activations a lane needs (its chunks of x for every row of M) are
//     loaded once into registers and reused for every weight row;
//   * the block's rows are visited in `npass` passes; the code loads of pass
//     p+1 are issued before pass p is computed (two passes in flight).
//
// Arithmetic per 16-byte chunk: codes become exact binary16 integers
// (rq_common.h), v_dot2_f32_f16 multiplies them by binary16 x and accumulates
// in binary32 (products exact), and the chunk sum is scaled once in binary32:
// acc += s * sum_k q x, and for the asymmetric layout also acc -= t * sum_k x
// with sum_k x precomputed per chunk.  Every chunk lies inside one group.
#include "rq_common.h"
#include "rq_internal.h"

#include <stdlib.h>

namespace rq {

template <int FMT>
struct RowBytes {
  static __device__ __forceinline__ size_t of(int K) {
    return (FMT == FMT_S8) ? (size_t)K : (size_t)K / 2;
  }
};

// Load the x values of one chunk (CPC halves starting at k0) of one row of x
// into dot2 pairs in the order the unpack of that format produces codes.
template <int FMT>
__device__ __forceinline__ void load_x_chunk(const _Float16* __restrict__ xrow, int k0,
                                             h2* dst, float* xsum) {
  constexpr int CPC = Chunk<FMT>::codes;
  const u32x4* src = reinterpret_cast<const u32x4*>(xrow + k0);
  float s = 0.0f;
#pragma unroll
  for (int v = 0; v < CPC / 8; v++) {
    const u32x4 w = src[v];
    if (FMT == FMT_S8) {
      dst[4 * v + 0] = as_h2(w.x);
      dst[4 * v + 1] = as_h2(w.y);
      dst[4 * v + 2] = as_h2(w.z);
      dst[4 * v + 3] = as_h2(w.w);
    } else {
      pair_x4(w.x, w.y, w.z, w.w, &dst[4 * v]);
    }
    if (FMT == FMT_A4) {
      s += half_lo(w.x) + half_hi(w.x) + half_lo(w.y) + half_hi(w.y) +
           half_lo(w.z) + half_hi(w.z) + half_lo(w.w) + half_hi(w.w);
    }
  }
  *xsum = s;
}

// sum_k q[k] * x[k] over one 16-byte chunk of codes, binary32.
template <int FMT>
__device__ __forceinline__ float chunk_dot(const u32x4 code, const h2* xp) {
  float a = 0.0f;
  const u32 d[4] = {code.x, code.y, code.z, code.w};
  if (FMT == FMT_S8) {
#pragma unroll
    for (int i = 0; i < 4; i++) {
      h2 q[2];
      unpack8(d[i], q);
      a = __builtin_amdgcn_fdot2(q[0], xp[2 * i + 0], a, false);
      a = __builtin_amdgcn_fdot2(q[1], xp[2 * i + 1], a, false);
    }
  } else {
#pragma unroll
    for (int i = 0; i < 4; i++) {
      h2 q[4];
      unpack4<FMT == FMT_S4>(d[i], q);
#pragma unroll
      for (int j = 0; j < 4; j++) a = __builtin_amdgcn_fdot2(q[j], xp[4 * i + j], a, false);
    }
  }
  return a;
}

template <int FMT, int CPL>
struct PassData {
  u32x4 code[CPL];
  float s[CPL];   // scale (sym) or d*sc_j (asym)
  float t[CPL];   // m*mn_j (asym)
};

template <int FMT, int CPL>
__device__ __forceinline__ void load_pass(PassData<FMT, CPL>& pd,
                                          const uint8_t* __restrict__ qw,
                                          const void* __restrict__ scales,
                                          const void* __restrict__ zeros, int n, int K,
                                          int group, const int* kc) {
  constexpr int CPC = Chunk<FMT>::codes;
  const uint8_t* row = qw + (size_t)n * RowBytes<FMT>::of(K);
#pragma unroll
  for (int c = 0; c < CPL; c++) pd.code[c] = load_stream16(row + (size_t)kc[c] * 16);
#pragma unroll
  for (int c = 0; c < CPL; c++) {
    const int k0 = kc[c] * CPC;
    if (FMT == FMT_A4) {
      const size_t rec = (size_t)n * (K / SUPERBLOCK) + k0 / SUPERBLOCK;
      const int j = (k0 % SUPERBLOCK) / SB_GROUP;
      pd.s[c] = record_value(reinterpret_cast<const u32x2*>(scales)[rec], j);
      pd.t[c] = record_value(reinterpret_cast<const u32x2*>(zeros)[rec], j);
    } else {
      const uint16_t sb =
          static_cast<const uint16_t*>(scales)[(size_t)n * (K / group) + k0 / group];
      pd.s[c] = (float)__builtin_bit_cast(_Float16, sb);
      pd.t[c] = 0.0f;
    }
  }
}

// Largest workgroup: 16 waves for one activation row, 8 waves above (the
// activation registers grow with M and a smaller workgroup leaves each wave
// more of the register file).
template <int MT>
struct GemvMax {
  static constexpr int threads = (MT >= 2) ? 512 : 1024;
};

template <int FMT, int LPR, int CPL, int MT>
__device__ __forceinline__ void gemv_pass(const PassData<FMT, CPL>& pd,
                                          const h2 (&xr)[MT][CPL][Chunk<FMT>::codes / 2],
                                          const float (&xs)[MT][CPL], float* __restrict__ y,
                                          float* part, int p, int row0, int RB, int w,
                                          int SK, int rs, int li, int Mrows, int N) {
  constexpr int RPW = 64 / LPR;
  float acc[MT];
#pragma unroll
  for (int m = 0; m < MT; m++) acc[m] = 0.0f;
#pragma unroll
  for (int c = 0; c < CPL; c++) {
#pragma unroll
    for (int m = 0; m < MT; m++) {
      const float d = chunk_dot<FMT>(pd.code[c], xr[m][c]);
      acc[m] = __builtin_fmaf(d, pd.s[c], acc[m]);
      if (FMT == FMT_A4) acc[m] = __builtin_fmaf(-pd.t[c], xs[m][c], acc[m]);
    }
  }
  const int n = row0 + p * RPW + rs;
#pragma unroll
  for (int m = 0; m < MT; m++) {
    const float v = group_sum<LPR>(acc[m]);
    if (li == 0) {
      if (SK == 1) {
        if (m < Mrows && n < N) y[(size_t)m * N + n] = v;
      } else {
        part[((size_t)w * RB + p * RPW + rs) * MT + m] = v;
      }
    }
  }
}

template <int FMT, int LPR, int CPL, int MT>
__global__ void __launch_bounds__(GemvMax<MT>::threads)
k_gemv(const uint8_t* __restrict__ qw, const void* __restrict__ scales,
       const void* __restrict__ zeros, const _Float16* __restrict__ x,
       float* __restrict__ y, int Mrows, int N, int K, int group, int npass) {
  constexpr int RPW = 64 / LPR;
  constexpr int CPC = Chunk<FMT>::codes;
  constexpr int XP = CPC / 2;
  extern __shared__ float part[];  // [SK][RB][MT]

  const int lane = threadIdx.x & 63;
  const int w = threadIdx.x >> 6;
  const int SK = blockDim.x >> 6;
  const int rs = lane / LPR;
  const int li = lane % LPR;
  const int RB = RPW * npass;
  const int row0 = blockIdx.x * RB;

  int kc[CPL];
#pragma unroll
  for (int c = 0; c < CPL; c++) kc[c] = w * (LPR * CPL) + c * LPR + li;

  h2 xr[MT][CPL][XP];
  float xs[MT][CPL];
#pragma unroll
  for (int m = 0; m < MT; m++) {
#pragma unroll
    for (int c = 0; c < CPL; c++) {
      if (m < Mrows) {
        load_x_chunk<FMT>(x + (size_t)m * K, kc[c] * CPC, xr[m][c], &xs[m][c]);
      } else {
#pragma unroll
        for (int i = 0; i < XP; i++) xr[m][c][i] = h2{0, 0};
        xs[m][c] = 0.0f;
      }
    }
  }

  // two passes in flight: b0 holds even passes, b1 odd ones
  PassData<FMT, CPL> b0, b1;
  load_pass<FMT, CPL>(b0, qw, scales, zeros, min(row0 + rs, N - 1), K, group, kc);
  for (int p = 0; p < npass; p += 2) {
    if (p + 1 < npass)
      load_pass<FMT, CPL>(b1, qw, scales, zeros, min(row0 + (p + 1) * RPW + rs, N - 1), K,
                          group, kc);
    gemv_pass<FMT, LPR, CPL, MT>(b0, xr, xs, y, part, p, row0, RB, w, SK, rs, li, Mrows, N);
    if (p + 1 < npass) {
      if (p + 2 < npass)
        load_pass<FMT, CPL>(b0, qw, scales, zeros, min(row0 + (p + 2) * RPW + rs, N - 1),
                            K, group, kc);
      gemv_pass<FMT, LPR, CPL, MT>(b1, xr, xs, y, part, p + 1, row0, RB, w, SK, rs, li,
                                   Mrows, N);
    }
  }

  if (SK > 1) {
    __syncthreads();
    for (int idx = threadIdx.x; idx < RB * Mrows; idx += blockDim.x) {
      const int r = idx / Mrows, m = idx % Mrows;
      float v = 0.0f;
      for (int ww = 0; ww < SK; ww++) v += part[((size_t)ww * RB + r) * MT + m];
      const int n = row0 + r;
      if (n < N) y[(size_t)m * N + n] = v;
    }
  }
}

// Any valid shape: one row per 16 lanes, lanes stride over the row's chunks,
// activations read from memory per chunk (slower; used when the chunk count of
// a row has no factorization the tuned kernel supports).
template <int FMT, int MT>
__global__ void __launch_bounds__(256)
k_gemv_generic(const uint8_t* __restrict__ qw, const void* __restrict__ scales,
               const void* __restrict__ zeros, const _Float16* __restrict__ x,
               float* __restrict__ y, int Mrows, int N, int K, int group) {
  constexpr int LPR = 16;
  constexpr int CPC = Chunk<FMT>::codes;
  constexpr int XP = CPC / 2;
  const int lane = threadIdx.x & 63;
  const int n = (blockIdx.x * blockDim.x + threadIdx.x) / LPR;
  const int li = lane % LPR;
  const int nn = min(n, N - 1);
  const int chunks = (int)(RowBytes<FMT>::of(K) / 16);
  float acc[MT];
#pragma unroll
  for (int m = 0; m < MT; m++) acc[m] = 0.0f;
  for (int c = li; c < chunks; c += LPR) {
    int kc[1] = {c};
    PassData<FMT, 1> pd;
    load_pass<FMT, 1>(pd, qw, scales, zeros, nn, K, group, kc);
#pragma unroll
    for (int m = 0; m < MT; m++) {
      if (m < Mrows) {
        h2 xp[XP];
        float xs;
        load_x_chunk<FMT>(x + (size_t)m * K, c * CPC, xp, &xs);
        const float d = chunk_dot<FMT>(pd.code[0], xp);
        acc[m] = __builtin_fmaf(d, pd.s[0], acc[m]);
        if (FMT == FMT_A4) acc[m] = __builtin_fmaf(-pd.t[0], xs, acc[m]);
      }
    }
  }
#pragma unroll
  for (int m = 0; m < MT; m++) {
    const float v = group_sum<LPR>(acc[m]);
    if (li == 0 && m < Mrows && n < N) y[(size_t)m * N + n] = v;
  }
}

// ---------------------------------------------------------------------------
// host side
// ---------------------------------------------------------------------------
static int env_int(const char* name, int dflt) {
  const char* v = getenv(name);
  return v ? atoi(v) : dflt;
}

GemvCfg choose_gemv(int fmt, int M, int N, int K) {
  GemvCfg c{};
  // activation rows per launch: the smallest of 1, 2, 4, 8 covering M (or 8)
  c.mt = M <= 1 ? 1 : (M == 2 ? 2 : (M <= 4 ? 4 : 8));
  const int chunks = (fmt == FMT_S8) ? K / 16 : K / 32;
  // Lane splits tried in order; the first whose wave count fits is taken.
  static const int pref[][2] = {{16, 1}, {32, 1}, {64, 1}, {8, 1},
                                {16, 2}, {32, 2}, {64, 2}, {8, 2}};
  c.lpr = 0;
  const int max_waves = (c.mt >= 2) ? 8 : 16;  // GemvMax
  for (auto& pr : pref) {
    const int lpr = pr[0], cpl = pr[1];
    if (c.mt >= 8 && cpl > 1) continue;  // keep x registers bounded
    if (chunks % (lpr * cpl)) continue;
    const int sk = chunks / (lpr * cpl);
    if (sk < 1 || sk > max_waves) continue;
    c.lpr = lpr;
    c.cpl = cpl;
    break;
  }
  const int forced = env_int("RQ_GEMV_LPR", 0);
  if (forced < 0) c.lpr = 0;  // force the generic kernel (testing)
  if (c.lpr == 0) {
    c.cpl = 1;
    c.npass = 1;
    return c;
  }
  // Rows per workgroup: enough workgroups to fill the chip twice over.
  const int rpw = 64 / c.lpr;
  int npass = N / (rpw * 512);
  npass = npass < 1 ? 1 : (npass > 8 ? 8 : npass);
  c.npass = env_int("RQ_GEMV_NPASS", npass);
  return c;
}

template <int FMT, int LPR, int CPL, int MT>
static void launch_t(const Problem& p, const GemvCfg& c, const _Float16* x, float* y,
                     int mrows, hipStream_t s) {
  const int chunks = (FMT == FMT_S8) ? p.K / 16 : p.K / 32;
  const int sk = chunks / (LPR * CPL);
  const int rb = (64 / LPR) * c.npass;
  const int blocks = (p.N + rb - 1) / rb;
  const size_t lds = (sk > 1) ? (size_t)sk * rb * MT * sizeof(float) : 0;
  hipLaunchKernelGGL((k_gemv<FMT, LPR, CPL, MT>), dim3(blocks), dim3(64 * sk), lds, s,
                     static_cast<const uint8_t*>(p.qweight), p.scales, p.zeros, x, y,
                     mrows, p.N, p.K, p.group, c.npass);
}

template <int FMT, int MT>
static void launch_mt(const Problem& p, const GemvCfg& c, const _Float16* x, float* y,
                      int mrows, hipStream_t s) {
  if (c.lpr == 0) {
    const int blocks = (p.N * 16 + 255) / 256;
    hipLaunchKernelGGL((k_gemv_generic<FMT, MT>), dim3(blocks), dim3(256), 0, s,
                       static_cast<const uint8_t*>(p.qweight), p.scales, p.zeros, x, y,
                       mrows, p.N, p.K, p.group);
    return;
  }
#define RQ_L(L, C) \
  if (c.lpr == L && c.cpl == C) return launch_t<FMT, L, C, MT>(p, c, x, y, mrows, s)
  RQ_L(16, 1); RQ_L(32, 1); RQ_L(64, 1); RQ_L(8, 1);
  if constexpr (MT < 8) { RQ_L(16, 2); RQ_L(32, 2); RQ_L(64, 2); RQ_L(8, 2); }
#undef RQ_L
}

template <int FMT>
static void launch_fmt(const Problem& p, const GemvCfg& c, const _Float16* x, float* y,
                       int mrows, hipStream_t s) {
  switch (c.mt) {
    case 1: return launch_mt<FMT, 1>(p, c, x, y, mrows, s);
    case 2: return launch_mt<FMT, 2>(p, c, x, y, mrows, s);
    case 4: return launch_mt<FMT, 4>(p, c, x, y, mrows, s);
    default: return launch_mt<FMT, 8>(p, c, x, y, mrows, s);
  }
}

hipError_t launch_gemv(const Problem& p, const GemvCfg& c, hipStream_t s) {
  const _Float16* x = static_cast<const _Float16*>(p.x);
  for (int m0 = 0; m0 < p.M; m0 += c.mt) {
    const int mrows = (p.M - m0 < c.mt) ? p.M - m0 : c.mt;
    const _Float16* xm = x + (size_t)m0 * p.K;
    float* ym = p.y + (size_t)m0 * p.N;
    if (p.fmt == FMT_S4) launch_fmt<FMT_S4>(p, c, xm, ym, mrows, s);
    else if (p.fmt == FMT_S8) launch_fmt<FMT_S8>(p, c, xm, ym, mrows, s);
    else launch_fmt<FMT_A4>(p, c, xm, ym, mrows, s);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace rq
