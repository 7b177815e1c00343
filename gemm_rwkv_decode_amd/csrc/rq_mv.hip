// rq_mv.hip -- y = x W^T for decode-sized M (1..4) with the products on the
// matrix cores.
//
// At M = 1 the vector-unit kernel (rq_gemv.hip) spends about 2.5 VALU
// operations per code on MI355X: exact unpack (1.0), v_dot2 (0.5) and the
// per-thread overhead of a short lane slice.  Here the unpacked codes feed a
// v_mfma_f32_16x16x32_f16 (v_mfma_f32_16x16x16_f16 for 8-bit codes) instead:
// the matrix core does the dot products and the cross-lane sum, the VALU only
// unpacks (1.0 per code for 4-bit codes) and scales once per group.  The
// MFMA's 16 activation rows hold the M real rows; the rest are padding whose
// outputs are never stored.  Numerics are those of rq_gemm.hip: exact codes
// times binary16 x, binary32 sums per group, then acc += s * P (asymmetric:
// acc -= t * sum_k x).
//
// Layout of one MFMA: A = x tile [16 m][KS k], B = W^T tile [KS k][16 n],
// D = [16 m][16 n], lane l holding D[4*(l/16) + i][l%16].  Lane l supplies row
// l%16 of A and column l%16 of B; its lane group h = l/16 supplies one
// quarter of the K-step.  For 4-bit codes a lane takes, per group of G, the
// G/4 consecutive codes of its row in quarter h, which unpack4 delivers
// pairwise as (q0,q4) (q1,q5) ...; the matching x is stored in LDS already
// permuted the same way (pair_x4).  The codes are read in 64-byte spans of a
// row, one 16-byte piece per quarter, and exchanged across the quarters
// (span_fix) once they have arrived.
//
// Work split: a workgroup of 8 waves owns 16 rows; wave w owns the w-th
// eighth of K, in chunks of CG groups.  It first copies its x range into its
// own LDS region (coalesced loads, permuted once), then streams its codes
// with the next chunk's loads in flight while the current one is multiplied.
// The eight K-slices are added in wave order through LDS at the end.
#include "rq_common.h"
#include "rq_internal.h"

namespace rq {

constexpr int MV_WAVES = 8;
constexpr int MV_ROWS = 16;
constexpr int MV_LDS = 144 * 1024;  // x regions of the eight waves, at most

// Halves per LDS row of a wave's x region holding kr halves: 8 past a
// multiple of 64, so the rows of several activation rows start in different
// banks.
constexpr int mv_xstr(int kr) { return ((kr + 63) & ~63) + 8; }
constexpr int mv_lds_bytes(int kr, int me) { return MV_WAVES * me * mv_xstr(kr) * 2; }

template <int FMT>
struct MvMfma {
  static constexpr int KS = (FMT == FMT_S8) ? 16 : 32;  // k per MFMA
};

template <int FMT>
__device__ __forceinline__ f4 mv_mfma(const u32* a, const u32* b, f4 c) {
  if constexpr (FMT == FMT_S8) {
    const h4 av = __builtin_bit_cast(h4, u32x2{a[0], a[1]});
    const h4 bv = __builtin_bit_cast(h4, u32x2{b[0], b[1]});
    return __builtin_amdgcn_mfma_f32_16x16x16f16(av, bv, c, 0, 0, 0);
  } else {
    const h8 av = __builtin_bit_cast(h8, u32x4{a[0], a[1], a[2], a[3]});
    const h8 bv = __builtin_bit_cast(h8, u32x4{b[0], b[1], b[2], b[3]});
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(av, bv, c, 0, 0, 0);
  }
}

// Groups per chunk: a superblock for the asymmetric layout, else 8.
template <int FMT>
constexpr int mv_cg() {
  return FMT == FMT_A4 ? SUPERBLOCK / SB_GROUP : 8;
}

// One problem of a launch and the table of up to MV_BATCH problems.  The
// first workgroups sit in one array at the front, so a workgroup finds its
// problem from one scalar load and compares, then reads that entry.
struct MvEntry {
  const uint8_t* qw;
  const void* sc;
  const void* zr;
  const _Float16* x;
  float* y;
  int N;
};
template <int B>
struct MvBatch {
  int begin[B];  // first workgroup of each problem
  int count;
  MvEntry e[B];
};

// Per-lane registers of one chunk: codes of CG groups, their scale material.
template <int FMT, int G>
struct MvChunk {
  static constexpr int CG = mv_cg<FMT>();
  static constexpr int DPG = (FMT == FMT_S8) ? G / 16 : G / 32;  // dwords per lane per group
  static constexpr int GB = (FMT == FMT_S8) ? G : G / 2;          // code bytes per group, row
  static constexpr int SG = 64 / GB;                              // groups per 64-byte span
  static constexpr int NSP = CG / SG;                             // spans per chunk
  // codes as loaded: one 16-byte piece per span (span_fix puts them in MFMA
  // order once they have arrived)
  u32 code[CG * DPG];
  u32 sc[CG / 2];   // sym: the chunk's binary16 scales of this lane's row
  u32x2 srec, zrec; // asym: the superblock's records
};

template <int FMT, int G>
__device__ __forceinline__ void mv_load(MvChunk<FMT, G>& r, const uint8_t* __restrict__ qw,
                                        const void* __restrict__ scales,
                                        const void* __restrict__ zeros, u32 row, int K,
                                        int kb, int h) {
  using R = MvChunk<FMT, G>;
  const u32 row_bytes = (FMT == FMT_S8) ? (u32)K : (u32)K / 2;
  // 64-byte spans of the row, 16 bytes per lane quarter (span_piece)
  const uint8_t* p = qw + (row * row_bytes + (u32)((FMT == FMT_S8) ? kb : kb / 2) +
                           (u32)(span_piece<R::SG>(h) * 16));
  // scale material first: waiting for it does not wait for the codes
  if constexpr (FMT == FMT_A4) {
    const u32 rec = row * (u32)(K / SUPERBLOCK) + (u32)(kb / SUPERBLOCK);
    r.srec = reinterpret_cast<const u32x2*>(scales)[rec];
    r.zrec = reinterpret_cast<const u32x2*>(zeros)[rec];
  } else {
    // CG = 8 scales, 16-byte aligned (a chunk starts on a multiple of 8 groups)
    const u32x4 v = *reinterpret_cast<const u32x4*>(static_cast<const uint16_t*>(scales) +
                                                    (row * (u32)(K / G) + (u32)(kb / G)));
    r.sc[0] = v.x; r.sc[1] = v.y; r.sc[2] = v.z; r.sc[3] = v.w;
  }
#pragma unroll
  for (int sp = 0; sp < R::NSP; sp++) {
    const u32x4 v = load_stream16(p + sp * 64);
    r.code[4 * sp + 0] = v.x; r.code[4 * sp + 1] = v.y;
    r.code[4 * sp + 2] = v.z; r.code[4 * sp + 3] = v.w;
  }
}

// Multiply one chunk: x of the chunk at column kx of this wave's LDS rows.
template <int FMT, int G, int ME>
__device__ __forceinline__ void mv_chunk(MvChunk<FMT, G>& r, const _Float16* xw,
                                         int xstr, int kx, int mrow, int h, f4& acc) {
  using R = MvChunk<FMT, G>;
  constexpr int KS = MvMfma<FMT>::KS;
  constexpr int QPL = G / 4;  // k per lane group per group
#pragma unroll
  for (int sp = 0; sp < R::NSP; sp++) span_fix<R::SG>(&r.code[4 * sp]);
#pragma unroll
  for (int g = 0; g < R::CG; g++) {
    u32 a[R::DPG][4];
#pragma unroll
    for (int s = 0; s < R::DPG; s++) {
      const _Float16* src = xw + mrow * xstr + kx + g * G + h * QPL + s * (KS / 4);
      if constexpr (FMT == FMT_S8) {
        const u32x2 v = *reinterpret_cast<const u32x2*>(src);
        a[s][0] = v.x; a[s][1] = v.y;
      } else {
        const u32x4 v = *reinterpret_cast<const u32x4*>(src);
        a[s][0] = v.x; a[s][1] = v.y; a[s][2] = v.z; a[s][3] = v.w;
      }
    }
    f4 P = {0, 0, 0, 0};
#pragma unroll
    for (int s = 0; s < R::DPG; s++) {
      u32 b[4];
      const u32 d = r.code[g * R::DPG + s];
      if constexpr (FMT == FMT_S8) {
        h2 q[2];
        unpack8(d, q);
        b[0] = as_u32(q[0]); b[1] = as_u32(q[1]);
      } else {
        h2 q[4];
        unpack4<FMT == FMT_S4>(d, q);
        b[0] = as_u32(q[0]); b[1] = as_u32(q[1]);
        b[2] = as_u32(q[2]); b[3] = as_u32(q[3]);
      }
      P = mv_mfma<FMT>(a[s], b, P);
    }
    float sc, t = 0.0f;
    f4 xg = {0, 0, 0, 0};
    if constexpr (FMT == FMT_A4) {
      // group sums of x in the layout of P: one MFMA against codes all 1
      const u32 one2 = 0x3C003C00u;
      const u32 ones[4] = {one2, one2, one2, one2};
      xg = mv_mfma<FMT>(a[0], ones, xg);
      sc = record_value(r.srec, g);
      t = record_value(r.zrec, g);
    } else {
      const u32 pair = r.sc[g / 2];
      sc = (g & 1) ? half_hi(pair) : half_lo(pair);
    }
    // only the ME real activation rows (P[i] of lanes 0..15) are kept
#pragma unroll
    for (int i = 0; i < ME; i++) {
      float v = __builtin_fmaf(sc, P[i], acc[i]);
      if constexpr (FMT == FMT_A4) v = __builtin_fmaf(-t, xg[i], v);
      acc[i] = v;
    }
  }
}

template <int FMT, int G, int ME, int B>
__global__ void __launch_bounds__(64 * MV_WAVES)
k_mv(const MvBatch<B> bt, int M, int K, int xstr) {
  using R = MvChunk<FMT, G>;
  constexpr int CK = R::CG * G;  // k per chunk
  extern __shared__ __attribute__((aligned(16))) char lds[];  // MV_WAVES * ME * xstr halves
  __shared__ float red[MV_WAVES][ME][MV_ROWS];

  // this workgroup's problem (uniform scan of a small table)
  int pi = 0;
#pragma unroll
  for (int i = 1; i < B; i++)
    if (i < bt.count && (int)blockIdx.x >= bt.begin[i]) pi = i;
  const MvEntry& e = bt.e[pi];
  const int row0 = ((int)blockIdx.x - bt.begin[pi]) * MV_ROWS;
  // the entry's fields and the launch arguments in scalar registers at once
  // (one round trip after the table scan, not one per use)
  asm volatile("" ::"s"(e.qw), "s"(e.sc), "s"(e.zr), "s"(e.x), "s"(e.y), "s"(e.N), "s"(row0),
               "s"(M), "s"(K));

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // uniform: scalar branches
  const int h = lane >> 4;
  const int col = lane & 15;
  const u32 row = (u32)min(row0 + col, e.N - 1);
  // this wave's chunks [c0, c1) of K
  const int nch = K / CK;
  const int c0 = wave * nch / MV_WAVES, c1 = (wave + 1) * nch / MV_WAVES;
  const int kw0 = c0 * CK;
  const int kr = (c1 - c0) * CK;  // k of this wave
  _Float16* xw = reinterpret_cast<_Float16*>(lds) + wave * (xstr * ME);

  // Stage x[0..M)[kw0, kw0+kr) into this wave's LDS rows, 4-bit formats in
  // the order unpack4 delivers codes (rows >= M repeat row M-1).  The first
  // XB pieces of 8 halves per lane and row are loaded before the first
  // chunk's codes (loads complete in order, so x is waited for without
  // waiting for the codes); longer ranges load the rest afterwards.  Lanes
  // past the end repeat the last piece (same value to the same place).
  constexpr int XB = ME == 4 ? 2 : 4;
  const int pr = kr / 8;  // pieces per activation row
  u32x4 v[ME][XB];
  auto x_load = [&](int p0) {
#pragma unroll
    for (int m = 0; m < ME; m++) {
      const _Float16* xr = e.x + ((u32)(m < M ? m : M - 1) * (u32)K + (u32)kw0);
#pragma unroll
      for (int j = 0; j < XB; j++) {
        const int p = min(p0 + j * 64 + lane, pr - 1);
        v[m][j] = *reinterpret_cast<const u32x4*>(xr + p * 8);
      }
    }
  };
  auto x_store = [&](int p0) {
#pragma unroll
    for (int m = 0; m < ME; m++) {
#pragma unroll
      for (int j = 0; j < XB; j++) {
        const int p = min(p0 + j * 64 + lane, pr - 1);
        u32x4 w = v[m][j];
        if constexpr (FMT != FMT_S8) {
          h2 q[4];
          pair_x4(w.x, w.y, w.z, w.w, q);
          w = u32x4{as_u32(q[0]), as_u32(q[1]), as_u32(q[2]), as_u32(q[3])};
        }
        *reinterpret_cast<u32x4*>(xw + m * xstr + p * 8) = w;
      }
    }
  };
  R r0, r1;
  x_load(0);
  __builtin_amdgcn_sched_barrier(0);
  mv_load<FMT, G>(r0, e.qw, e.sc, e.zr, row, K, kw0, h);
  __builtin_amdgcn_sched_barrier(0);
  x_store(0);
  for (int p0 = 64 * XB; p0 < pr; p0 += 64 * XB) {
    x_load(p0);
    x_store(p0);
  }
  // this wave's LDS writes land before its lanes read each other's pieces
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  // padding rows of the MFMA read the last real row
  const int mrow = col < ME ? (col < M ? col : M - 1) : M - 1;

  // Chunks c0 .. c1-1 (at least one; the host checks K / CK >= 8), the next
  // one's loads in flight while the current one is multiplied.  Each path
  // issues its loads unconditionally, so the waits count exactly.
  f4 acc = {0, 0, 0, 0};
  for (int c = c0;; c += 2) {
    if (c + 1 >= c1) {
      mv_chunk<FMT, G, ME>(r0, xw, xstr, (c - c0) * CK, mrow, h, acc);
      break;
    }
    mv_load<FMT, G>(r1, e.qw, e.sc, e.zr, row, K, (c + 1) * CK, h);
    mv_chunk<FMT, G, ME>(r0, xw, xstr, (c - c0) * CK, mrow, h, acc);
    if (c + 2 >= c1) {
      mv_chunk<FMT, G, ME>(r1, xw, xstr, (c + 1 - c0) * CK, mrow, h, acc);
      break;
    }
    mv_load<FMT, G>(r0, e.qw, e.sc, e.zr, row, K, (c + 2) * CK, h);
    mv_chunk<FMT, G, ME>(r1, xw, xstr, (c + 1 - c0) * CK, mrow, h, acc);
  }

  // add the eight K-slices in wave order; lanes 0..15 hold rows m < ME
  if (h == 0) {
#pragma unroll
    for (int i = 0; i < ME; i++) red[wave][i][col] = acc[i];
  }
  __syncthreads();
  if (wave == 0 && h == 0) {
    const int n = row0 + col;
#pragma unroll
    for (int i = 0; i < ME; i++) {
      float v = red[0][i][col];
#pragma unroll
      for (int w = 1; w < MV_WAVES; w++) v += red[w][i][col];
      if (i < M && n < e.N) e.y[(size_t)i * e.N + n] = v;
    }
  }
}

// ---------------------------------------------------------------------------
// host side
// ---------------------------------------------------------------------------
static int mv_ck(int fmt, int group) {
  return (fmt == FMT_A4 ? SUPERBLOCK / SB_GROUP : 8) * group;
}

bool mv_supports(int fmt, int M, int K, int group) {
  if (M < 1 || M > 4) return false;
  // FP8 and 5-/6-bit codes run on the vector-unit kernel
  if (fmt == FMT_F8 || fmt == FMT_A5 || fmt == FMT_A6) return false;
  const int ck = mv_ck(fmt, group);
  if (K % ck != 0 || K / ck < MV_WAVES) return false;
  const int me = M <= 1 ? 1 : (M <= 2 ? 2 : 4);
  // the x ranges of the eight waves must fit LDS
  const int nch = K / ck;
  const int kr = ((nch + MV_WAVES - 1) / MV_WAVES) * ck;
  return mv_lds_bytes(kr, me) <= MV_LDS;
}

template <int FMT, int G, int ME>
static hipError_t launch_mv_t(const Problem* const* p, int count, int M, hipStream_t s) {
  constexpr int B = MV_BATCH;
  MvBatch<B> bt{};
  int blocks = 0;
  for (int i = 0; i < count; i++) {
    bt.e[i] = MvEntry{static_cast<const uint8_t*>(p[i]->qweight), p[i]->scales, p[i]->zeros,
                      static_cast<const _Float16*>(p[i]->x), p[i]->y, p[i]->N};
    bt.begin[i] = blocks;
    blocks += (p[i]->N + MV_ROWS - 1) / MV_ROWS;
  }
  bt.count = count;
  const int K = p[0]->K;
  const int ck = MvChunk<FMT, G>::CG * G;
  const int kr = ((K / ck + MV_WAVES - 1) / MV_WAVES) * ck;
  const int lds = mv_lds_bytes(kr, ME);
  if (lds > MV_LDS) return hipErrorInvalidValue;
  static bool raised = false;  // allow the full LDS once per instantiation
  if (!raised) {
    const hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(k_mv<FMT, G, ME, B>),
                                             hipFuncAttributeMaxDynamicSharedMemorySize, MV_LDS);
    if (e != hipSuccess) return e;
    raised = true;
  }
  hipLaunchKernelGGL((k_mv<FMT, G, ME, B>), dim3(blocks), dim3(64 * MV_WAVES), lds, s, bt, M, K,
                     mv_xstr(kr));
  return hipGetLastError();
}

template <int FMT, int G>
static hipError_t launch_mv_me(const Problem* const* p, int count, int M, hipStream_t s) {
  if (M <= 1) return launch_mv_t<FMT, G, 1>(p, count, M, s);
  if (M <= 2) return launch_mv_t<FMT, G, 2>(p, count, M, s);
  return launch_mv_t<FMT, G, 4>(p, count, M, s);
}

hipError_t launch_mv_many(const Problem* const* p, int count, hipStream_t s) {
  for (int base = 0; base < count; base += MV_BATCH) {
    const int n = count - base < MV_BATCH ? count - base : MV_BATCH;
    const Problem* const* q = p + base;
    const int fmt = q[0]->fmt, g = q[0]->group, M = q[0]->M;
    hipError_t e;
    if (fmt == FMT_S4) {
      e = g == 32 ? launch_mv_me<FMT_S4, 32>(q, n, M, s)
                  : (g == 64 ? launch_mv_me<FMT_S4, 64>(q, n, M, s)
                             : launch_mv_me<FMT_S4, 128>(q, n, M, s));
    } else if (fmt == FMT_S8) {
      e = g == 16 ? launch_mv_me<FMT_S8, 16>(q, n, M, s)
                  : (g == 32 ? launch_mv_me<FMT_S8, 32>(q, n, M, s)
                             : launch_mv_me<FMT_S8, 64>(q, n, M, s));
    } else {
      e = launch_mv_me<FMT_A4, 32>(q, n, M, s);
    }
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace rq
