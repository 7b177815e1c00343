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
//   * a lane visits NP rows of the block and issues the code loads of all of
//     them (NP*CPL 16-byte loads) before it waits for the first: the loads of
//     a small matrix are all in flight at once.
//
// Arithmetic per 16-byte chunk: codes become exact binary16 integers
// (rq_common.h), v_dot2_f32_f16 multiplies them by binary16 x and accumulates
// in binary32 (products exact), and the chunk sum is scaled once in binary32:
// acc += s * sum_k q x, and for the asymmetric layout also acc -= t * sum_k x
// with sum_k x precomputed per chunk.  Every chunk lies inside one group.
#include "rq_common.h"
#include "rq_internal.h"


namespace rq {

// Sums of V values per lane (V a power of two, V <= LPR) over the LPR
// consecutive lanes of a row group, the values halved at the first levels:
// each level pairs a lane with one whose level bit differs, the lane keeps
// one half of its values (the upper half where its bit is set) and adds the
// partner's copy of that half, so a level costs one exchange per kept value
// instead of one per value.  Levels run from the widest distance down:
// 32 and 16 by v_permlane32/16_swap (which also select the half, no
// per-lane choice), 8 by row_mirror (lane ^ 15), 4 by row_half_mirror
// (lane ^ 7), 2 and 1 by quad permutes; each pairs lanes that agree on the
// bits already decided, and together they cover the whole group.  On return
// v[0] holds the group total of value li >> (log2 LPR - log2 V) (li: lane
// index in the group); the other entries are spent.
template <int D>
__device__ __forceinline__ float level_partner(float v) {
  if constexpr (D == 8) return dpp_mov<0x140>(v);       // row_mirror
  else if constexpr (D == 4) return dpp_mov<0x141>(v);  // row_half_mirror
  else if constexpr (D == 2) return dpp_mov<0x4E>(v);   // quad_perm(2,3,0,1)
  else return dpp_mov<0xB1>(v);                         // quad_perm(1,0,3,2)
}

template <int LPR, int V>
__device__ __forceinline__ void group_sum_multi(float* v, int li) {
  static_assert(V >= 1 && V <= LPR && (V & (V - 1)) == 0 && (LPR & (LPR - 1)) == 0, "V, LPR");
  constexpr int LEVELS = __builtin_ctz(LPR);
  int w = V;  // live values
#pragma unroll
  for (int lv = 0; lv < LEVELS; lv++) {
    const int d = LPR >> (lv + 1);
    if (w > 1) {
      const int half = w / 2;
#pragma unroll
      for (int j = 0; j < half; j++) {
        if (d >= 16) {
          // rows (16 lanes) pair up at distance d; the swap leaves the kept
          // half in one register and the partner's copy in the other
          u32 a = __builtin_bit_cast(u32, v[j]), b = __builtin_bit_cast(u32, v[j + half]);
          if (d == 32) lane_swap32(a, b);
          else lane_swap16(a, b);
          v[j] = __builtin_bit_cast(float, a) + __builtin_bit_cast(float, b);
        } else {
          const bool hi = (li & d) != 0;
          const float keep = hi ? v[j + half] : v[j];
          const float send = hi ? v[j] : v[j + half];
          if (d == 8) v[j] = keep + level_partner<8>(send);
          else if (d == 4) v[j] = keep + level_partner<4>(send);
          else if (d == 2) v[j] = keep + level_partner<2>(send);
          else v[j] = keep + level_partner<1>(send);
        }
      }
      w = half;
    } else {
      if (d >= 16) {
        u32 a = __builtin_bit_cast(u32, v[0]), b = a;
        if (d == 32) lane_swap32(a, b);
        else lane_swap16(a, b);
        v[0] = __builtin_bit_cast(float, a) + __builtin_bit_cast(float, b);
      } else if (d == 8) {
        v[0] += level_partner<8>(v[0]);
      } else if (d == 4) {
        v[0] += level_partner<4>(v[0]);
      } else if (d == 2) {
        v[0] += level_partner<2>(v[0]);
      } else {
        v[0] += level_partner<1>(v[0]);
      }
    }
  }
}

template <int FMT>
struct RowBytes {
  static __device__ __forceinline__ size_t of(int K) {
    return (FMT == FMT_S8 || FMT == FMT_F8) ? (size_t)K : (size_t)K / 2;
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
    if (FMT == FMT_S8 || FMT == FMT_F8) {
      dst[4 * v + 0] = as_h2(w.x);
      dst[4 * v + 1] = as_h2(w.y);
      dst[4 * v + 2] = as_h2(w.z);
      dst[4 * v + 3] = as_h2(w.w);
    } else {
      pair_x4(w.x, w.y, w.z, w.w, &dst[4 * v]);
    }
    if (is_asym(FMT)) {
      s += half_lo(w.x) + half_hi(w.x) + half_lo(w.y) + half_hi(w.y) +
           half_lo(w.z) + half_hi(w.z) + half_lo(w.w) + half_hi(w.w);
    }
  }
  *xsum = s;
}

// sum_k q[k] * x[k] over one 16-byte chunk of codes, binary32.  hw: the
// chunk's high-bit words (5- and 6-bit codes only).
template <int FMT>
__device__ __forceinline__ float chunk_dot(const u32x4 code, const h2* xp,
                                           const u32* hw = nullptr) {
  float a = 0.0f;
  const u32 d[4] = {code.x, code.y, code.z, code.w};
  if (FMT == FMT_S8 || FMT == FMT_F8) {
#pragma unroll
    for (int i = 0; i < 4; i++) {
      h2 q[2];
      if (FMT == FMT_F8) unpack_fp8(d[i], q);
      else unpack8(d[i], q);
      a = __builtin_amdgcn_fdot2(q[0], xp[2 * i + 0], a, false);
      a = __builtin_amdgcn_fdot2(q[1], xp[2 * i + 1], a, false);
    }
  } else {
#pragma unroll
    for (int i = 0; i < 4; i++) {
      h2 q[4];
      if constexpr (hi_bits(FMT) > 0) {
        u32 hlo, hhi;
        hi_words<hi_bits(FMT)>(hw, i, &hlo, &hhi);
        unpack4h<hi_bits(FMT)>(d[i], hlo, hhi, q);
      } else {
        unpack4<FMT == FMT_S4>(d[i], q);
      }
#pragma unroll
      for (int j = 0; j < 4; j++) a = __builtin_amdgcn_fdot2(q[j], xp[4 * i + j], a, false);
    }
  }
  return a;
}

// Byte offset of the high-bit words of chunk kc of row n (5- and 6-bit codes):
// the plane follows the N x K/2 nibbles; a row holds K*HB/8 bytes, a chunk 4*HB.
template <int FMT>
__device__ __forceinline__ u32 hi_offset(int N, int K, u32 n, int kc) {
  constexpr int HB = hi_bits(FMT);
  return (u32)N * (u32)(K / 2) + n * (u32)(K / 8 * HB) + (u32)kc * (4u * HB);
}

template <int FMT, int CPL>
struct PassData {
  u32x4 code[CPL];
  u32 hw[CPL][2];  // high-bit words (5- and 6-bit codes)
  float s[CPL];   // scale (sym) or d*sc_j (asym)
  float t[CPL];   // m*mn_j (asym)
};

template <int FMT, int CPL>
__device__ __forceinline__ void load_pass(PassData<FMT, CPL>& pd,
                                          const uint8_t* __restrict__ qw,
                                          const void* __restrict__ scales,
                                          const void* __restrict__ zeros, int n, int N,
                                          int K, int group, const int* kc) {
  constexpr int CPC = Chunk<FMT>::codes;
  const uint8_t* row = qw + (size_t)n * RowBytes<FMT>::of(K);
#pragma unroll
  for (int c = 0; c < CPL; c++) pd.code[c] = load_stream16(row + (size_t)kc[c] * 16);
  if constexpr (hi_bits(FMT) > 0) {
#pragma unroll
    for (int c = 0; c < CPL; c++) {
      const uint8_t* hp = qw + hi_offset<FMT>(N, K, (u32)n, kc[c]);
      pd.hw[c][0] = *reinterpret_cast<const u32*>(hp);
      pd.hw[c][1] = hi_bits(FMT) == 2 ? reinterpret_cast<const u32*>(hp)[1] : 0u;
    }
  }
#pragma unroll
  for (int c = 0; c < CPL; c++) {
    const int k0 = kc[c] * CPC;
    if (FMT == FMT_F8) {  // one scale for the matrix, applied to the row sum
      pd.s[c] = 1.0f;
      pd.t[c] = 0.0f;
    } else if (is_asym(FMT)) {
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

// Problems of one launch: they share the format, K and M; blocks
// [begin[i], begin[i+1]) belong to entry i.
struct GemvEntry {
  const uint8_t* qw;
  const uint8_t* sc;
  const uint8_t* zr;
  const _Float16* x;
  float* y;
  int N;
};

// The first workgroups of the problems sit in one array at the front, so a
// workgroup finds its problem from one scalar load and compares, then reads
// that problem's entry (two dependent loads, not one per problem).
template <int B>
struct GemvBatch {
  int begin[B];  // first workgroup of each problem
  int count;
  GemvEntry e[B];
};

// Raw scale material of one chunk, kept undecoded until it is used so that
// no wait on its load stands between the loads of a wave.
template <int FMT>
struct ScaleRaw {
  u32x2 s;  // sym: binary16 bits in s.x; asym: scale record
  u32x2 z;  // asym: zero record
};

// Largest workgroup: the activation registers grow with MT*CPL, and a smaller
// workgroup leaves each wave more of the register file.
constexpr int gemv_max_threads(int mt, int cpl) {
  return (mt * cpl >= 4) ? 256 : (mt * cpl >= 2 ? 512 : 1024);
}

// One workgroup: SK waves (one K-slice each) x RB = (64/LPR)*NP rows.  Every
// lane issues the loads of all NP rows it visits before it waits for any of
// them: NP*CPL 16-byte code loads in flight per lane.
//
// Offsets are 32-bit (the host keeps every operand below 2 GiB), so loads use
// a scalar base plus a vector offset.  `ssh` turns a row's code offset into
// its scale offset: a row holds K*bits/8 code bytes and 2K/group scale bytes
// (sym) or K/32 record bytes (asym), a power-of-two ratio.  `gsh` = log2 of
// the group size.
template <int FMT, int LPR, int CPL, int MT, int NP, int B>
__global__ void __launch_bounds__(gemv_max_threads(MT, CPL))
k_gemv(const GemvBatch<B> bt, int Mrows, int K, int gsh, int ssh) {
  constexpr int RPW = 64 / LPR;
  constexpr int RB = RPW * NP;
  constexpr int CPC = Chunk<FMT>::codes;
  constexpr int XP = CPC / 2;
  extern __shared__ float part[];  // [SK][RB][MT]

  // the problem this workgroup belongs to (uniform scan of the table)
  int pi = 0;
#pragma unroll
  for (int i = 1; i < B; i++)
    if (i < bt.count && (int)blockIdx.x >= bt.begin[i]) pi = i;
  const GemvEntry& ent = bt.e[pi];
  const uint8_t* __restrict__ qw = ent.qw;
  const uint8_t* __restrict__ scales = ent.sc;
  const uint8_t* __restrict__ zeros = ent.zr;
  const _Float16* __restrict__ x = ent.x;
  float* __restrict__ y = ent.y;
  const int N = ent.N;
  const int block0 = bt.begin[pi];

  // Every argument in scalar registers before the first load.  Otherwise the
  // compiler fetches the arguments that only the code loads use after it has
  // issued the x loads: one more scalar round trip before the first code load.
  asm volatile("" ::"s"(qw), "s"(scales), "s"(zeros), "s"(x), "s"(y), "s"(N), "s"(block0),
               "s"(K), "s"(gsh), "s"(ssh), "s"(Mrows));

  // FP8: one binary32 scale for the matrix, applied to each finished sum
  const float mscale = (FMT == FMT_F8) ? *reinterpret_cast<const float*>(scales) : 1.0f;

  const int lane = threadIdx.x & 63;
  const int w = threadIdx.x >> 6;
  const int SK = blockDim.x >> 6;
  const int rs = lane / LPR;
  const int li = lane % LPR;
  const int row0 = ((int)blockIdx.x - block0) * RB;
  const u32 row_bytes = (FMT == FMT_S8 || FMT == FMT_F8) ? (u32)K : (u32)K / 2;

  int kc[CPL];
#pragma unroll
  for (int c = 0; c < CPL; c++) kc[c] = w * (LPR * CPL) + c * LPR + li;

  // each visited row (rows past the end re-read the last row) and its code
  // offset: one multiply, then adds (the clamp commutes with the scaling)
  u32 rowi[NP], roff[NP];
  const u32 r0 = (u32)(row0 + rs), rlast = (u32)(N - 1);
  const u32 off0 = r0 * row_bytes, ostep = (u32)RPW * row_bytes, olast = rlast * row_bytes;
#pragma unroll
  for (int p = 0; p < NP; p++) {
    rowi[p] = min(r0 + (u32)(p * RPW), rlast);
    roff[p] = min(off0 + (u32)p * ostep, olast);
  }

  // 1. the activations of this lane's chunks (from L2), issued first: loads of
  //    one wave complete in order, so the pairing below waits for x alone
  constexpr int XV = CPC / 8;  // 16-byte pieces of x per chunk
  u32x4 xraw[MT][CPL][XV];
#pragma unroll
  for (int m = 0; m < MT; m++) {
    // rows past Mrows re-read the last row (always valid) and are zeroed
    // after the loads, so no branch or wait sits between the loads
    const u32 mm = (MT == 1) ? 0u : (u32)min(m, Mrows - 1);
#pragma unroll
    for (int c = 0; c < CPL; c++)
#pragma unroll
      for (int v = 0; v < XV; v++)
        xraw[m][c][v] = reinterpret_cast<const u32x4*>(x + (mm * (u32)K + kc[c] * CPC))[v];
  }
#pragma unroll
  for (int m = 1; m < MT; m++)
    if (m >= Mrows)
#pragma unroll
      for (int c = 0; c < CPL; c++)
#pragma unroll
        for (int v = 0; v < XV; v++) xraw[m][c][v] = u32x4{0, 0, 0, 0};
  __builtin_amdgcn_sched_barrier(0);
  // 2. row by row: the codes this lane takes of the row (5-/6-bit: and their
  //    high bits), then the row's scale material; row p's products below
  //    wait for these loads and the ones before them only
  u32x4 code[NP][CPL];
  u32 hw[NP][CPL][2];
  ScaleRaw<FMT> sr[NP][CPL];
#pragma unroll
  for (int p = 0; p < NP; p++) {
#pragma unroll
    for (int c = 0; c < CPL; c++) code[p][c] = load_stream16(qw + (roff[p] + kc[c] * 16u));
    if constexpr (hi_bits(FMT) > 0) {
#pragma unroll
      for (int c = 0; c < CPL; c++) {
        const uint8_t* hp = qw + hi_offset<FMT>(N, K, rowi[p], kc[c]);
        if constexpr (hi_bits(FMT) == 1) {
          hw[p][c][0] = load_stream4(hp);
          hw[p][c][1] = 0u;
        } else {
          const u32x2 v = load_stream8(hp);
          hw[p][c][0] = v.x;
          hw[p][c][1] = v.y;
        }
      }
    }
    const u32 srow = roff[p] >> ssh;
#pragma unroll
    for (int c = 0; c < CPL; c++) {
      const u32 k0 = (u32)kc[c] * CPC;
      if constexpr (FMT == FMT_F8) {  // the matrix scale is applied to the row sum
        (void)k0;
        sr[p][c].s = u32x2{0, 0};
        sr[p][c].z = u32x2{0, 0};
      } else if constexpr (is_asym(FMT)) {
        const u32 o = srow + (k0 / SUPERBLOCK) * 8u;
        sr[p][c].s = *reinterpret_cast<const u32x2*>(scales + o);
        sr[p][c].z = *reinterpret_cast<const u32x2*>(zeros + o);
      } else {
        sr[p][c].s.x = *reinterpret_cast<const uint16_t*>(scales + srow + ((k0 >> gsh) << 1));
        sr[p][c].s.y = 0;
        sr[p][c].z = u32x2{0, 0};
      }
    }
  }
  __builtin_amdgcn_sched_barrier(0);
  h2 xr[MT][CPL][XP];
  float xs[MT][CPL];
#pragma unroll
  for (int m = 0; m < MT; m++) {
#pragma unroll
    for (int c = 0; c < CPL; c++) {
      float sum = 0.0f;
#pragma unroll
      for (int v = 0; v < XV; v++) {
        const u32x4 wv = xraw[m][c][v];
        if constexpr (FMT == FMT_S8 || FMT == FMT_F8) {
          xr[m][c][4 * v + 0] = as_h2(wv.x);
          xr[m][c][4 * v + 1] = as_h2(wv.y);
          xr[m][c][4 * v + 2] = as_h2(wv.z);
          xr[m][c][4 * v + 3] = as_h2(wv.w);
        } else {
          pair_x4(wv.x, wv.y, wv.z, wv.w, &xr[m][c][4 * v]);
        }
        if constexpr (is_asym(FMT))
          sum += half_lo(wv.x) + half_hi(wv.x) + half_lo(wv.y) + half_hi(wv.y) +
                 half_lo(wv.z) + half_hi(wv.z) + half_lo(wv.w) + half_hi(wv.w);
      }
      xs[m][c] = sum;
    }
  }
  // 4. multiply, row by row
  float acc[NP][MT];
#pragma unroll
  for (int p = 0; p < NP; p++) {
#pragma unroll
    for (int m = 0; m < MT; m++) acc[p][m] = 0.0f;
#pragma unroll
    for (int c = 0; c < CPL; c++) {
      float sc, t = 0.0f;
      if constexpr (FMT == FMT_F8) {
        sc = 1.0f;
      } else if constexpr (is_asym(FMT)) {
        const int j = ((kc[c] * CPC) % SUPERBLOCK) / SB_GROUP;
        sc = record_value(sr[p][c].s, j);
        t = record_value(sr[p][c].z, j);
      } else {
        sc = half_lo(sr[p][c].s.x);
      }
#pragma unroll
      for (int m = 0; m < MT; m++) {
        const float d = chunk_dot<FMT>(code[p][c], xr[m][c], hw[p][c]);
        acc[p][m] = __builtin_fmaf(d, sc, acc[p][m]);
        if (is_asym(FMT)) acc[p][m] = __builtin_fmaf(-t, xs[m][c], acc[p][m]);
      }
    }
  }
  // 5. each (row, activation row) summed over the row's LPR lanes
  constexpr int V = NP * MT;
  if constexpr (V <= LPR) {
    // all sums at once, halving the values per exchange level; the SUB
    // lanes li = idx*SUB .. idx*SUB+SUB-1 end with the total of value idx
    float v[V];
#pragma unroll
    for (int p = 0; p < NP; p++)
#pragma unroll
      for (int m = 0; m < MT; m++) v[p * MT + m] = acc[p][m];
    group_sum_multi<LPR, V>(v, li);
    constexpr int SUB = LPR / V;
    if (li % SUB == 0) {
      const int idx = li / SUB;
      const int p = idx / MT, m = idx % MT;
      const int r = p * RPW + rs;
      const int n = row0 + r;
      if (SK == 1) {
        if (m < Mrows && n < N) y[(u32)m * (u32)N + (u32)n] = v[0] * mscale;
      } else {
        part[(w * RB + r) * MT + m] = v[0];
      }
    }
  } else {
#pragma unroll
    for (int p = 0; p < NP; p++) {
      const int n = row0 + p * RPW + rs;
#pragma unroll
      for (int m = 0; m < MT; m++) {
        const float v = group_sum<LPR>(acc[p][m]);
        if (li == 0) {
          if (SK == 1) {
            if (m < Mrows && n < N) y[(u32)m * (u32)N + (u32)n] = v * mscale;
          } else {
            part[(w * RB + p * RPW + rs) * MT + m] = v;
          }
        }
      }
    }
  }

  if (SK > 1) {
    __syncthreads();
    // Each output (row r, activation row m) adds SK <= 16 partials: the 16
    // lanes of a lane group read one each and add them across the group (one
    // LDS read per lane instead of SK in a row).  Outputs are numbered
    // m * RB + r; a group's lanes share o, so all of them take part in the
    // cross-lane adds.
    const int lg = threadIdx.x >> 4, wl = threadIdx.x & 15;
    for (int o = lg; o < RB * Mrows; o += (int)(blockDim.x >> 4)) {
      const int r = o % RB, m = o / RB;
      const float pv = wl < SK ? part[(wl * RB + r) * MT + m] : 0.0f;
      const float v = group_sum<16>(pv);
      const int n = row0 + r;
      if (wl == 0 && n < N) y[(u32)m * (u32)N + (u32)n] = v * mscale;
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
  const float mscale = (FMT == FMT_F8) ? *static_cast<const float*>(scales) : 1.0f;
  float acc[MT];
#pragma unroll
  for (int m = 0; m < MT; m++) acc[m] = 0.0f;
  for (int c = li; c < chunks; c += LPR) {
    int kc[1] = {c};
    PassData<FMT, 1> pd;
    load_pass<FMT, 1>(pd, qw, scales, zeros, nn, N, K, group, kc);
#pragma unroll
    for (int m = 0; m < MT; m++) {
      if (m < Mrows) {
        h2 xp[XP];
        float xs;
        load_x_chunk<FMT>(x + (size_t)m * K, c * CPC, xp, &xs);
        const float d = chunk_dot<FMT>(pd.code[0], xp, pd.hw[0]);
        acc[m] = __builtin_fmaf(d, pd.s[0], acc[m]);
        if (is_asym(FMT)) acc[m] = __builtin_fmaf(-pd.t[0], xs, acc[m]);
      }
    }
  }
#pragma unroll
  for (int m = 0; m < MT; m++) {
    const float v = group_sum<LPR>(acc[m]);
    if (li == 0 && m < Mrows && n < N) y[(size_t)m * N + n] = v * mscale;
  }
}

// ---------------------------------------------------------------------------
// host side
// ---------------------------------------------------------------------------
static int ilog2(int v) {
  int r = 0;
  while ((1 << (r + 1)) <= v) r++;
  return r;
}


// Launch shapes.  A lane streams NP rows x CPL chunks; a wave covers 64/LPR
// rows and one K-slice of LPR*CPL chunks; a workgroup stacks the K-slices of
// a row block.  The table lists (LPR, CPL, NP) per activation-row count in
// order of preference; the first that splits the row into at most the
// allowed number of waves and gives at least 256 workgroups (or the most) wins.
GemvCfg choose_gemv(int fmt, int M, int N, int K) {
  GemvCfg c{};
  // activation rows per launch: the smallest of 1, 2, 4, 8 covering M (or 8)
  c.mt = M <= 1 ? 1 : (M == 2 ? 2 : (M <= 4 ? 4 : 8));
  const int chunks = (fmt == FMT_S8 || fmt == FMT_F8) ? K / 16 : K / 32;
  // measured on MI355X (width-4096 shapes, weights cold in HBM, graph
  // replay): one 16-byte chunk per lane beats wider per-lane slices, whose
  // extra registers cost occupancy; four rows per lane, or two where that
  // leaves fewer than 512 workgroups (4096x4096: 4.78 -> 4.23 us)
  static const int cand1[][3] = {{16, 1, 4}, {32, 1, 4}, {64, 1, 4}, {16, 1, 8},
                                 {32, 1, 8}, {64, 1, 8}, {16, 2, 4}, {8, 1, 4},
                                 {8, 1, 8}, {16, 1, 2}, {32, 1, 2}, {64, 1, 2},
                                 {8, 1, 2}, {8, 2, 4}, {8, 4, 2}, {16, 1, 1},
                                 {32, 1, 1}, {64, 1, 1}, {8, 1, 1}};
  static const int cand2[][3] = {{16, 1, 4}, {32, 1, 4}, {8, 1, 4}, {64, 1, 4},
                                 {16, 1, 2}, {32, 1, 2}, {8, 1, 2}, {64, 1, 2},
                                 {16, 1, 1}, {32, 1, 1}, {8, 1, 1}, {64, 1, 1}};
  int best = -1, best_blocks = 0;
  const int (*cand)[3] = (c.mt == 1) ? cand1 : cand2;
  const int ncand = (c.mt == 1) ? (int)(sizeof(cand1) / sizeof(cand1[0]))
                                : (int)(sizeof(cand2) / sizeof(cand2[0]));
  // M = 1: 16 lanes per row with four, else two, rows per lane where that
  // gives at least 512 workgroups
  if (c.mt == 1 && chunks % 16 == 0 && chunks / 16 <= gemv_max_threads(1, 1) / 64) {
    if ((N + 15) / 16 >= 512) best = 0;        // {16, 1, 4}
    else if ((N + 7) / 8 >= 512) best = 9;     // {16, 1, 2}
  }
  const bool picked = best >= 0;
  for (int i = 0; i < ncand && !picked; i++) {
    const int lpr = cand[i][0], cpl = cand[i][1], np = cand[i][2];
    if (chunks % (lpr * cpl)) continue;
    const int sk = chunks / (lpr * cpl);
    if (sk < 1 || sk > gemv_max_threads(c.mt, cpl) / 64) continue;
    const int blocks = (N + (64 / lpr) * np - 1) / ((64 / lpr) * np);
    if (blocks >= 256) { best = i; break; }
    if (blocks > best_blocks) { best = i; best_blocks = blocks; }
  }
  const Tuning& tu = tuning();
  const int forced = tu.gemv_lpr;
  if (best < 0 || forced < 0) {  // no usable split: the generic kernel
    c.lpr = 0;
    c.cpl = 1;
    c.npass = 1;
    return c;
  }
  c.lpr = cand[best][0];
  c.cpl = cand[best][1];
  c.npass = cand[best][2];
  // few, long rows at M = 1 (the FFN value of widths 2048..2560): four rows
  // per lane leave 256..320 workgroups; two rows per lane, where that stays
  // at most 640 workgroups, measured faster (weights cold: int4 2048x8192
  // 4.99 -> 4.07 us, int8 2048x8192 5.56 -> 5.08 us, asymmetric 2560x10240
  // 7.37 -> 6.39 us; 4096x16384 keeps four: 512 workgroups, 8.45 against
  // 9.8 us)
  if (c.mt == 1 && c.npass == 4 && (N + (64 / c.lpr) * 2 - 1) / ((64 / c.lpr) * 2) <= 640)
    c.npass = 2;
  // Measured at M = 1 (weights cold, interleaved repeats): the heavier codes
  // of these RWKV-7 shapes run faster in workgroups of at most 8 waves than
  // in the 16-wave ones the rules above give -- 5-bit 4096x16384 13.65 ->
  // 11.70 us, 6-bit 14.57 -> 12.42, 5-bit 2560x10240 7.15 -> 6.78 (64 lanes
  // per row), FP8 16384x4096 14.12 -> 11.48 us, FP8 4096x4096 4.66 -> 4.56
  // (two 16-code chunks per lane, the codes per lane of one 4-bit chunk).
  struct Tuned {
    int fmt, N, K, lpr, cpl, npass;
  };
  static const Tuned tuned[] = {
      {FMT_A5, 4096, 16384, 64, 1, 4}, {FMT_A6, 4096, 16384, 64, 1, 4},
      {FMT_A5, 2560, 10240, 64, 1, 4}, {FMT_F8, 16384, 4096, 16, 2, 2},
      {FMT_F8, 4096, 4096, 16, 2, 2},
  };
  if (c.mt == 1) {
    for (const Tuned& t : tuned) {
      if (t.fmt == fmt && t.N == N && t.K == K && chunks % (t.lpr * t.cpl) == 0 &&
          chunks / (t.lpr * t.cpl) <= gemv_max_threads(1, t.cpl) / 64) {
        c.lpr = t.lpr;
        c.cpl = t.cpl;
        c.npass = t.npass;
        break;
      }
    }
  }
  if (forced > 0) {  // tuning: RQ_GEMV_LPR / RQ_GEMV_CPL / RQ_GEMV_NPASS
    const int cpl = tu.gemv_cpl ? tu.gemv_cpl : c.cpl;
    // only the pairs launch_mt instantiates for this pass size
    const bool inst = (forced == 8 || forced == 16 || forced == 32 || forced == 64) &&
                      (cpl == 1 || (c.mt == 1 && ((forced == 8 && (cpl == 2 || cpl == 4)) ||
                                                  (forced == 16 && cpl == 2))));
    if (inst && chunks % (forced * cpl) == 0 &&
        chunks / (forced * cpl) <= gemv_max_threads(c.mt, cpl) / 64) {
      c.lpr = forced;
      c.cpl = cpl;
    }
  }
  const int np = tu.gemv_npass ? tu.gemv_npass : c.npass;
  if (np == 1 || np == 2 || np == 4 || np == 8) c.npass = np;
  if (c.mt >= 4 && c.npass > 4) c.npass = 4;
  return c;
}

// One launch over up to B problems sharing K (x and y already offset to the
// activation rows of this launch).
struct Launch {
  const Problem* p[GEMV_BATCH];
  const _Float16* x[GEMV_BATCH];
  float* y[GEMV_BATCH];
  int count;
  int K, group, mrows;
};

template <int FMT, int LPR, int CPL, int MT, int NP>
static void launch_t(const Launch& L, hipStream_t s) {
  const int chunks = (FMT == FMT_S8 || FMT == FMT_F8) ? L.K / 16 : L.K / 32;
  const int sk = chunks / (LPR * CPL);
  constexpr int rb = (64 / LPR) * NP;
  const size_t lds = (sk > 1) ? (size_t)sk * rb * MT * sizeof(float) : 0;
  const int gsh = ilog2(L.group > 0 ? L.group : 1);
  // code bytes per row : scale bytes per row = 2^ssh
  //   int4 sym: (K/2)/(2K/G) = G/4; int8 sym: K/(2K/G) = G/2; asym: (K/2)/(K/32) = 16
  const int ssh = is_asym(FMT) ? 4 : (FMT == FMT_S8 ? gsh - 1 : gsh - 2);
  auto fill = [&](GemvEntry* e, int* begin, int* blocks) {
    int b = 0;
    for (int i = 0; i < L.count; i++) {
      e[i] = GemvEntry{static_cast<const uint8_t*>(L.p[i]->qweight),
                       static_cast<const uint8_t*>(L.p[i]->scales),
                       static_cast<const uint8_t*>(L.p[i]->zeros), L.x[i], L.y[i],
                       L.p[i]->N};
      begin[i] = b;
      b += (L.p[i]->N + rb - 1) / rb;
    }
    *blocks = b;
  };
  int blocks = 0;
  if (L.count == 1) {
    GemvBatch<1> bt{};
    fill(bt.e, bt.begin, &blocks);
    bt.count = 1;
    hipLaunchKernelGGL((k_gemv<FMT, LPR, CPL, MT, NP, 1>), dim3(blocks), dim3(64 * sk), lds,
                       s, bt, L.mrows, L.K, gsh, ssh);
  } else {
    GemvBatch<GEMV_BATCH> bt{};
    fill(bt.e, bt.begin, &blocks);
    bt.count = L.count;
    hipLaunchKernelGGL((k_gemv<FMT, LPR, CPL, MT, NP, GEMV_BATCH>), dim3(blocks),
                       dim3(64 * sk), lds, s, bt, L.mrows, L.K, gsh, ssh);
  }
}

template <int FMT, int LPR, int CPL, int MT>
static void launch_np(const Launch& L, const GemvCfg& c, hipStream_t s) {
  switch (c.npass) {
    case 1: return launch_t<FMT, LPR, CPL, MT, 1>(L, s);
    case 2: return launch_t<FMT, LPR, CPL, MT, 2>(L, s);
    case 4: return launch_t<FMT, LPR, CPL, MT, 4>(L, s);
    default:
      if constexpr (MT < 4 && CPL == 1) return launch_t<FMT, LPR, CPL, MT, 8>(L, s);
      else return launch_t<FMT, LPR, CPL, MT, 4>(L, s);
  }
}

template <int FMT, int MT>
static void launch_generic(const Launch& L, hipStream_t s) {
  for (int i = 0; i < L.count; i++) {
    const Problem& p = *L.p[i];
    const int blocks = (p.N * 16 + 255) / 256;
    hipLaunchKernelGGL((k_gemv_generic<FMT, MT>), dim3(blocks), dim3(256), 0, s,
                       static_cast<const uint8_t*>(p.qweight), p.scales, p.zeros, L.x[i],
                       L.y[i], L.mrows, p.N, p.K, p.group);
  }
}

template <int FMT, int MT>
static void launch_mt(const Launch& L, const GemvCfg& c, hipStream_t s) {
  if (c.lpr == 0) return launch_generic<FMT, MT>(L, s);
#define RQ_L(LP, C) \
  if (c.lpr == LP && c.cpl == C) return launch_np<FMT, LP, C, MT>(L, c, s)
  RQ_L(8, 1); RQ_L(16, 1); RQ_L(32, 1); RQ_L(64, 1);
  if constexpr (MT == 1) { RQ_L(8, 2); RQ_L(16, 2); RQ_L(8, 4); }
#undef RQ_L
  // a forced combination that is not instantiated: the generic kernel
  launch_generic<FMT, MT>(L, s);
}

template <int FMT>
static void launch_fmt(const Launch& L, const GemvCfg& c, hipStream_t s) {
  switch (c.mt) {
    case 1: return launch_mt<FMT, 1>(L, c, s);
    case 2: return launch_mt<FMT, 2>(L, c, s);
    case 4: return launch_mt<FMT, 4>(L, c, s);
    default: return launch_mt<FMT, 8>(L, c, s);
  }
}

// Problems p[0..count) share fmt, K, group and M; launches cover up to
// GEMV_BATCH of them each, in passes of c.mt activation rows.
hipError_t launch_gemv_many(const Problem* const* p, int count, const GemvCfg& c,
                            hipStream_t s) {
  const int M = p[0]->M, K = p[0]->K;
  for (int first = 0; first < count; first += GEMV_BATCH) {
    const int n = (count - first < GEMV_BATCH) ? count - first : GEMV_BATCH;
    for (int m0 = 0; m0 < M; m0 += c.mt) {
      Launch L{};
      L.count = n;
      L.K = K;
      L.group = p[0]->group;
      L.mrows = (M - m0 < c.mt) ? M - m0 : c.mt;
      for (int i = 0; i < n; i++) {
        const Problem* q = p[first + i];
        L.p[i] = q;
        L.x[i] = static_cast<const _Float16*>(q->x) + (size_t)m0 * K;
        L.y[i] = q->y + (size_t)m0 * q->N;
      }
      if (p[0]->fmt == FMT_S4) launch_fmt<FMT_S4>(L, c, s);
      else if (p[0]->fmt == FMT_S8) launch_fmt<FMT_S8>(L, c, s);
      else if (p[0]->fmt == FMT_F8) launch_fmt<FMT_F8>(L, c, s);
      else if (p[0]->fmt == FMT_A5) launch_fmt<FMT_A5>(L, c, s);
      else if (p[0]->fmt == FMT_A6) launch_fmt<FMT_A6>(L, c, s);
      else launch_fmt<FMT_A4>(L, c, s);
      hipError_t e = hipGetLastError();
      if (e != hipSuccess) return e;
    }
  }
  return hipSuccess;
}

hipError_t launch_gemv(const Problem& p, const GemvCfg& c, hipStream_t s) {
  const Problem* one = &p;
  return launch_gemv_many(&one, 1, c, s);
}

}  // namespace rq
