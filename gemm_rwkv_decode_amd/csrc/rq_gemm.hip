// rq_gemm.hip -- y = x W^T on the matrix cores for small batches (M <= 64).
//
// Numerics.  The codes are small integers, exact in binary16, and x is
// binary16 already, so one fp16 MFMA per K-step forms the exact products
// q*x and sums them in binary32.  Each MFMA covers K-steps that lie inside
// one quantization group; at the end of a group the binary32 group sum P is
// scaled in binary32: acc += s * P (and, asymmetric, acc -= t * sum_k x).
// (Rounding x or the dequantized weight to a 16-bit type before the product
// would cost up to 2^-9 of a term -- far above the 1e-3 per-output budget on
// activations with massive channels; exact codes avoid that.)
//
// Layout of one MFMA (v_mfma_f32_16x16x32_f16 for 4-bit codes,
// v_mfma_f32_16x16x16_f16 for 8-bit codes): A = x tile [16 m][KS k],
// B = W^T tile [KS k][16 n], D = [16 m][16 n] with lane l holding
// D[4*(l/16) + i][l%16].  Lane l supplies row l%16 of A and column l%16 of B;
// its lane group h = l/16 supplies one quarter of the K-step.  Which k a
// (lane group, element) slot carries is free as long as A and B agree, so a
// lane takes the G/4 consecutive codes of its row that fall in its quarter of
// the group (one 4-, 8- or 16-byte load per group) and the matching x.
//
// Work split.  A workgroup of 4 waves owns 64*NT rows and one K-range (the
// K dimension is split across workgroups when the rows alone would not fill
// the chip).  Wave w owns N-tiles w*NT .. w*NT+NT-1.  The x tile of the
// K-range passes through LDS in chunks of KC k (double buffered, one barrier
// per chunk), shared by the four waves; codes and scales of chunk c+1 are
// loaded into registers while chunk c is multiplied.
//
// Split-K reduction.  When the K dimension is split, every K-range writes its
// partial tile to a workspace with plain stores and a second, small kernel
// adds the partials in K-range order into y.  Results are deterministic; no
// workgroup waits for another and no device-wide fence is needed (a fence per
// workgroup would write the whole L2 back each time).
#include "rq_common.h"
#include "rq_internal.h"


namespace rq {

constexpr int GEMM_WAVES = 4;

// k per LDS chunk of x.  Larger chunks put more code bytes in flight per
// wave (the next chunk is loaded while this one is multiplied); the double
// buffered x tile is 2 * 16*MT * (KC+8) halves.
// At most 8 groups per chunk: every group of a chunk is unrolled.
constexpr int gemm_kc(int fmt, int mt, int g) {
  const int base = fmt == FMT_S8 ? (mt >= 3 ? 128 : 256) : (mt >= 3 ? 256 : 512);
  return base < 8 * g ? base : 8 * g;
}

template <int FMT>
struct MfmaT {
  static constexpr int KS = (FMT == FMT_S8) ? 16 : 32;  // k per MFMA
  static constexpr int EPL = (FMT == FMT_S8) ? 4 : 8;   // elements per lane
};

template <int FMT>
__device__ __forceinline__ f4 mfma_step(const u32* a, const u32* b, f4 c) {
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

// Per-lane register image of one chunk of codes and scale material for NT
// N-tiles: DPC dwords of codes per tile, one scale (sym) or record pair
// (asym) per group.
template <int FMT, int NT, int KC, int G>
struct ChunkRegs {
  static constexpr int GPC = KC / G;                                 // groups per chunk
  static constexpr int DPG = (FMT == FMT_S8) ? G / 16 : G / 32;      // dwords per lane per group
  static constexpr int DPC = GPC * DPG;
  static constexpr int SCW = (GPC + 1) / 2;                         // dwords of scales
  u32 code[NT][DPC];
  u32 sc[NT][SCW];           // sym: binary16 scales of the chunk's groups, 2 per dword
  u32x2 srec[NT], zrec[NT];  // asym: records of the chunk's superblock
};

template <int FMT, int NT, int KC, int G>
__device__ __forceinline__ void load_chunk(ChunkRegs<FMT, NT, KC, G>& r,
                                           const uint8_t* __restrict__ qw,
                                           const void* __restrict__ scales,
                                           const void* __restrict__ zeros, const int* rows,
                                           int K, int kb, int h) {
  using R = ChunkRegs<FMT, NT, KC, G>;
  constexpr int BPL = R::DPG * 4;  // bytes per lane per group
  const size_t row_bytes = (FMT == FMT_S8) ? (size_t)K : (size_t)K / 2;
  const int byte0 = (FMT == FMT_S8) ? kb : kb / 2;  // chunk start in the row
  const int gbytes = (FMT == FMT_S8) ? G : G / 2;   // bytes per group in a row
#pragma unroll
  for (int nt = 0; nt < NT; nt++) {
    const uint8_t* row = qw + (size_t)rows[nt] * row_bytes + byte0 + h * BPL;
#pragma unroll
    for (int g = 0; g < R::GPC; g++) {
      const uint8_t* p = row + g * gbytes;
      if constexpr (BPL == 16) {
        const u32x4 v = load_stream16(p);
        r.code[nt][g * 4 + 0] = v.x; r.code[nt][g * 4 + 1] = v.y;
        r.code[nt][g * 4 + 2] = v.z; r.code[nt][g * 4 + 3] = v.w;
      } else if constexpr (BPL == 8) {
        const u32x2 v = load_stream8(p);
        r.code[nt][g * 2 + 0] = v.x; r.code[nt][g * 2 + 1] = v.y;
      } else {
        r.code[nt][g] = load_stream4(p);
      }
    }
    if constexpr (FMT == FMT_A4) {
      const size_t rec = (size_t)rows[nt] * (K / SUPERBLOCK) + kb / SUPERBLOCK;
      r.srec[nt] = reinterpret_cast<const u32x2*>(scales)[rec];
      r.zrec[nt] = reinterpret_cast<const u32x2*>(zeros)[rec];
    } else {
      // the chunk's GPC scales are contiguous and aligned to their size
      const uint16_t* sp =
          static_cast<const uint16_t*>(scales) + (size_t)rows[nt] * (K / G) + kb / G;
      if constexpr (R::GPC == 1) {
        r.sc[nt][0] = *sp;
      } else if constexpr (R::GPC == 2) {
        r.sc[nt][0] = *reinterpret_cast<const u32*>(sp);
      } else if constexpr (R::GPC == 4) {
        const u32x2 v = *reinterpret_cast<const u32x2*>(sp);
        r.sc[nt][0] = v.x; r.sc[nt][1] = v.y;
      } else {
#pragma unroll
        for (int i = 0; i < R::SCW / 4; i++) {
          const u32x4 v = reinterpret_cast<const u32x4*>(sp)[i];
          r.sc[nt][4 * i + 0] = v.x; r.sc[nt][4 * i + 1] = v.y;
          r.sc[nt][4 * i + 2] = v.z; r.sc[nt][4 * i + 3] = v.w;
        }
      }
    }
  }
}

// Stage x[0..M)[kb, kb+KC) into LDS as binary16 rows of stride KC+8 halves;
// 4-bit formats store every aligned block of 8 as (x0,x4,x1,x5,x2,x6,x3,x7),
// the order unpack4 delivers codes in.  Rows >= M are zero.  For the
// asymmetric format also store the 32-wide group sums of x, [KC/32][MP].
template <int FMT, int MP, int KC>
struct Stage {
  static constexpr int PER = MP * KC / 8 / (64 * GEMM_WAVES);  // 16-byte pieces per thread
  u32x4 v[PER];
};

template <int FMT, int MP, int KC>
__device__ __forceinline__ void stage_load(Stage<FMT, MP, KC>& st,
                                           const _Float16* __restrict__ x, int M, int K,
                                           int kb) {
#pragma unroll
  for (int i = 0; i < Stage<FMT, MP, KC>::PER; i++) {
    const int piece = i * 64 * GEMM_WAVES + threadIdx.x;
    const int m = piece / (KC / 8);
    const int k = kb + (piece % (KC / 8)) * 8;
    if (m < M) st.v[i] = *reinterpret_cast<const u32x4*>(x + (size_t)m * K + k);
    else st.v[i] = u32x4{0, 0, 0, 0};
  }
}

template <int FMT, int MP, int KC>
__device__ __forceinline__ void stage_store(const Stage<FMT, MP, KC>& st, _Float16* xl,
                                            float* xsum) {
  constexpr int XSTR = KC + 8;
#pragma unroll
  for (int i = 0; i < Stage<FMT, MP, KC>::PER; i++) {
    const int piece = i * 64 * GEMM_WAVES + threadIdx.x;
    const int m = piece / (KC / 8);
    const int kk = (piece % (KC / 8)) * 8;
    u32x4 v = st.v[i];
    if (FMT != FMT_S8) {
      h2 p[4];
      pair_x4(v.x, v.y, v.z, v.w, p);
      v = u32x4{as_u32(p[0]), as_u32(p[1]), as_u32(p[2]), as_u32(p[3])};
    }
    *reinterpret_cast<u32x4*>(xl + m * XSTR + kk) = v;
    if (FMT == FMT_A4) {
      // four consecutive threads hold one 32-wide group of one row
      const u32x4 w = st.v[i];
      float s = half_lo(w.x) + half_hi(w.x) + half_lo(w.y) + half_hi(w.y) +
                half_lo(w.z) + half_hi(w.z) + half_lo(w.w) + half_hi(w.w);
      s += __shfl_xor(s, 1, 4);
      s += __shfl_xor(s, 2, 4);
      if ((threadIdx.x & 3) == 0) xsum[(kk / 32) * MP + m] = s;
    }
  }
}

// Multiply one chunk (x in LDS buffer `xb`, codes in `r`) into acc.
template <int FMT, int MT, int NT, int KC, int G>
__device__ __forceinline__ void gemm_chunk(const ChunkRegs<FMT, NT, KC, G>& r,
                                           const _Float16* xb, const float* xsb, int kb,
                                           int h, int col, f4 (&acc)[NT][MT]) {
  constexpr int MP = 16 * MT;
  constexpr int XSTR = KC + 8;
  constexpr int KS = MfmaT<FMT>::KS;
  using R = ChunkRegs<FMT, NT, KC, G>;
  constexpr int GPC = R::GPC;
  constexpr int DPG = R::DPG;  // dwords (= MFMA steps) per lane per group
  constexpr int QPL = G / 4;   // k per lane group per group
#pragma unroll
  for (int g = 0; g < GPC; g++) {
    f4 P[NT][MT];
    // A fragments of every K-step of the group and every M-tile, read from
    // LDS before the first MFMA so the reads overlap each other
    u32 a[DPG][MT][4];
#pragma unroll
    for (int s = 0; s < DPG; s++)
#pragma unroll
      for (int mt = 0; mt < MT; mt++) {
        const _Float16* src = xb + (mt * 16 + col) * XSTR + g * G + h * QPL + s * (KS / 4);
        if constexpr (FMT == FMT_S8) {
          const u32x2 v = *reinterpret_cast<const u32x2*>(src);
          a[s][mt][0] = v.x; a[s][mt][1] = v.y;
        } else {
          const u32x4 v = *reinterpret_cast<const u32x4*>(src);
          a[s][mt][0] = v.x; a[s][mt][1] = v.y; a[s][mt][2] = v.z; a[s][mt][3] = v.w;
        }
      }
#pragma unroll
    for (int s = 0; s < DPG; s++) {
#pragma unroll
      for (int nt = 0; nt < NT; nt++) {
        u32 b[4];
        const u32 d = r.code[nt][g * DPG + s];
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
#pragma unroll
        for (int mt = 0; mt < MT; mt++)
          P[nt][mt] = mfma_step<FMT>(a[s][mt], b, s == 0 ? f4{0, 0, 0, 0} : P[nt][mt]);
      }
    }
    // group epilogue in binary32
    f4 xg[MT];
    if constexpr (FMT == FMT_A4) {
#pragma unroll
      for (int mt = 0; mt < MT; mt++)
        xg[mt] = *reinterpret_cast<const f4*>(&xsb[((g * G) / 32) * MP + mt * 16 + 4 * h]);
    }
#pragma unroll
    for (int nt = 0; nt < NT; nt++) {
      float sc, t = 0.0f;
      if constexpr (FMT == FMT_A4) {
        const int j = ((kb % SUPERBLOCK) + g * G) / SB_GROUP;
        sc = record_value(r.srec[nt], j);
        t = record_value(r.zrec[nt], j);
      } else {
        const u32 pair = r.sc[nt][g / 2];
        sc = (g & 1) ? half_hi(pair) : half_lo(pair);
      }
#pragma unroll
      for (int mt = 0; mt < MT; mt++) {
#pragma unroll
        for (int i = 0; i < 4; i++) {
          float v = __builtin_fmaf(sc, P[nt][mt][i], acc[nt][mt][i]);
          if constexpr (FMT == FMT_A4) v = __builtin_fmaf(-t, xg[mt][i], v);
          acc[nt][mt][i] = v;
        }
      }
    }
    // keep the scheduler from hoisting later groups' LDS reads into this one
    // (it would hold every group's fragments in registers at once)
    if constexpr (MT * NT >= 4) __builtin_amdgcn_sched_barrier(0);
  }
}

template <int FMT, int MT, int NT, int KC, int G>
__global__ void __launch_bounds__(64 * GEMM_WAVES)
k_gemm(const uint8_t* __restrict__ qw, const void* __restrict__ scales,
       const void* __restrict__ zeros, const _Float16* __restrict__ x,
       float* __restrict__ out, int M, int N, int K, int kr) {
  constexpr int MP = 16 * MT;
  constexpr int XSTR = KC + 8;
  constexpr int XSN = (FMT == FMT_A4) ? (KC / 32) * MP : 4;
  using R = ChunkRegs<FMT, NT, KC, G>;

  __shared__ __attribute__((aligned(16))) _Float16 xl[2][MP * XSTR];
  __shared__ __attribute__((aligned(16))) float xsum[2][XSN];

  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int h = lane >> 4;
  const int col = lane & 15;
  const int split = blockIdx.y;
  const int k_begin = split * kr;
  // y itself, or this K-range's slice of the partial-sum workspace
  float* __restrict__ y = out + (size_t)split * M * N;
  const int nchunks = kr / KC;
  const int row_base = blockIdx.x * (64 * NT) + wave * (16 * NT);

  int rows[NT];
#pragma unroll
  for (int nt = 0; nt < NT; nt++) rows[nt] = min(row_base + nt * 16 + col, N - 1);

  f4 acc[NT][MT];
#pragma unroll
  for (int nt = 0; nt < NT; nt++)
#pragma unroll
    for (int mt = 0; mt < MT; mt++) acc[nt][mt] = f4{0, 0, 0, 0};

  // Chunks alternate between (LDS buffer 0, registers r0) and (1, r1); the
  // next chunk's x and codes are fetched while the current one is multiplied.
  Stage<FMT, MP, KC> st;
  R r0, r1;
  stage_load<FMT, MP, KC>(st, x, M, K, k_begin);
  load_chunk<FMT, NT, KC, G>(r0, qw, scales, zeros, rows, K, k_begin, h);
  stage_store<FMT, MP, KC>(st, xl[0], xsum[0]);
  __syncthreads();

  for (int c = 0; c < nchunks; c += 2) {
    const int kb = k_begin + c * KC;
    const bool more1 = c + 1 < nchunks;
    if (more1) {
      stage_load<FMT, MP, KC>(st, x, M, K, kb + KC);
      load_chunk<FMT, NT, KC, G>(r1, qw, scales, zeros, rows, K, kb + KC, h);
    }
    gemm_chunk<FMT, MT, NT, KC, G>(r0, xl[0], xsum[0], kb, h, col, acc);
    if (more1) stage_store<FMT, MP, KC>(st, xl[1], xsum[1]);
    __syncthreads();
    if (!more1) break;
    const bool more2 = c + 2 < nchunks;
    if (more2) {
      stage_load<FMT, MP, KC>(st, x, M, K, kb + 2 * KC);
      load_chunk<FMT, NT, KC, G>(r0, qw, scales, zeros, rows, K, kb + 2 * KC, h);
    }
    gemm_chunk<FMT, MT, NT, KC, G>(r1, xl[1], xsum[1], kb + KC, h, col, acc);
    if (more2) stage_store<FMT, MP, KC>(st, xl[0], xsum[0]);
    __syncthreads();
  }

  // ---- write out -----------------------------------------------------------
#pragma unroll
  for (int nt = 0; nt < NT; nt++) {
    const int n = row_base + nt * 16 + col;
#pragma unroll
    for (int mt = 0; mt < MT; mt++)
#pragma unroll
      for (int i = 0; i < 4; i++) {
        const int m = mt * 16 + 4 * h + i;
        if (m < M && n < N) y[(size_t)m * N + n] = acc[nt][mt][i];
      }
  }
}

// y[i] = sum over K-ranges s = 0..splits-1 (in order) of ws[s][i], i < count.
__global__ void __launch_bounds__(256)
k_split_reduce(const float* __restrict__ ws, float* __restrict__ y, size_t count,
               int splits) {
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < count;
       i += (size_t)gridDim.x * blockDim.x) {
    float v = 0.0f;
    for (int sp = 0; sp < splits; sp++) v += ws[(size_t)sp * count + i];
    y[i] = v;
  }
}

// ---------------------------------------------------------------------------
// host side
// ---------------------------------------------------------------------------
size_t gemm_workspace_floats(const GemmCfg& c, int M, int N) {
  return c.splits > 1 ? (size_t)c.splits * M * N : 0;
}


bool gemm_supports(int fmt, int M, int K, int group) {
  const int mt = (M + 15) / 16;
  return K % gemm_kc(fmt, mt, group) == 0;
}

GemmCfg choose_gemm(int fmt, int M, int N, int K, int group) {
  GemmCfg c{};
  c.mt = (M + 15) / 16;
  c.nt = 1;  // two N-tiles per wave measured slower (registers, occupancy)
  const Tuning& tu = tuning();
  if (tu.gemm_nt) c.nt = tu.gemm_nt == 1 ? 1 : 2;
  if (c.mt > 2) c.nt = 1;
  const int rowblocks = (N + 64 * c.nt - 1) / (64 * c.nt);
  const int kc = gemm_kc(fmt, c.mt, group);
  const int maxsplit = K / kc;  // the caller has checked K % kc == 0
  // About 256 workgroups (512 for K >= 8192, whose rows are long enough to
  // split further), measured best on MI355X for the RWKV-7 shapes; splits must
  // divide K into whole chunks and the partial sums stay under 64 MiB.
  const int target = (K >= 8192) ? 512 : 256;
  int want = (target + rowblocks - 1) / rowblocks;
  if (tu.gemm_splits) want = tu.gemm_splits;
  if (want > maxsplit) want = maxsplit;
  if (want < 1) want = 1;
  int s = want;
  while (s > 1 && (maxsplit % s != 0 || (size_t)s * M * N * 4 > ((size_t)64 << 20))) s--;
  c.splits = s;
  return c;
}

template <int FMT, int MT, int NT, int G>
static void launch_g(const Problem& p, const GemmCfg& c, float* ws, hipStream_t s) {
  constexpr int KC = gemm_kc(FMT, MT, G);
  const int rowblocks = (p.N + 64 * NT - 1) / (64 * NT);
  const int kr = p.K / c.splits;
  float* out = (c.splits > 1) ? ws : p.y;
  hipLaunchKernelGGL((k_gemm<FMT, MT, NT, KC, G>), dim3(rowblocks, c.splits),
                     dim3(64 * GEMM_WAVES), 0, s, static_cast<const uint8_t*>(p.qweight),
                     p.scales, p.zeros, static_cast<const _Float16*>(p.x), out, p.M, p.N,
                     p.K, kr);
  if (c.splits > 1) {
    const size_t count = (size_t)p.M * p.N;
    size_t blocks = (count + 255) / 256;
    if (blocks > 1024) blocks = 1024;
    hipLaunchKernelGGL(k_split_reduce, dim3((unsigned)blocks), dim3(256), 0, s, ws, p.y,
                       count, c.splits);
  }
}

template <int FMT, int MT, int NT>
static void launch_group(const Problem& p, const GemmCfg& c, float* ws, hipStream_t s) {
  if constexpr (FMT == FMT_S8) {
    if (p.group == 16) return launch_g<FMT, MT, NT, 16>(p, c, ws, s);
    if (p.group == 32) return launch_g<FMT, MT, NT, 32>(p, c, ws, s);
    return launch_g<FMT, MT, NT, 64>(p, c, ws, s);
  } else if constexpr (FMT == FMT_A4) {
    return launch_g<FMT, MT, NT, 32>(p, c, ws, s);
  } else {
    if (p.group == 32) return launch_g<FMT, MT, NT, 32>(p, c, ws, s);
    if (p.group == 64) return launch_g<FMT, MT, NT, 64>(p, c, ws, s);
    return launch_g<FMT, MT, NT, 128>(p, c, ws, s);
  }
}

template <int FMT>
static void launch_fmt(const Problem& p, const GemmCfg& c, float* ws, hipStream_t s) {
#define RQ_G(MT_, NT_) \
  if (c.mt == MT_ && c.nt == NT_) return launch_group<FMT, MT_, NT_>(p, c, ws, s)
  // two N-tiles per wave only up to M = 32 (above, the registers run out)
  RQ_G(1, 2); RQ_G(2, 2);
  RQ_G(1, 1); RQ_G(2, 1); RQ_G(3, 1); RQ_G(4, 1);
#undef RQ_G
}

hipError_t launch_gemm(const Problem& p, const GemmCfg& c, float* ws, hipStream_t s) {
  if (p.fmt == FMT_S4) launch_fmt<FMT_S4>(p, c, ws, s);
  else if (p.fmt == FMT_S8) launch_fmt<FMT_S8>(p, c, ws, s);
  else launch_fmt<FMT_A4>(p, c, ws, s);
  return hipGetLastError();
}

}  // namespace rq
