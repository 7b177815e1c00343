// rq_gemm_impl.h -- the matrix-core kernel k_mm and its launch templates,
// shared by rq_gemm_plan.h (plan choice), rq_gemm.hip (dispatch) and the
// per-format translation units rq_gemm_<format>.hip that instantiate it (so
// the instances compile in parallel).
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
// Work split (MI355X: 256 CUs, 64 B/clk per CU from L2, ~160 B/clk of LDS
// reads).  A workgroup owns WR*NT*16 rows and the whole K range (or one
// K-range when K is split across workgroups).  Its W = WR*WK multiplying
// waves form WR row groups of NT 16-row tiles times WK K-slices; MM_XP + MM_CP
// more waves only copy.  K advances in rounds of WK*KC k: in a round, K-slice
// w multiplies the w-th KC-wide chunk.  The copying waves stream the round's
// x tile [MP][WK*KC] (from L2) and the rows' codes and scale material (from
// HBM) into LDS rings of DX+1 and DC+1 round slots, DX and DC rounds ahead,
// with global->LDS buffer loads; one barrier per round hands a slot over, and
// every multiplying wave reads its MFMA fragments from there.  At the end
// the WK K-slices of a row group are added in a fixed order through LDS.
// Every workgroup stages all of x (MP*K*2 bytes), and a wave issues about one
// 1 KB global->LDS copy per 50 cycles, so the copies bound the 16-row plans;
// splitting K over workgroups shortens them at the price of a partial-sum
// workspace and the in-launch reduction below, used only where that wins.
//
// Split-K reduction, in the same launch.  When the K dimension is split, each
// multiplying wave that stores a 16-row tile writes its partial tile to the
// workspace with device-scope (coherent) stores, waits until they are
// acknowledged, and counts itself on the tile's counter with one relaxed
// device-scope atomic.  The wave that arrives last -- it reads splits - 1 --
// loads the other K-ranges' partials with device-scope loads, adds them in
// K-range order (its own from registers: the value it stored) and writes y,
// then resets the counter to 0 for the next launch.  No wave ever waits for
// another, so no launch order or residency is assumed, and the sum is the same
// whichever wave is last: results are deterministic.  No fence is used: a
// __threadfence() writes the L2 back and costs about 50 ns per workgroup,
// serialized over the device; coherent stores need no write-back.
#pragma once

#include "rq_common.h"
#include "rq_internal.h"

#include <type_traits>

namespace rq {

// One byte per code (int8, FP8); FP8 has no per-group scale material (one
// binary32 scale for the matrix, applied to the finished sums), and its
// groups are nominal 64-wide units of work.
constexpr bool mm_byte(int fmt) { return fmt == FMT_S8 || fmt == FMT_F8; }
constexpr int MM_F8_GROUP = 64;

template <int FMT>
struct MfmaT {
  static constexpr int KS = mm_byte(FMT) ? 16 : 32;  // k per MFMA
};

template <int FMT>
__device__ __forceinline__ f4 mfma_step(const u32* a, const u32* b, f4 c) {
  if constexpr (mm_byte(FMT)) {
    const h4 av = __builtin_bit_cast(h4, u32x2{a[0], a[1]});
    const h4 bv = __builtin_bit_cast(h4, u32x2{b[0], b[1]});
    return __builtin_amdgcn_mfma_f32_16x16x16f16(av, bv, c, 0, 0, 0);
  } else {
    const h8 av = __builtin_bit_cast(h8, u32x4{a[0], a[1], a[2], a[3]});
    const h8 bv = __builtin_bit_cast(h8, u32x4{b[0], b[1], b[2], b[3]});
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(av, bv, c, 0, 0, 0);
  }
}

// Rounds are sized so one x round of the M-tile is about 32 KB (rd = 1) or
// 16 KB (rd = 2): k per round 1024 / MT rounded down to a power of two, / rd.
constexpr int mm_round_target(int mt) { return mt == 1 ? 1024 : (mt == 2 ? 512 : 256); }

// k per wave chunk: whole groups, at least one MFMA K-step, at most 8 groups.
constexpr int mm_kc(int fmt, int mt, int wk, int g, int rd) {
  const int want = mm_round_target(mt) / rd / wk;
  const int lo = g > 32 ? g : 32;
  const int kc = want > lo ? want : lo;
  return kc < 8 * g ? kc : 8 * g;
}

constexpr int LDS_LIMIT = 160 * 1024;
constexpr int MM_XP = 3;           // waves copying x
constexpr int MM_CP = 1;           // waves copying codes and scale material
constexpr int MM_MAX_XDEPTH = 6;   // x rounds copied ahead (x comes from L2)
constexpr int MM_MAX_CDEPTH = 13;  // code rounds copied ahead (codes come from HBM)
constexpr int MM_CODE_AHEAD = 32 * 1024;  // code bytes to keep in flight, at least
constexpr int MM_MAX_SPLITS = 8;          // K-ranges a product may be split into

// Rows of x staged per round: 16 per M-tile, or 4 / 8 when M <= 4 / 8 (one
// M-tile whose MFMA rows past them re-read the staged rows: their outputs are
// never stored); xr = 0 means 16 * mt.
constexpr int mm_xr(int mt, int xr) { return xr > 0 ? xr : 16 * mt; }

// Bytes of one x round slot ([MP][ROUND+8] halves) and of one code round
// slot (the workgroup's code rows [ROWS][ROUND*bits/8], then its scale
// material).
constexpr int mm_round(int fmt, int mt, int wk, int g, int rd) {
  return wk * mm_kc(fmt, mt, wk, g, rd);
}
constexpr int mm_xslot(int fmt, int mt, int g, int wk, int rd, int xr = 0) {
  return mm_xr(mt, xr) * (mm_round(fmt, mt, wk, g, rd) + 8) * 2;
}
// Scale material is copied in whole 64-lane copies of 4-byte elements; each
// kind's region is padded to whole copies (the lanes past the last row copy
// the last row again into the padding), so no copy needs a lane predicate.
// 5-/6-bit codes add the rows' high-bit plane for the round (round/8 bytes
// per high bit and row), in 16-byte pieces, padded to whole copies too.
constexpr int mm_hi_copies(int fmt, int round, int rows) {
  return (rows * (round / 8 * hi_bits(fmt)) / 16 + 63) / 64;
}
constexpr int mm_cslot(int fmt, int mt, int g, int wr, int wk, int nt, int rd) {
  const int round = mm_round(fmt, mt, wk, g, rd);
  const int rows = 16 * nt * wr;
  const int codes = rows * (mm_byte(fmt) ? round : round / 2) + mm_hi_copies(fmt, round, rows) * 1024;
  if (fmt == FMT_F8) return codes;
  const int srd = is_asym(fmt) ? 2 * (round / SUPERBLOCK) : round / g / 2;  // dwords per row
  const int region = (rows * srd + 63) / 64 * 256;
  return codes + (is_asym(fmt) ? 2 : 1) * region;
}
// copy instructions per round: x row segments; code pieces and scale dwords
constexpr int mm_xcopies(int fmt, int mt, int g, int wk, int rd, int xr = 0) {
  const int round = mm_round(fmt, mt, wk, g, rd);
  const int seg = round * 2 < 1024 ? round * 2 : 1024;
  return mm_xr(mt, xr) * (round * 2 / seg);
}
constexpr int mm_ccopies(int fmt, int mt, int g, int wr, int wk, int nt, int rd) {
  const int round = mm_round(fmt, mt, wk, g, rd);
  const int rows = 16 * nt * wr;
  const int cc = (rows * (mm_byte(fmt) ? round : round / 2) / 16 + 63) / 64;
  const int sd = fmt == FMT_F8 ? 0
                 : is_asym(fmt) ? rows * (round / SUPERBLOCK) * 2 : rows * (round / g) / 2;
  return cc + mm_hi_copies(fmt, round, rows) + (is_asym(fmt) ? 2 : 1) * ((sd + 63) / 64);
}
// Rounds copied ahead.  Code slots to keep MM_CODE_AHEAD bytes in flight
// come first (at least 2 rounds), then as many x rounds as fit (at most
// MM_MAX_XDEPTH), then the rest of the LDS goes to more code rounds; each
// copying wave's pending copies must fit its counter (63).
constexpr int mm_xdepth(int fmt, int mt, int g, int wr, int wk, int nt, int rd, int occ,
                        int xr = 0) {
  const int lds = LDS_LIMIT / occ;
  const int xs = mm_xslot(fmt, mt, g, wk, rd, xr), cs = mm_cslot(fmt, mt, g, wr, wk, nt, rd);
  const int xpp = (mm_xcopies(fmt, mt, g, wk, rd, xr) + MM_XP - 1) / MM_XP;
  int dcmin = (MM_CODE_AHEAD / occ + cs - 1) / cs;
  dcmin = dcmin < 2 ? 2 : (dcmin > MM_MAX_CDEPTH ? MM_MAX_CDEPTH : dcmin);
  int d = MM_MAX_XDEPTH;
  while (d > 0 && ((d + 1) * xs + (dcmin + 1) * cs > lds || (d - 1) * xpp > 63)) d--;
  return d;
}
constexpr int mm_cdepth(int fmt, int mt, int g, int wr, int wk, int nt, int rd, int occ,
                        int xr = 0) {
  const int left = LDS_LIMIT / occ - (mm_xdepth(fmt, mt, g, wr, wk, nt, rd, occ, xr) + 1) *
                                         mm_xslot(fmt, mt, g, wk, rd, xr);
  const int cs = mm_cslot(fmt, mt, g, wr, wk, nt, rd);
  const int cpp = (mm_ccopies(fmt, mt, g, wr, wk, nt, rd) + MM_CP - 1) / MM_CP;
  int d = MM_MAX_CDEPTH;
  while (d > 0 && ((d + 1) * cs > left || (d - 1) * cpp > 63)) d--;
  return d;
}

// Workgroup arrangements: row groups x K-slices x 16-row tiles per wave, the
// round size (rd = 2: half the default round) and the workgroups meant to
// share a CU (occ = 2: each takes at most half the LDS and of the registers).
struct Plan {
  int wr, wk, nt, rd;
  int occ = 1;
};
static constexpr Plan kPlans[] = {
    {1, 4, 1, 1},  // 0: 16 rows, 4 K-slices
    {1, 8, 1, 1},  // 1: 16 rows, 8 K-slices
    {4, 1, 1, 1},  // 2: 64 rows, whole chunks per wave
    {2, 4, 1, 1},  // 3: 32 rows, 4 K-slices
    {2, 2, 1, 1},  // 4: 32 rows, 2 K-slices
    {4, 2, 1, 1},  // 5: 64 rows, 2 K-slices
    {1, 4, 1, 2},  // 6: as 0, half rounds
    {4, 2, 1, 2},  // 7: as 5, half rounds
    {2, 4, 1, 2},  // 8: as 3, half rounds
    {4, 1, 1, 2},  // 9: as 2, half rounds
    // two 16-row tiles per wave: each A fragment read from LDS feeds two MFMAs
    {2, 2, 2, 1},  // 10: 64 rows, 2 K-slices
    {2, 4, 2, 1},  // 11: 64 rows, 4 K-slices
    {1, 8, 2, 1},  // 12: 32 rows, 8 K-slices
    {1, 4, 2, 1},  // 13: 32 rows, 4 K-slices
    {4, 2, 2, 1},  // 14: 128 rows, 2 K-slices
    // three row groups: 48-row workgroups (12288 rows -> 256 workgroups)
    {3, 2, 1, 1},  // 15: 48 rows, 2 K-slices
    {3, 2, 1, 2},  // 16: as 15, half rounds
    {3, 4, 1, 1},  // 17: 48 rows, 4 K-slices
    // two workgroups per CU (half the LDS each), half rounds
    {1, 8, 1, 2, 2},  // 18: 16 rows, 8 K-slices
    {1, 4, 1, 2, 2},  // 19: 16 rows, 4 K-slices
    {4, 2, 1, 2, 2},  // 20: 64 rows, 2 K-slices
    {2, 4, 1, 2, 2},  // 21: 32 rows, 4 K-slices
    {2, 2, 2, 2, 2},  // 22: 64 rows, 2 K-slices, two tiles per wave
    {3, 2, 1, 2, 2},  // 23: 48 rows, 2 K-slices
    // 128 rows per workgroup (a quarter of the x staging per row of 32-row
    // ones), half rounds; meant for K split over workgroups
    {8, 1, 1, 2},  // 24: 8 row groups, whole chunks per wave
    {4, 2, 2, 2},  // 25: 4 row groups of two tiles, 2 K-slices
    {4, 1, 2, 2},  // 26: 4 row groups of two tiles, whole chunks per wave
};
constexpr int kNumPlans = sizeof(kPlans) / sizeof(kPlans[0]);

// Compile-time shape of one kernel instance.
template <int FMT_, int MT_, int NT_, int WR_, int WK_, int G_, int RD_, int OCC_ = 1,
          int XR_ = 0>
struct Mm {
  static constexpr int FMT = FMT_, MT = MT_, NT = NT_, WR = WR_, WK = WK_, G = G_, RD = RD_;
  static constexpr int XR = mm_xr(MT_, XR_);        // x rows staged per round
  static_assert(XR == 16 * MT || (MT == 1 && (XR == 4 || XR == 8)), "x rows");
  static constexpr int OCC = OCC_;                  // workgroups meant to share a CU
  static constexpr int LDS_MAX = LDS_LIMIT / OCC;   // LDS bytes this workgroup may take
  static constexpr int W = WR * WK;                 // multiplying waves
  static constexpr int THREADS = 64 * (W + MM_XP + MM_CP);
  static constexpr int KC = mm_kc(FMT, MT, WK, G, RD);  // k per wave chunk
  static constexpr int ROUND = WK * KC;             // k per round
  static constexpr int DX = mm_xdepth(FMT, MT, G, WR, WK, NT, RD, OCC, XR);  // x rounds ahead
  static constexpr int DC = mm_cdepth(FMT, MT, G, WR, WK, NT, RD, OCC, XR);  // code rounds ahead
  static constexpr int MP = XR;                     // staged activation rows
  static constexpr int TR = 16 * NT;                // rows per wave
  static constexpr int ROWS = TR * WR;              // rows per workgroup
  static constexpr int XSTR = ROUND + 8;            // halves per LDS row of x
  static constexpr int GPC = KC / G;                // groups per chunk
  static constexpr int DPG = mm_byte(FMT) ? G / 16 : G / 32;  // dwords per lane per group
  static constexpr int BPL = DPG * 4;               // code bytes per lane per group
  static constexpr int GB = mm_byte(FMT) ? G : G / 2;  // code bytes per group of a row
  static constexpr int RS = mm_byte(FMT) ? ROUND : ROUND / 2;  // code bytes per row and round
  static constexpr int PR = RS / 16;                // 16-byte code pieces per row and round
  // piece swizzle: row n's piece p sits at n*PR + (p ^ (n & SWZ)); 16 rows of
  // a fragment read then start in 16 (PR >= 16) or 8 different bank groups
  static constexpr int SWZ = PR >= 16 ? 15 : 7;
  static constexpr int NSB = ROUND / SUPERBLOCK;    // superblocks per round (asym)
  // scale dwords per row and round: sym, the round's binary16 scales; asym,
  // per kind (scale records, zero records) two dwords per superblock
  static constexpr int SRD = (FMT == FMT_F8) ? 0 : is_asym(FMT) ? 2 * NSB : ROUND / G / 2;
  // 5-/6-bit codes: the high-bit plane of the round, HRS bytes per row
  static constexpr int HB = hi_bits(FMT);
  static constexpr int HRS = ROUND / 8 * HB;
  static constexpr int HPR = HRS / 16;              // 16-byte pieces per row and round
  // LDS: x ring (DX+1 slots), then code ring (DC+1 slots)
  static constexpr int XSLOT = mm_xslot(FMT, MT, G, WK, RD, XR);
  static constexpr int CSLOT = mm_cslot(FMT, MT, G, WR, WK, NT, RD);
  static constexpr int CRING = (DX + 1) * XSLOT;    // byte offset of the code ring
  static constexpr int C_OFF = 0;                   // within a code slot
  static constexpr int HN = mm_hi_copies(FMT, ROUND, ROWS);  // high-bit copies
  static constexpr int H_OFF = ROWS * RS;           // high-bit plane (rows of HRS bytes)
  static constexpr int S_OFF = H_OFF + HN * 1024;
  static constexpr int Z_OFF = S_OFF + ((ROWS * SRD + 63) / 64) * 256;  // asym zero records
  // copies of one round
  static constexpr int SEG = ROUND * 2 < 1024 ? ROUND * 2 : 1024;  // x bytes per copy
  static constexpr int SEG_LANES = SEG / 16;
  static constexpr int SEGS_PER_ROW = ROUND * 2 / SEG;
  static constexpr int XN = MP * SEGS_PER_ROW;
  static constexpr int CPIECES = ROWS * PR;
  static constexpr int CN = (CPIECES + 63) / 64;
  static constexpr int SDK = ROWS * SRD;            // scale dwords per kind
  static constexpr int SNK = (SDK + 63) / 64;
  static constexpr int SN = (is_asym(FMT) ? 2 : 1) * SNK;
  static constexpr int CHN = CN + HN;                // code and high-bit copies
  static constexpr int COPIES = XN + CHN + SN;
  static constexpr int XPP = (XN + MM_XP - 1) / MM_XP;         // per x-copying wave
  static constexpr int CPP = (CHN + SN + MM_CP - 1) / MM_CP;   // per code-copying wave
  static constexpr int RED = (WK > 1) ? W * 64 * NT * MT * 4 : 0;  // floats
  static constexpr int LDS_BYTES = CRING + (DC + 1) * CSLOT;
  // structural conditions (the host's plan_fits checks the same)
  static constexpr bool VALID =
      GPC >= 1 && GPC <= 8 && KC % G == 0 &&
      (!is_asym(FMT) || (SUPERBLOCK % KC == 0 && ROUND % SUPERBLOCK == 0)) &&
      (is_asym(FMT) || (ROUND / G) % 2 == 0) && PR >= 8 && (PR & (PR - 1)) == 0 &&
      SEG_LANES <= 64 && ROUND * 2 % SEG == 0 && THREADS <= 1024;
  // accumulator tiles per wave the register file holds without spilling:
  // 12 waves per workgroup leave 168 registers a lane (half that with two
  // workgroups per CU)
  static constexpr bool REGS = NT * MT * OCC <= (THREADS > 512 ? 4 : 8);
  static constexpr bool FITS = VALID && REGS && DX >= 1 && DC >= 1 &&
                               LDS_BYTES <= LDS_MAX && RED * 4 <= LDS_MAX;
  static_assert(!FITS || (XN == mm_xcopies(FMT, MT, G, WK, RD, XR) &&
                          CHN + SN == mm_ccopies(FMT, MT, G, WR, WK, NT, RD)),
                "copy counts");
  static_assert(CPIECES % 64 == 0, "code rows are whole copies");
  static_assert(!FITS || ((DX - 1) * XPP <= 63 && (DC - 1) * CPP <= 63),
                "wait counts fit the counter");
};

// s_waitcnt on the vector-memory counter only (gfx9 encoding: vmcnt in bits
// 3:0 and 15:14; expcnt 7 and lgkmcnt 15 mean "do not wait").
template <int N>
__device__ __forceinline__ void wait_vm() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | ((N >> 4) << 14));
}

// Wait until at most k*STEP vector loads of this wave are pending, k in
// [0, KMAX] (a switch: the counter takes an immediate).
template <int STEP, int KMAX>
__device__ __forceinline__ void wait_vm_rounds(int k) {
  if constexpr (KMAX > 0) {
    if (k >= KMAX) {
      wait_vm<KMAX * STEP>();
      return;
    }
    wait_vm_rounds<STEP, KMAX - 1>(k);
  } else {
    wait_vm<0>();
  }
}

// Global->LDS copies as buffer loads: the array's base in a buffer resource
// and the round's offset in scalar registers, the lane's offset (fixed for
// the whole launch) in a vector register, so a copy needs no address
// arithmetic of its own (a global load with a 64-bit address costs one VALU
// add per copy).  The resource's range is the whole 32-bit offset space; the
// host keeps every array below 2 GiB.  Word 3: 32-bit data format, which
// untyped loads require on this architecture.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t mm_rsrc(const void* p) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), 0, -1, 0x00020000);
}
__device__ __forceinline__ void lds_copy16(__amdgpu_buffer_rsrc_t r, void* dst, u32 voff,
                                           u32 soff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)dst, 16,
                                           voff, soff, 0, 0);
}
__device__ __forceinline__ void lds_copy4(__amdgpu_buffer_rsrc_t r, void* dst, u32 voff,
                                          u32 soff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)dst, 4,
                                           voff, soff, 0, 0);
}

// Copy c of a round, c in [0, COPIES): x row segments first (rows >= M
// repeat row M-1; they only feed outputs that are never stored), then code
// pieces (row n's 16-byte piece p stored at position n*PR + (p ^ (n & SWZ)), so
// that the 16 rows a fragment read touches spread over the banks), then, for
// 5-/6-bit codes, high-bit pieces (row n's piece p at n*HPR + p), then scale
// dwords (row n's dword d at n*SRD + d; asym: scale records, then zero
// records).  The lanes past the last row repeat it into the region's padding.
// copy_off gives this lane's byte offset from the copy's base,
// which does not change from round to round; copy_soff/copy_dst the uniform
// parts.
template <class S>
__device__ __forceinline__ u32 copy_off(int c, int M, int K, int N, int row0, int lane) {
  if (c < S::XN) {
    const int m = c / S::SEGS_PER_ROW, seg = c % S::SEGS_PER_ROW;
    const int mr = m < M ? m : M - 1;
    return ((u32)mr * (u32)K + (u32)(seg * (S::SEG / 2) + lane * 8)) * 2u;
  } else if (c < S::XN + S::CN) {
    const int pos = (c - S::XN) * 64 + lane;  // piece position in the slot
    const int n = pos / S::PR, sp = pos % S::PR;
    const int row = min(row0 + min(n, S::ROWS - 1), N - 1);
    const u32 row_bytes = mm_byte(S::FMT) ? (u32)K : (u32)K / 2;
    return (u32)row * row_bytes + (u32)(sp ^ (n & S::SWZ)) * 16u;
  } else if (c < S::XN + S::CHN) {
    // high-bit pieces: the round's HRS bytes of a row, K/8*HB bytes apart
    constexpr int HPR1 = S::HPR > 0 ? S::HPR : 1;
    const int pos = (c - S::XN - S::CN) * 64 + lane;
    const int n = pos / HPR1, hp = pos % HPR1;
    const int row = min(row0 + min(n, S::ROWS - 1), N - 1);
    return (u32)row * (u32)(K / 8 * S::HB) + (u32)hp * 16u;
  } else {
    // scale copies (none for FP8: SNK is 0 and no copy index reaches here)
    const int j = (c - S::XN - S::CHN) % (S::SNK > 0 ? S::SNK : 1);
    const int q = j * 64 + lane;
    constexpr int SRD1 = S::SRD > 0 ? S::SRD : 1;
    const int n = q / SRD1, dw = q % SRD1;
    const int row = min(row0 + min(n, S::ROWS - 1), N - 1);
    if constexpr (is_asym(S::FMT))
      return ((u32)row * (u32)(K / SUPERBLOCK) * 2u + (u32)dw) * 4u;
    else  // K / G is even (host check): a row's scales start on a dword
      return ((u32)row * (u32)(K / S::G) / 2u + (u32)dw) * 4u;
  }
}

// The round's byte offset of copy c from its array's base (k0: the round's
// first k): x, the codes, the high-bit plane (which follows every row's
// nibbles), the scales (asym: and the zero records).
template <class S>
__device__ __forceinline__ u32 copy_soff(int c, u32 k0) {
  if (c < S::XN) return k0 * 2u;
  if (c < S::XN + S::CN) return mm_byte(S::FMT) ? k0 : k0 / 2u;
  if (c < S::XN + S::CHN) return k0 / 8u * (u32)S::HB;
  if constexpr (is_asym(S::FMT)) return k0 / (u32)SUPERBLOCK * 8u;
  else return k0 / (u32)S::G * 2u;
}

// Destination offset of copy c within its slot.
template <class S>
__device__ __forceinline__ int copy_dst(int c) {
  if (c < S::XN) {
    const int m = c / S::SEGS_PER_ROW, seg = c % S::SEGS_PER_ROW;
    return (m * S::XSTR + seg * (S::SEG / 2)) * 2;
  }
  if (c < S::XN + S::CN) return S::C_OFF + (c - S::XN) * 1024;
  if (c < S::XN + S::CHN) return S::H_OFF + (c - S::XN - S::CN) * 1024;
  const int i = c - S::XN - S::CHN;
  return ((is_asym(S::FMT) && i >= S::SNK) ? S::Z_OFF : S::S_OFF) +
         (i % (S::SNK > 0 ? S::SNK : 1)) * 256;
}

// Multiply one chunk into acc from the LDS x slot `xsl` and code slot `sl`:
// x of the chunk at column kx of the x tile, code bytes at cb0 of the rows'
// round segments,
// the chunk's groups j0 .. j0+GPC-1 of the round's scales.  kb is the
// chunk's first k.
template <class S>
__device__ __forceinline__ void mm_chunk(const char* __restrict__ xsl,
                                         const char* __restrict__ sl, int kx, int cb0, int j0,
                                         int kb, int wr, int h, int col,
                                         f4 (&acc)[S::NT][S::MT]) {
  constexpr int FMT = S::FMT, G = S::G, MT = S::MT, NT = S::NT, DPG = S::DPG;
  constexpr int KS = MfmaT<FMT>::KS;
  constexpr int QPL = G / 4;  // k per lane group per group
  const _Float16* xb = reinterpret_cast<const _Float16*>(xsl);
  // asymmetric: the chunk lies inside one superblock, so each row's scale and
  // zero records are read and split once per chunk: the binary16 bases
  // converted, the 48-bit sub-code fields moved down to the chunk's first group
  float dbase[NT], mbase[NT];
  uint64_t sfield[NT], zfield[NT];
  if constexpr (is_asym(FMT)) {
    const int kin0 = kb % S::ROUND;  // the chunk's first k within the round
    const int sb = kin0 / SUPERBLOCK, jb = (kin0 % SUPERBLOCK) / SB_GROUP;
#pragma unroll
    for (int nt = 0; nt < NT; nt++) {
      const int n = wr * S::TR + nt * 16 + col;
      const u32* sr = reinterpret_cast<const u32*>(sl + S::S_OFF) + n * S::SRD + 2 * sb;
      const u32* zr = reinterpret_cast<const u32*>(sl + S::Z_OFF) + n * S::SRD + 2 * sb;
      dbase[nt] = half_lo(sr[0]);
      mbase[nt] = half_lo(zr[0]);
      sfield[nt] = ((((uint64_t)sr[1] << 32) | sr[0]) >> 16) >> (6 * jb);
      zfield[nt] = ((((uint64_t)zr[1] << 32) | zr[0]) >> 16) >> (6 * jb);
    }
  }
  // one group's LDS fragments: the lane's codes (row n, bytes [cb0 + g*GB +
  // h*BPL, +BPL) of the row), for 5-/6-bit codes the high-bit dwords of the
  // row's 32-code chunk, and the A fragments of every K-step and M-tile
  struct Frag {
    u32 code[S::NT][S::DPG];
    u32 hw[S::NT][2];
    u32 a[S::DPG][S::MT][4];
  };
  auto fetch = [&](int g, Frag& f) {
#pragma unroll
    for (int nt = 0; nt < NT; nt++) {
      const int n = wr * S::TR + nt * 16 + col;
      const int byte = cb0 + g * S::GB + h * S::BPL;
      const char* src =
          sl + S::C_OFF + (n * S::PR + ((byte / 16) ^ (n & S::SWZ))) * 16 + byte % 16;
      if constexpr (S::BPL == 16) {
        const u32x4 v = *reinterpret_cast<const u32x4*>(src);
        f.code[nt][0] = v.x; f.code[nt][1] = v.y; f.code[nt][2] = v.z; f.code[nt][3] = v.w;
      } else if constexpr (S::BPL == 8) {
        const u32x2 v = *reinterpret_cast<const u32x2*>(src);
        f.code[nt][0] = v.x; f.code[nt][1] = v.y;
      } else {
        f.code[nt][0] = *reinterpret_cast<const u32*>(src);
      }
    }
    if constexpr (S::HB > 0) {
#pragma unroll
      for (int nt = 0; nt < NT; nt++) {
        const int n = wr * S::TR + nt * 16 + col;
        const u32* hp = reinterpret_cast<const u32*>(sl + S::H_OFF + n * S::HRS +
                                                     (cb0 / 16 + g) * 4 * S::HB);
        f.hw[nt][0] = hp[0];
        f.hw[nt][1] = S::HB == 2 ? hp[1] : 0u;
      }
    }
#pragma unroll
    for (int s = 0; s < DPG; s++)
#pragma unroll
      for (int mt = 0; mt < MT; mt++) {
        const _Float16* src =
            xb + (S::XR < 16 ? (col & (S::XR - 1)) : mt * 16 + col) * S::XSTR + kx + g * G +
            h * QPL + s * (KS / 4);
        if constexpr (mm_byte(FMT)) {
          const u32x2 v = *reinterpret_cast<const u32x2*>(src);
          f.a[s][mt][0] = v.x; f.a[s][mt][1] = v.y;
        } else {
          const u32x4 v = *reinterpret_cast<const u32x4*>(src);
          f.a[s][mt][0] = v.x; f.a[s][mt][1] = v.y; f.a[s][mt][2] = v.z; f.a[s][mt][3] = v.w;
        }
      }
  };
  // group g's MFMAs and binary32 epilogue
  auto compute = [&](int g, const Frag& f) {
    f4 P[NT][MT];
#pragma unroll
    for (int s = 0; s < DPG; s++) {
#pragma unroll
      for (int nt = 0; nt < NT; nt++) {
        u32 b[4];
        const u32 d = f.code[nt][s];
        if constexpr (mm_byte(FMT)) {
          h2 q[2];
          if constexpr (FMT == FMT_F8) unpack_fp8(d, q);
          else unpack8(d, q);
          b[0] = as_u32(q[0]); b[1] = as_u32(q[1]);
        } else if constexpr (S::HB > 0) {
          // this lane's nibble dword is dword h of the group's 32-code chunk
          u32 hlo, hhi;
          hi_words<S::HB>(f.hw[nt], h, &hlo, &hhi);
          h2 q[4];
          unpack4h<S::HB>(d, hlo, hhi, q);
          // pairs (q0,q4) (q1,q5) (q2,q6) (q3,q7) -> k order (q0,q1) .. (q6,q7)
          const u32 p0 = as_u32(q[0]), p1 = as_u32(q[1]), p2 = as_u32(q[2]), p3 = as_u32(q[3]);
          b[0] = __builtin_amdgcn_perm(p1, p0, 0x05040100u);
          b[1] = __builtin_amdgcn_perm(p3, p2, 0x05040100u);
          b[2] = __builtin_amdgcn_perm(p1, p0, 0x07060302u);
          b[3] = __builtin_amdgcn_perm(p3, p2, 0x07060302u);
        } else {
          h2 q[4];
          unpack4n<FMT == FMT_S4>(d, q);
          b[0] = as_u32(q[0]); b[1] = as_u32(q[1]);
          b[2] = as_u32(q[2]); b[3] = as_u32(q[3]);
        }
#pragma unroll
        for (int mt = 0; mt < MT; mt++) {
          // FP8: no group scale, so the products accumulate straight into acc
          const f4 c0 = (FMT == FMT_F8) ? acc[nt][mt] : f4{0, 0, 0, 0};
          P[nt][mt] = mfma_step<FMT>(f.a[s][mt], b, s == 0 ? c0 : P[nt][mt]);
        }
      }
    }
    // asymmetric: the group sums of x, in the layout of P, from one more MFMA
    // against codes that are all 1 (a group is one K-step)
    f4 xg[MT];
    if constexpr (is_asym(FMT)) {
      const u32 one2 = 0x3C003C00u;  // binary16 (1, 1)
      const u32 ones[4] = {one2, one2, one2, one2};
#pragma unroll
      for (int mt = 0; mt < MT; mt++) xg[mt] = mfma_step<FMT>(f.a[0][mt], ones, f4{0, 0, 0, 0});
    }
    // group epilogue in binary32
#pragma unroll
    for (int nt = 0; nt < NT && FMT == FMT_F8; nt++)
#pragma unroll
      for (int mt = 0; mt < MT; mt++) acc[nt][mt] = P[nt][mt];
#pragma unroll
    for (int nt = 0; nt < NT && FMT != FMT_F8; nt++) {
      const int n = wr * S::TR + nt * 16 + col;
      float sc, t = 0.0f;
      if constexpr (is_asym(FMT)) {
        // group g of the chunk: sub-codes at bits 6g..6g+5 of the moved fields;
        // d * sc_j and m * mn_j are exact in binary32 (11 + 6 significant bits)
        (void)n;
        sc = dbase[nt] * (float)(u32)((sfield[nt] >> (6 * g)) & 0x3Fu);
        t = mbase[nt] * (float)(u32)((zfield[nt] >> (6 * g)) & 0x3Fu);
      } else {
        const int j = j0 + g;  // group within the round
        const u32 pair = reinterpret_cast<const u32*>(sl + S::S_OFF)[n * S::SRD + j / 2];
        sc = (j & 1) ? half_hi(pair) : half_lo(pair);
        // converted once here: the compiler would otherwise fold the conversion
        // into each of the MT*4 FMAs below as v_fma_mix_f32, which issues at half
        // the rate of v_fma_f32 (same result: the conversion is exact)
        asm volatile("" : "+v"(sc));
      }
#pragma unroll
      for (int mt = 0; mt < MT; mt++) {
#pragma unroll
        for (int i = 0; i < 4; i++) {
          float v = __builtin_fmaf(sc, P[nt][mt][i], acc[nt][mt][i]);
          if constexpr (is_asym(FMT)) v = __builtin_fmaf(-t, xg[mt][i], v);
          acc[nt][mt][i] = v;
        }
      }
    }
  };
  if constexpr (NT == 1 && MT <= 2 && S::OCC == 1 && S::XR == 16 * MT) {
    // one 16-row tile per wave, one workgroup per CU, M <= 32: group g+1's
    // fragments are read from LDS while group g is multiplied (two register
    // sets; the scheduling barriers keep that order), which hides the LDS
    // latency (int4, M = 32: 2-7% faster for these plans).  Plans with two
    // tiles per wave hold twice the fragments and were 1-5% slower this way,
    // and so were the M <= 8 steps, whose plans share a CU between two
    // workgroups (half the registers each): 5-11%.
    Frag f[2];
    fetch(0, f[0]);
#pragma unroll
    for (int g = 0; g < S::GPC; g++) {
      if (g + 1 < S::GPC) fetch(g + 1, f[(g + 1) & 1]);
      __builtin_amdgcn_sched_barrier(0);
      compute(g, f[g & 1]);
      __builtin_amdgcn_sched_barrier(0);
    }
  } else {
#pragma unroll
    for (int g = 0; g < S::GPC; g++) {
      Frag f;
      fetch(g, f);
      compute(g, f);
      // keep the scheduler from hoisting later groups' LDS reads into this one
      // (it would hold every group's fragments in registers at once)
      if constexpr (MT * NT >= 4) __builtin_amdgcn_sched_barrier(0);
    }
  }
}

// The copying waves.  x waves take the round's x copies p, p+XP, ...; the
// code wave takes its code and scale copies.  Each group runs its own number
// of rounds ahead of the multiplying waves (x: DX, codes: DC); a wave's
// copies complete in issue order, so before the barrier of round r it waits
// until only rounds r+1 .. r+ahead-1 may be in flight.  After the barrier
// the slots of round r-1 are free and take round r+ahead.  (A copy index
// past the end repeats the last copy: every wave issues the same number.)
template <class S, bool XW>
__device__ __forceinline__ void copy_rounds(int p, char* lds, const _Float16* x,
                                            const uint8_t* qw, const void* scales,
                                            const void* zeros, int M, int K, int N, int row0,
                                            int k_begin, int nrounds, int lane) {
  constexpr int NC = XW ? S::XPP : S::CPP;
  constexpr int AHEAD = XW ? S::DX : S::DC;
  static_assert(MM_CP == 1, "the code wave's copies are compile-time");
  // copy index of position i (uniform)
  auto cidx = [&](int i) {
    return XW ? min(i * MM_XP + p, S::XN - 1) : S::XN + min(i, S::CHN + S::SN - 1);
  };
  u32 off[NC];
#pragma unroll
  for (int i = 0; i < NC; i++) off[i] = copy_off<S>(cidx(i), M, K, N, row0, lane);
  const __amdgpu_buffer_rsrc_t rx = mm_rsrc(x), rc = mm_rsrc(qw), rs = mm_rsrc(scales),
                               rz = mm_rsrc(zeros),
                               rh = mm_rsrc(qw + (S::HB > 0 ? (size_t)N * (K / 2) : 0));
  auto issue = [&](int t) {
    char* slot = XW ? lds + (t % (S::DX + 1)) * S::XSLOT
                    : lds + S::CRING + (t % (S::DC + 1)) * S::CSLOT;
    const u32 k0 = (u32)(k_begin + t * S::ROUND);
#pragma unroll
    for (int i = 0; i < NC; i++) {
      const int c = cidx(i);
      char* dst = slot + copy_dst<S>(c);
      if constexpr (XW) {
        // every x copy of a round has the same lane count
        if (S::SEG_LANES == 64 || lane < S::SEG_LANES)
          lds_copy16(rx, dst, off[i], copy_soff<S>(c, k0));
      } else {
        // Code, high-bit and scale copies are whole-wave instructions with no
        // lane predicate: the code rows are whole copies, the other regions
        // are padded to whole copies.  (Predicated copies of different lane
        // counts in one unrolled sequence were once merged by the compiler
        // into a block that issued some of them under another copy's mask.)
        const int cc = S::XN + (i < S::CHN + S::SN ? i : S::CHN + S::SN - 1);
        const u32 so = copy_soff<S>(cc, k0);
        if (cc < S::XN + S::CN) {
          lds_copy16(rc, dst, off[i], so);
        } else if (cc < S::XN + S::CHN) {
          lds_copy16(rh, dst, off[i], so);
        } else {
          const bool zr = is_asym(S::FMT) && (cc - S::XN - S::CHN) >= S::SNK;
          lds_copy4(zr ? rz : rs, dst, off[i], so);
        }
      }
    }
  };
#pragma unroll 1
  for (int t = 0; t < AHEAD; t++)
    if (t < nrounds) issue(t);
#pragma unroll 1
  for (int r = 0; r < nrounds; r++) {
    wait_vm_rounds<NC, AHEAD - 1>(min(AHEAD - 1, nrounds - 1 - r));
    __builtin_amdgcn_s_barrier();
    if (r + AHEAD < nrounds) issue(r + AHEAD);
  }
}

// Problems of one launch (they share the format, M, K and the group size):
// workgroups [begin[i], begin[i+1]) along x belong to entry i.  The starts sit
// in one array at the front, so a workgroup finds its problem from one scalar
// load and compares, then reads that entry.
struct MmEntry {
  const uint8_t* qw;
  const void* sc;
  const void* zr;
  const _Float16* x;
  float* out;  // y, or the partial-sum workspace when K is split
  float* y;    // y (the split-K result goes here)
  int N;
};

// Split-K workspace layout: SPLIT_COUNTERS arrival counters (one per 16-row
// tile, zero between launches), then the partial tiles [split][M][N].
__device__ __forceinline__ void store_coherent(float* p, float v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float load_coherent(const float* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
struct MmBatch {
  int begin[MM_BATCH];
  int count;
  MmEntry e[MM_BATCH];
};

template <class S>
__global__ void __launch_bounds__(S::THREADS, S::OCC)
k_mm(const MmBatch bt, int M, int K, int kr, unsigned* counters) {
  constexpr int NT = S::NT, MT = S::MT;
  static_assert(S::FITS, "LDS budget and prefetch depth");
  constexpr int LDS_BYTES = S::LDS_BYTES > S::RED * 4 ? S::LDS_BYTES : S::RED * 4;
  __shared__ __attribute__((aligned(16))) char lds[LDS_BYTES];

  // this workgroup's problem (uniform scan of the table)
  int pi = 0;
#pragma unroll
  for (int i = 1; i < MM_BATCH; i++)
    if (i < bt.count && (int)blockIdx.x >= bt.begin[i]) pi = i;
  const MmEntry& e = bt.e[pi];
  const uint8_t* __restrict__ qw = e.qw;
  const void* __restrict__ scales = e.sc;
  const void* __restrict__ zeros = e.zr;
  const _Float16* __restrict__ x = e.x;
  const int N = e.N;
  const int begin = bt.begin[pi];
  float* const out = e.out;
  // The entry's fields and the launch arguments in scalar registers at once:
  // otherwise the compiler spreads their loads over two dependent round trips
  // before the first copy (int4 1-3% faster).  Not for FP8, whose matrix
  // scale, read through the entry, would then be waited for here (2-6%
  // slower).
  if constexpr (S::FMT != FMT_F8)
    asm volatile("" ::"s"(qw), "s"(scales), "s"(zeros), "s"(x), "s"(N), "s"(begin), "s"(out),
                 "s"(M), "s"(K), "s"(kr));

  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int split = blockIdx.y;
  const int k_begin = split * kr;
  // y itself, or this K-range's slice of the partial-sum workspace
  float* __restrict__ y = out + (size_t)split * M * N;
  // FP8: the matrix scale multiplies every finished sum (or partial sum)
  const float mscale = (S::FMT == FMT_F8) ? *static_cast<const float*>(scales) : 1.0f;
  const int nrounds = kr / S::ROUND;
  const int row0 = ((int)blockIdx.x - begin) * S::ROWS;

  if (wave >= S::W) {
    if (wave < S::W + MM_XP)
      copy_rounds<S, true>(wave - S::W, lds, x, qw, scales, zeros, M, K, N, row0, k_begin,
                           nrounds, lane);
    else
      copy_rounds<S, false>(wave - S::W - MM_XP, lds, x, qw, scales, zeros, M, K, N, row0,
                            k_begin, nrounds, lane);
  } else {
    // ---- multiplying wave: row group wr, K-slice wk
    const int wk = wave % S::WK;
    const int wr = wave / S::WK;
    const int h = lane >> 4;
    const int col = lane & 15;
    f4 acc[NT][MT];
#pragma unroll
    for (int nt = 0; nt < NT; nt++)
#pragma unroll
      for (int mt = 0; mt < MT; mt++) acc[nt][mt] = f4{0, 0, 0, 0};
    const int kx = wk * S::KC;  // chunk within the round
    const int cb0 = mm_byte(S::FMT) ? kx : kx / 2;
    const int j0 = kx / S::G;
    for (int r = 0; r < nrounds; r++) {
      __builtin_amdgcn_s_barrier();  // round r is in LDS
      mm_chunk<S>(lds + (r % (S::DX + 1)) * S::XSLOT,
                  lds + S::CRING + (r % (S::DC + 1)) * S::CSLOT, kx, cb0, j0,
                  k_begin + r * S::ROUND + kx, wr, h, col, acc);
    }
    if constexpr (S::WK > 1) {
      __syncthreads();  // every wave is done with the slots
      float* red = reinterpret_cast<float*>(lds);
#pragma unroll
      for (int nt = 0; nt < NT; nt++)
#pragma unroll
        for (int mt = 0; mt < MT; mt++)
#pragma unroll
          for (int i = 0; i < 4; i++)
            red[((wave * NT + nt) * MT + mt) * 256 + i * 64 + lane] = acc[nt][mt][i];
      __syncthreads();
      if (wk != 0) return;
#pragma unroll
      for (int nt = 0; nt < NT; nt++)
#pragma unroll
        for (int mt = 0; mt < MT; mt++)
#pragma unroll
          for (int i = 0; i < 4; i++) {
            float v = acc[nt][mt][i];
#pragma unroll
            for (int q = 1; q < S::WK; q++)
              v += red[(((wave + q) * NT + nt) * MT + mt) * 256 + i * 64 + lane];
            acc[nt][mt][i] = v;
          }
    }
    const int splits = gridDim.y;
    if (splits == 1) {
#pragma unroll
      for (int nt = 0; nt < NT; nt++) {
        const int n = row0 + wr * S::TR + nt * 16 + col;
#pragma unroll
        for (int mt = 0; mt < MT; mt++)
#pragma unroll
          for (int i = 0; i < 4; i++) {
            const int m = mt * 16 + 4 * h + i;
            if (m < M && n < N) y[(size_t)m * N + n] = acc[nt][mt][i] * mscale;
          }
      }
      return;
    }
    // ---- K split: partial tile, arrival, and the last wave's sum
#pragma unroll
    for (int nt = 0; nt < NT; nt++) {
      const int n = row0 + wr * S::TR + nt * 16 + col;
#pragma unroll
      for (int mt = 0; mt < MT; mt++)
#pragma unroll
        for (int i = 0; i < 4; i++) {
          const int m = mt * 16 + 4 * h + i;
          if (m < M && n < N) store_coherent(&y[(size_t)m * N + n], acc[nt][mt][i] * mscale);
        }
    }
    // the stores are acknowledged before the arrival is counted
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    __builtin_amdgcn_s_waitcnt(0);
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    unsigned* ctr = counters + (row0 + wr * S::TR) / 16;
    unsigned before = 0;
    if (lane == 0)
      before = __hip_atomic_fetch_add(ctr, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    before = __builtin_amdgcn_readfirstlane(before);
    if (before != (unsigned)(splits - 1)) return;
    if (lane == 0) __hip_atomic_store(ctr, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    float* __restrict__ yf = e.y;
    const size_t plane = (size_t)M * N;
    // the K-ranges' partials added in K-range order, four K-ranges at a time:
    // the loads of four ranges for every tile of the wave are issued together
    // before any is used (one round trip per four ranges)
    constexpr int SB = 4;
    float sum[NT][MT][4];
#pragma unroll
    for (int nt = 0; nt < NT; nt++)
#pragma unroll
      for (int mt = 0; mt < MT; mt++)
#pragma unroll
        for (int i = 0; i < 4; i++) sum[nt][mt][i] = 0.0f;
#pragma unroll
    for (int s0 = 0; s0 < MM_MAX_SPLITS; s0 += SB) {
      if (s0 >= splits) break;
      float part[SB][NT][MT][4];
#pragma unroll
      for (int q = 0; q < SB; q++)
#pragma unroll
        for (int nt = 0; nt < NT; nt++) {
          const int nc = min(row0 + wr * S::TR + nt * 16 + col, N - 1);
#pragma unroll
          for (int mt = 0; mt < MT; mt++)
#pragma unroll
            for (int i = 0; i < 4; i++) {
              const int sp = s0 + q;
              const int mc = min(mt * 16 + 4 * h + i, M - 1);
              part[q][nt][mt][i] =
                  (sp < splits && sp != split)
                      ? load_coherent(out + sp * plane + (size_t)mc * N + nc)
                      : acc[nt][mt][i] * mscale;
            }
        }
#pragma unroll
      for (int q = 0; q < SB; q++)
#pragma unroll
        for (int nt = 0; nt < NT; nt++)
#pragma unroll
          for (int mt = 0; mt < MT; mt++)
#pragma unroll
            for (int i = 0; i < 4; i++)
              if (s0 + q < splits) sum[nt][mt][i] += part[q][nt][mt][i];
    }
#pragma unroll
    for (int nt = 0; nt < NT; nt++) {
      const int n = row0 + wr * S::TR + nt * 16 + col;
#pragma unroll
      for (int mt = 0; mt < MT; mt++)
#pragma unroll
        for (int i = 0; i < 4; i++) {
          const int m = mt * 16 + 4 * h + i;
          if (m < M && n < N) yf[(size_t)m * N + n] = sum[nt][mt][i];
        }
    }
    return;
  }
  // copying waves join the reduction's two barriers
  if constexpr (S::WK > 1) {
    __syncthreads();
    __syncthreads();
  }
}

// One launch over p[0..count), count <= MM_BATCH; K is split (c.splits > 1,
// counters and partial sums in ws) only for a single problem.
template <class S>
hipError_t launch_s(const Problem* const* p, int count, const GemmCfg& c, float* ws,
                    hipStream_t s) {
  if constexpr (!S::FITS) {
    // plan_ok never chooses such a plan; a caller that does gets an error
    // instead of an output that was never written
    return hipErrorInvalidValue;
  } else {
  MmBatch bt{};
  int blocks = 0;
  for (int i = 0; i < count; i++) {
    bt.e[i] = MmEntry{static_cast<const uint8_t*>(p[i]->qweight), p[i]->scales, p[i]->zeros,
                      static_cast<const _Float16*>(p[i]->x),
                      c.splits > 1 ? ws + SPLIT_COUNTERS : p[i]->y, p[i]->y, p[i]->N};
    bt.begin[i] = blocks;
    blocks += (p[i]->N + S::ROWS - 1) / S::ROWS;
  }
  bt.count = count;
  const int M = p[0]->M, K = p[0]->K;
  unsigned* counters = c.splits > 1 ? reinterpret_cast<unsigned*>(ws) : nullptr;
  hipLaunchKernelGGL((k_mm<S>), dim3(blocks, c.splits), dim3(S::THREADS), 0, s, bt, M, K,
                     K / c.splits, counters);
  return hipGetLastError();
  }
}

// The instance of plan P (an index into kPlans); XR as in Mm.
template <int FMT, int MT, int G, int P, int XR = 0>
using MmPlan = Mm<FMT, MT, kPlans[P].nt, kPlans[P].wr, kPlans[P].wk, G, kPlans[P].rd,
                  kPlans[P].occ, XR>;

template <int FMT, int MT, int G, int XR, int P = 0>
hipError_t launch_plan(const Problem* const* p, int n, const GemmCfg& c, float* ws,
                       hipStream_t s) {
  if constexpr (P >= kNumPlans) {
    return hipErrorInvalidValue;  // no such plan
  } else {
    if (c.plan == P) return launch_s<MmPlan<FMT, MT, G, P, XR>>(p, n, c, ws, s);
    return launch_plan<FMT, MT, G, XR, P + 1>(p, n, c, ws, s);
  }
}

template <int FMT, int MT, int XR = 0>
hipError_t launch_group(const Problem* const* p, int n, const GemmCfg& c, float* ws,
                        hipStream_t s) {
  const int g = p[0]->group;
  if constexpr (FMT == FMT_F8) {
    return launch_plan<FMT, MT, MM_F8_GROUP, XR>(p, n, c, ws, s);
  } else if constexpr (FMT == FMT_S8) {
    if (g == 16) return launch_plan<FMT, MT, 16, XR>(p, n, c, ws, s);
    if (g == 32) return launch_plan<FMT, MT, 32, XR>(p, n, c, ws, s);
    return launch_plan<FMT, MT, 64, XR>(p, n, c, ws, s);
  } else if constexpr (is_asym(FMT)) {
    return launch_plan<FMT, MT, 32, XR>(p, n, c, ws, s);
  } else {
    if (g == 32) return launch_plan<FMT, MT, 32, XR>(p, n, c, ws, s);
    if (g == 64) return launch_plan<FMT, MT, 64, XR>(p, n, c, ws, s);
    return launch_plan<FMT, MT, 128, XR>(p, n, c, ws, s);
  }
}

template <int FMT>
hipError_t launch_fmt(const Problem* const* p, int n, const GemmCfg& c, float* ws,
                      hipStream_t s) {
  switch (c.mt) {
    case 1:
      if (c.xr == 4) return launch_group<FMT, 1, 4>(p, n, c, ws, s);
      if (c.xr == 8) return launch_group<FMT, 1, 8>(p, n, c, ws, s);
      return launch_group<FMT, 1>(p, n, c, ws, s);
    case 2: return launch_group<FMT, 2>(p, n, c, ws, s);
    case 3: return launch_group<FMT, 3>(p, n, c, ws, s);
    default: return launch_group<FMT, 4>(p, n, c, ws, s);
  }
}

// One per format, each in its own translation unit (rq_gemm_<format>.hip).
hipError_t launch_gemm_fmt_s4(const Problem* const* p, int n, const GemmCfg& c, float* ws, hipStream_t s);
hipError_t launch_gemm_fmt_s8(const Problem* const* p, int n, const GemmCfg& c, float* ws, hipStream_t s);
hipError_t launch_gemm_fmt_a4(const Problem* const* p, int n, const GemmCfg& c, float* ws, hipStream_t s);
hipError_t launch_gemm_fmt_a5(const Problem* const* p, int n, const GemmCfg& c, float* ws, hipStream_t s);
hipError_t launch_gemm_fmt_a6(const Problem* const* p, int n, const GemmCfg& c, float* ws, hipStream_t s);
hipError_t launch_gemm_fmt_f8(const Problem* const* p, int n, const GemmCfg& c, float* ws, hipStream_t s);

}  // namespace rq
