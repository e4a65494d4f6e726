// Device-side building blocks shared by the MFMA GEMM kernels for gfx950:
// vector types, buffer resources, the tile raster, the LDS XOR swizzle, MFMA
// fragment reads (direct and transposing), scheduling hints, E4M3 widening and the
// alpha/beta epilogue.  Included by the kernel translation units only.
#pragma once

#include <type_traits>

#include "e4m3_codec.h"
#include "gemm_internal.h"

namespace dbgemm {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef int i32x2 __attribute__((ext_vector_type(2)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef unsigned short u16x4 __attribute__((ext_vector_type(4)));

typedef __attribute__((address_space(3))) char lds_char;
#define LDS_PTR(T, base, off) ((__attribute__((address_space(3))) T*)((base) + (off)))

constexpr uint32_t kOOB = 0x80000000u;  // offset past every buffer's num_records

__device__ inline __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}

// Workgroup id -> output tile.  First an XCD-aware remap: the hardware hands
// consecutive workgroup ids to the XCDs round-robin, so id b runs on XCD b % xcd;
// the remap gives each XCD one contiguous run of the raster order, which keeps the
// A and B panels that neighbouring tiles share inside one XCD's L2.  Then a grouped
// raster: `group` tile-rows are walked column by column (or the transpose).  Both
// maps are bijections, so every tile is computed exactly once.  With split-K the ids
// cover tiles x splits; the splits of one tile are neighbours in the remapped order
// (so they run on one XCD) and `split` is the id's position among them.
// xcd < -1 (the K-banded grids, walked longest tile first): -xcd XCDs take runs of four
// consecutive raster positions in turn, so each XCD's L2 serves runs of neighbouring tiles
// while every XCD keeps to the same stretch of the longest-first order.
__device__ inline int xcd_remap(int bid, int total, int xcd) {
  if (xcd > 1) {
    const int q = total / xcd;
    if (bid < q * xcd) return (bid % xcd) * q + bid / xcd;
  } else if (xcd < -1) {
    const int n = -xcd, chunk = 4 * n;
    if (bid < total / chunk * chunk) return bid / chunk * chunk + (bid % n) * 4 + (bid / n) % 4;
  }
  return bid;
}

// Position L of the raster order -> output tile (tm, tn).
__device__ inline void raster_tile(int L, const GemmArgs& a, int& tm, int& tn);

__device__ inline void tile_of(int bid, const GemmArgs& a, int& tm, int& tn, int& split) {
  int L = xcd_remap(bid, grid_tiles(a), a.xcd);
  split = L % a.splits;
  L /= a.splits;
  raster_tile(L, a, tm, tn);
}

__device__ inline void raster_tile(int L, const GemmArgs& a, int& tm, int& tn) {
  if (a.tri) {
    // triangle of the tile grid, row by row: tile row r holds tiles (r, 0 .. r), which
    // start at L = r(r+1)/2.  r from the square root, then corrected to be exact.
    int r = (int)((__builtin_sqrtf(8.f * (float)L + 1.f) - 1.f) * 0.5f);
    while (r > 0 && r * (r + 1) / 2 > L) --r;
    while ((r + 1) * (r + 2) / 2 <= L) ++r;
    const int c = L - r * (r + 1) / 2;
    tm = a.tri == TRI_LOWER ? r : c;  // the upper triangle is the transposed walk
    tn = a.tri == TRI_LOWER ? c : r;
    return;
  }
  const int major = a.raster_n ? a.tiles_m : a.tiles_n;  // tiles along the walk
  const int minor = a.raster_n ? a.tiles_n : a.tiles_m;  // grouped dimension
  const int width = a.group * major;
  const int g = L / width;
  const int first = g * a.group;
  const int gs = min(minor - first, a.group);
  const int r = L - g * width;
  const int i_minor = first + r % gs;
  const int i_major = r / gs;
  tm = a.raster_n ? i_major : i_minor;
  tn = a.raster_n ? i_minor : i_major;
  // K bands: walk the tiles with the longest K range first (the host groups the raster
  // along the banded dimension), so that later, shorter tiles fill the last round
  if (a.kband == KBAND_A_LOWER) tm = a.tiles_m - 1 - tm;
  if (a.kband == KBAND_B_UPPER) tn = a.tiles_n - 1 - tn;
}

// Input modes: IN_BF16 (bf16 operands, bf16 MFMA); IN_E4M3 (E4M3 operands widened
// exactly to bf16 on their way into LDS, bf16 MFMA: full fp32 accumulation);
// IN_E4M3_NATIVE (E4M3 operands fed to the f8f6f4 MFMA as they are); IN_MX (E4M3
// operands with a UE8M0 scale per 32 along K, widened to bf16 times their scale);
// IN_MX_NATIVE (the same operands on the scaled f8f6f4 MFMA, which applies the scales);
// IN_E4M3_LDS (E4M3 operands kept as E4M3 bytes in LDS and widened exactly to bf16 in
// registers after each fragment read, bf16 MFMA: the ping-pong kernel); IN_MX_LDS (the same
// with a UE8M0 scale per 32 along K, applied by the widening: the ping-pong kernel).
enum { IN_BF16 = 0, IN_E4M3 = 1, IN_E4M3_NATIVE = 2, IN_MX = 3, IN_MX_NATIVE = 4, IN_E4M3_LDS = 5, IN_MX_LDS = 6 };

// READ_: 1 reads M/N-contiguous fragments with the transposing ds_read_b64_tr_*; 0 reads
// them one element at a time (ds_read_u16), the plain-load rung of the read ablation.
template <int BM_, int BN_, int BK_, int WM_, int WN_, int MT_, int STAGES_, int IN_, bool TA_, bool TB_,
          int READ_ = 1>
struct Cfg {
  static constexpr int BM = BM_, BN = BN_, BK = BK_, WM = WM_, WN = WN_, MT = MT_, STAGES = STAGES_;
  static constexpr int IN = IN_;
  static constexpr int READ = READ_;
  static_assert(READ == 1 || (IN != IN_E4M3_NATIVE && IN != IN_MX_NATIVE), "element-wise reads are for bf16");
  static constexpr bool TA = TA_, TB = TB_;
  static constexpr bool MXN = IN == IN_MX_NATIVE;  // block scales ride in LDS next to the tiles
  static constexpr bool FP8 = IN == IN_E4M3_NATIVE || MXN;  // fragments and MFMA are E4M3
  static constexpr int THREADS = WM * WN * 64;
  static constexpr int GES = IN == IN_BF16 ? 2 : 1;  // bytes per element in global memory
  static constexpr int ES = (FP8 || IN == IN_E4M3_LDS || IN == IN_MX_LDS) ? 1 : 2;  // bytes per element in LDS
  static constexpr int WIDEN = ES / GES;             // LDS chunks per global 16-byte chunk
  static constexpr int VEC = 16 / GES;               // elements per global 16-byte chunk
  static constexpr int WTM = BM / WM, WTN = BN / WN;
  static constexpr int KT = FP8 ? (MT == 32 ? 64 : 128) : (MT == 32 ? 16 : 32);  // K per MFMA
  static constexpr int KPL = FP8 ? 32 : 8;                                        // K per lane
  static constexpr int FM = WTM / MT, FN = WTN / MT;
  static constexpr int KSTEPS = BK / KT;
  static constexpr int ACC = MT * MT / 64;  // accumulator floats per lane per block
  // operand tiles in LDS: rows x cols elements, cols contiguous
  static constexpr bool A_KC = !TA, B_KC = TB;
  static constexpr int A_ROWS = A_KC ? BM : BK, A_COLS = A_KC ? BK : BM;
  static constexpr int B_ROWS = B_KC ? BN : BK, B_COLS = B_KC ? BK : BN;
  static constexpr int A_RB = A_COLS * ES, B_RB = B_COLS * ES;  // LDS row bytes
  static constexpr int A_CPR = A_RB / 16, B_CPR = B_RB / 16;    // LDS chunks per row
  static constexpr int A_GCPR = A_COLS * GES / 16, B_GCPR = B_COLS * GES / 16;  // global chunks per row
  static constexpr int A_BYTES = A_ROWS * A_RB, B_BYTES = B_ROWS * B_RB;
  // scaled native E4M3: one 32-bit word per tile row holding the UE8M0 bytes of the tile's
  // four 32-element K blocks, A rows then B rows
  static constexpr int A_SC_BYTES = MXN ? BM * 4 : 0, B_SC_BYTES = MXN ? BN * 4 : 0;
  static constexpr int SC_OFF = A_BYTES + B_BYTES;
  static constexpr int STAGE_BYTES = A_BYTES + B_BYTES + A_SC_BYTES + B_SC_BYTES;
  static constexpr int A_CH = A_ROWS * A_GCPR / THREADS, B_CH = B_ROWS * B_GCPR / THREADS;

  // LDS read instructions per fragment and per K step of one wave
  static constexpr int A_FRAG_READS = A_KC ? (FP8 ? 2 : 1) : (FP8 ? 4 : 2);
  static constexpr int B_FRAG_READS = B_KC ? (FP8 ? 2 : 1) : (FP8 ? 4 : 2);
  static constexpr int DS_READS_PER_STEP = FM * A_FRAG_READS + FN * B_FRAG_READS;

  static_assert(WTM % MT == 0 && WTN % MT == 0, "wave tile must hold whole MFMA blocks");
  static_assert(BK % KT == 0, "BK must hold whole MFMA K steps");
  static_assert(STAGES * STAGE_BYTES <= 160 * 1024, "LDS budget");
  static_assert(!MXN || (BK == 128 && MT == 32 && STAGES == 2 && !TA && TB),
                "scaled native E4M3: K tiles of four scale blocks, 32x32x64 MFMA, A [M][K], B [N][K]");
};

// XOR swizzle of the 16-byte chunk index of LDS row r.  The LDS serves 256 bytes per
// clock (64 banks); a 128-byte row puts even and odd rows on the two bank halves.
//  * K-contiguous tiles (row = 64, 128 or 256 bytes) are read by ds_read_b128.  On
//    gfx950 the lanes served together are 0-7 with 24-31 and 8-15 with 16-23 (and the
//    same in the upper half wave), as measured with the LDS bank-conflict counter.  A
//    32x32 fragment puts lanes 0-31 on rows r..r+31 at one chunk column; a 16x16 one
//    puts lanes 0-15 on rows r..r+15 at chunk c and lanes 16-31 on the same rows at
//    c+1.  For 128-byte bf16 rows the xor (r>>1)&7 keeps both shapes conflict-free:
//    every serving group then covers each bank slot once.
//  * M/N-contiguous bf16 tiles are read by ds_read_b64_tr_b16: each group of 16
//    lanes reads 4 consecutive rows of one 32-byte column pair; a half wave reads
//    either two neighbouring pairs of the same rows (32x32 MFMA) or one pair of rows
//    r..r+3 and r+8..r+11 (16x16).  Rows of 256 bytes or more all start on bank 0, so
//    the pair moves by ((r&3)<<1)|((r>>3)&1); 128-byte rows alternate bank halves, so
//    only the rows of one parity must separate: by 4 chunks for r&2 and 2 for r&8.
//  * M/N-contiguous E4M3 tiles are read by ds_read_b64_tr_b8: 16 lanes read 8
//    consecutive rows of one 16-byte chunk; a half wave reads two neighbouring
//    chunks of the same rows (32x32) or rows r..r+7 and r+32..r+39 (16x16).
// The result is masked to the row's chunk count, so a swizzled chunk never leaves
// its row whatever the tile width.
template <bool KC, bool FP8, int CPR, int MT = 16>
__device__ inline int swz(int r) {
  int x;
  if constexpr (KC) {
    if constexpr (CPR == 4) {
      // 64-byte rows, four to a bank line.  No xor of the row's own low bits helps every
      // MFMA shape: measured with the LDS bank-conflict counter on gfx950, (r>>1)&3 is
      // conflict-free for 16x16 fragments and (r>>2)&3 for 32x32 ones
      if constexpr (FP8)
        x = ((r >> 1) ^ (r >> 3)) & 3;
      else if constexpr (MT == 16)
        x = (r >> 1) & 3;
      else
        x = (r >> 2) & 3;
    } else if constexpr (CPR == 8) {
      if constexpr (FP8)
        x = (r & 7) ^ ((r >> 3) & 1);
      else
        x = (r >> 1) & 7;
    } else {
      x = r & 15;
    }
  } else if constexpr (!FP8) {
    if constexpr (CPR == 8)
      x = (((r >> 1) & 1) << 2) | (((r >> 3) & 1) << 1);
    else
      x = (((r & 3) << 1) | ((r >> 3) & 1)) << 1;
  } else {
    x = ((r & 7) << 1) | ((r >> 5) & 1);
  }
  return x & (CPR - 1);
}

__device__ inline void mma(f32x16& acc, const bf16x8& b, const bf16x8& a) {
  acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(b, a, acc, 0, 0, 0);
}
__device__ inline void mma(f32x4& acc, const bf16x8& b, const bf16x8& a) {
  acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(b, a, acc, 0, 0, 0);
}
__device__ inline void mma(f32x16& acc, const i32x8& b, const i32x8& a) {
  // cbsz = blgp = 0: both operands OCP E4M3; zero scale operands give the unscaled op
  acc = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(b, a, acc, 0, 0, 0, 0, 0, 0);
}
__device__ inline void mma(f32x4& acc, const i32x8& b, const i32x8& a) {
  acc = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(b, a, acc, 0, 0, 0, 0, 0, 0);
}

// Scaled f8f6f4 MFMA: the first operand (the B fragment, rows n) is scaled by byte SELB
// of sb, the second (the A fragment, rows m) by byte SELA of sa, each byte a UE8M0
// exponent (127 = 1); each lane's 32 K values form one scale block.
template <int SELB, int SELA>
__device__ inline void mma_mx(f32x16& acc, const i32x8& b, const i32x8& a, int sb, int sa) {
  acc = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(b, a, acc, 0, 0, SELB, sb, SELA, sa);
}

template <bool FP8> struct FragOf { using T = bf16x8; };
template <> struct FragOf<true> { using T = i32x8; };
template <int MT> struct AccOf { using T = f32x16; };
template <> struct AccOf<16> { using T = f32x4; };

// Fragment of one MFMA operand for lane `lane`: MT rows (M or N index, x0..x0+MT)
// times KPL consecutive K values starting at kbase + (lane / MT) * KPL.
//  K-contiguous tile (rows = x, cols = k): one or two ds_read_b128.
//  M/N-contiguous tile (rows = k, cols = x): transposing reads; within each group of
//  16 lanes, lane s supplies the address of row (s / (16/E)) and column chunk
//  (s % (16/E)) * E of an E-row by 16-column block, and lane i receives column i of
//  all E rows (E = 4 for bf16, 8 for E4M3).
template <class C, bool KC, int RB>
__device__ inline typename FragOf<C::FP8>::T load_frag(const lds_char* base, int x0, int kbase,
                                                        int lane, int sw_on) {
  using Frag = typename FragOf<C::FP8>::T;
  constexpr int CPR = RB / 16;
  Frag f;
  if constexpr (KC) {
    const int r = x0 + lane % C::MT;
    const int k = kbase + (lane / C::MT) * C::KPL;
    const int c = k * C::ES / 16;
    const int s = sw_on ? swz<true, C::FP8, CPR, C::MT>(r) : 0;
    if constexpr (!C::FP8) {
      const uint32_t off = r * RB + ((c ^ s) << 4);
      f = *LDS_PTR(bf16x8, base, off);
    } else {
      // The scaled MFMA reads the first 16 bytes of every lane as scale block 0 of the
      // step (its scale from lanes 0-31) and the last 16 as block 1 (lanes 32-63), as
      // measured on gfx950; so with scales lane half h holds the 16-byte K chunks h
      // and h + 2 of the step, and 32-wide block b is chunks 2b and 2b + 1.  Without
      // scales only the K order of A and B must agree: consecutive chunks.
      const int c0 = C::MXN ? kbase * C::ES / 16 + lane / C::MT : c;
      const int c1 = C::MXN ? c0 + 2 : c + 1;
      const uint32_t off0 = r * RB + ((c0 ^ s) << 4);
      const uint32_t off1 = r * RB + ((c1 ^ s) << 4);
      i32x4 lo = *LDS_PTR(i32x4, base, off0);
      i32x4 hi = *LDS_PTR(i32x4, base, off1);
      f = (i32x8){lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
    }
  } else if constexpr (C::READ == 0) {
    // one ds_read_u16 per element: lane holds column x (its M or N index) of rows
    // k .. k+7 (its K values)
    const int x = x0 + lane % C::MT;
    const int k0 = kbase + (lane / C::MT) * C::KPL;
    const int xb = x * C::ES;
    typedef unsigned short u16x8 __attribute__((ext_vector_type(8)));
    u16x8 all;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int k = k0 + e;
      const int sw = sw_on ? swz<false, false, CPR, C::MT>(k) : 0;
      const uint32_t off = k * RB + ((((xb >> 4) ^ sw) << 4) | (xb & 15));
      all[e] = *LDS_PTR(uint16_t, base, off);
    }
    f = __builtin_bit_cast(bf16x8, all);
  } else {
    constexpr int E = C::FP8 ? 8 : 4;
    constexpr int LPR = 16 / E;  // lanes per row inside a 16-lane group
    const int g = lane >> 4, s = lane & 15;
    const int coloff = (C::MT == 32) ? 16 * (g & 1) : 0;
    const int kgrp = (C::MT == 32) ? (g >> 1) : g;
    const int x = x0 + coloff + (s % LPR) * E;  // first column of this lane's 8 bytes
    const int xb = x * C::ES;                   // byte column
    if constexpr (!C::FP8) {
      u16x4 part[2];
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int k = kbase + kgrp * C::KPL + h * E + s / LPR;
        const int sw = sw_on ? swz<false, false, CPR, C::MT>(k) : 0;
        const uint32_t off = k * RB + ((((xb >> 4) ^ sw) << 4) | (xb & 15));
        s16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16(LDS_PTR(s16x4, base, off));
        part[h] = __builtin_bit_cast(u16x4, v);
      }
      u16x4 lo = part[0], hi = part[1];
      typedef unsigned short u16x8 __attribute__((ext_vector_type(8)));
      u16x8 all = (u16x8){lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
      f = __builtin_bit_cast(bf16x8, all);
    } else {
      i32x2 part[4];
#pragma unroll
      for (int h = 0; h < 4; ++h) {
        const int k = kbase + kgrp * C::KPL + h * E + s / LPR;
        const int sw = sw_on ? swz<false, true, CPR, C::MT>(k) : 0;
        const uint32_t off = k * RB + ((((xb >> 4) ^ sw) << 4) | (xb & 15));
        part[h] = __builtin_amdgcn_ds_read_tr8_b64_v2i32(LDS_PTR(i32x2, base, off));
      }
      f = (i32x8){part[0][0], part[0][1], part[1][0], part[1][1],
                  part[2][0], part[2][1], part[3][0], part[3][1]};
    }
  }
  return f;
}

__device__ inline uint16_t f32_to_bf16_bits(float v) {
  return __builtin_bit_cast(uint16_t, static_cast<__bf16>(v));
}
__device__ inline float bf16_bits_to_f32(uint16_t b) {
  return __builtin_bit_cast(float, (uint32_t)b << 16);
}

// Compile-time loop: f(integral_constant<int, 0>) ... f(integral_constant<int, N-1>).
template <int N, int I = 0, class F>
__device__ __forceinline__ void static_for(F&& f) {
  if constexpr (I < N) {
    f(std::integral_constant<int, I>{});
    static_for<N, I + 1>(f);
  }
}

// Instruction-scheduling hints for one K step: NMF MFMAs, each followed by its even
// share of NDS LDS reads, NVM global loads and NDW LDS writes (the groups are
// matched in order by the scheduler within the current basic block).
template <int NMF, int NDS, int NVM, int NDW, int I = 0>
__device__ __forceinline__ void interleave() {
  if constexpr (I < NMF) {
    constexpr int ds = NDS * (I + 1) / NMF - NDS * I / NMF;
    constexpr int vm = NVM * (I + 1) / NMF - NVM * I / NMF;
    constexpr int dw = NDW * (I + 1) / NMF - NDW * I / NMF;
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // MFMA
    if constexpr (ds > 0) __builtin_amdgcn_sched_group_barrier(0x100, ds, 0);  // DS read
    if constexpr (vm > 0) __builtin_amdgcn_sched_group_barrier(0x020, vm, 0);  // VMEM read
    if constexpr (dw > 0) __builtin_amdgcn_sched_group_barrier(0x200, dw, 0);  // DS write
    interleave<NMF, NDS, NVM, NDW, I + 1>();
  }
}

// 16 E4M3 values -> 16 bf16 values (exact: every E4M3 number, subnormals included, is
// a bf16 number) with the gfx950 packed conversion at unit scale.
__device__ inline void widen_e4m3(const i32x4& v, i32x4& lo, i32x4& hi, float scale = 1.0f) {
  int w[8];
#pragma unroll
  for (int d = 0; d < 4; ++d) {
    w[2 * d] = __builtin_bit_cast(int, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(v[d], scale, false));
    w[2 * d + 1] = __builtin_bit_cast(int, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(v[d], scale, true));
  }
  lo = (i32x4){w[0], w[1], w[2], w[3]};
  hi = (i32x4){w[4], w[5], w[6], w[7]};
}

// Stores one global chunk into LDS at byte offset `off` (its first LDS chunk).  A
// widened chunk fills two logically adjacent LDS chunks; under the XOR swizzle their
// physical positions differ only in bit 4 of the offset.
// UE8M0 byte -> the fp32 power of two it stands for (255 is NaN; 0 is 2^-127).
__device__ inline float ue8m0_value(uint32_t e) {
  return e == 255u ? __builtin_nanf("") : __builtin_bit_cast(float, e == 0u ? 0x00400000u : e << 23);
}

template <class C>
__device__ inline void put_chunk(lds_char* sbase, uint32_t off, const i32x4& v, float scale = 1.0f) {
  if constexpr (C::WIDEN == 1) {
    *LDS_PTR(i32x4, sbase, off) = v;
  } else {
    i32x4 lo, hi;
    widen_e4m3(v, lo, hi, scale);
    *LDS_PTR(i32x4, sbase, off) = lo;
    *LDS_PTR(i32x4, sbase, off ^ 16u) = hi;
  }
}

// Epilogue of one group of four accumulator values: acc float4 number p of this lane
// (block (i, j), quarter q) holds C[m][n .. n+3]; C <- alpha*v + beta*C_old, rounded
// to C's type (bf16 and E4M3 to nearest even, E4M3 saturating at +-448).  store_tile
// applies it to every group.
template <class C>
__device__ __forceinline__ void store_group_tri(const GemmArgs& a, f32x4 v, int p, int row0, int col0, int lane) {
  const int q = p % (C::ACC / 4), j = (p / (C::ACC / 4)) % C::FN, i = p / (C::ACC / 4) / C::FN;
  const int m = row0 + i * C::MT + lane % C::MT;
  const int n = col0 + j * C::MT + (C::MT == 32 ? 8 * q + 4 * (lane / 32) : 4 * (lane / 16));
  if (m >= a.M) return;
  // elements [e0, e1) of the four columns are written: the last columns stop at N, and a
  // triangle keeps n + e <= m (lower) or n + e >= m (upper)
  int e0 = 0, e1 = a.N - n < 4 ? a.N - n : 4;
  if (a.tri == TRI_LOWER) e1 = m - n + 1 < e1 ? m - n + 1 : e1;
  if (a.tri == TRI_UPPER) e0 = m - n > 0 ? m - n : 0;
  if (e1 <= e0) return;
  const float alpha = a.alpha, beta = a.beta;
  float w[4];
#pragma unroll
  for (int e = 0; e < 4; ++e) w[e] = alpha * v[e];
  const int64_t base = (int64_t)m * a.ldc + n;
  if (e0 == 0 && e1 == 4) {
    if (a.c_kind == C_F32) {
      float* cp = (float*)a.C + base;
      if (beta != 0.f) {
        f32x4 old = *(const f32x4*)cp;
#pragma unroll
        for (int e = 0; e < 4; ++e) w[e] += beta * old[e];
      }
      *(f32x4*)cp = (f32x4){w[0], w[1], w[2], w[3]};
    } else if (a.c_kind == C_E4M3) {  // four codes in one 32-bit word (n is a multiple of 4)
      uint32_t* cp = (uint32_t*)((uint8_t*)a.C + base);
      if (beta != 0.f) {
        const uint32_t old = *cp;
        w[0] += beta * __builtin_amdgcn_cvt_f32_fp8((int)old, 0);
        w[1] += beta * __builtin_amdgcn_cvt_f32_fp8((int)old, 1);
        w[2] += beta * __builtin_amdgcn_cvt_f32_fp8((int)old, 2);
        w[3] += beta * __builtin_amdgcn_cvt_f32_fp8((int)old, 3);
      }
      *cp = e4m3x4_from_f32(w[0], w[1], w[2], w[3]);
    } else {
      uint16_t* cp = (uint16_t*)a.C + base;
      if (beta != 0.f) {
        u16x4 old = *(const u16x4*)cp;
#pragma unroll
        for (int e = 0; e < 4; ++e) w[e] += beta * bf16_bits_to_f32(old[e]);
      }
      *(u16x4*)cp = (u16x4){f32_to_bf16_bits(w[0]), f32_to_bf16_bits(w[1]), f32_to_bf16_bits(w[2]),
                            f32_to_bf16_bits(w[3])};
    }
  } else {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      if (e < e0 || e >= e1) continue;
      if (a.c_kind == C_F32) {
        float* cp = (float*)a.C + base + e;
        *cp = w[e] + (beta != 0.f ? beta * *cp : 0.f);
      } else if (a.c_kind == C_E4M3) {
        uint8_t* cp = (uint8_t*)a.C + base + e;
        *cp = (uint8_t)e4m3x4_from_f32(w[e] + (beta != 0.f ? beta * __builtin_amdgcn_cvt_f32_fp8(*cp, 0) : 0.f),
                                       0.f, 0.f, 0.f);
      } else {
        uint16_t* cp = (uint16_t*)a.C + base + e;
        *cp = f32_to_bf16_bits(w[e] + (beta != 0.f ? beta * bf16_bits_to_f32(*cp) : 0.f));
      }
    }
  }
}

template <class C>
__device__ __forceinline__ void store_group(const GemmArgs& a, f32x4 v, int p, int row0, int col0, int lane) {
  // a triangle of C takes its own path, so that the common one keeps its register budget;
  // only bf16 square tiles serve triangles (the host picks no other), the rest compile it out
  if constexpr (C::IN == IN_BF16 && C::BM == C::BN)
    if (a.tri != TRI_NONE) return store_group_tri<C>(a, v, p, row0, col0, lane);
  const int q = p % (C::ACC / 4), j = (p / (C::ACC / 4)) % C::FN, i = p / (C::ACC / 4) / C::FN;
  const int m = row0 + i * C::MT + lane % C::MT;
  const int n = col0 + j * C::MT + (C::MT == 32 ? 8 * q + 4 * (lane / 32) : 4 * (lane / 16));
  if (m >= a.M) return;
  const float alpha = a.alpha, beta = a.beta;
  float w[4];
#pragma unroll
  for (int e = 0; e < 4; ++e) w[e] = alpha * v[e];
  const int64_t base = (int64_t)m * a.ldc + n;
  if (n + 3 < a.N) {
    if (a.c_kind == C_F32) {
      float* cp = (float*)a.C + base;
      if (beta != 0.f) {
        f32x4 old = *(const f32x4*)cp;
#pragma unroll
        for (int e = 0; e < 4; ++e) w[e] += beta * old[e];
      }
      *(f32x4*)cp = (f32x4){w[0], w[1], w[2], w[3]};
    } else if (a.c_kind == C_E4M3) {  // four codes in one 32-bit word (n is a multiple of 4)
      uint32_t* cp = (uint32_t*)((uint8_t*)a.C + base);
      if (beta != 0.f) {
        const uint32_t old = *cp;
        w[0] += beta * __builtin_amdgcn_cvt_f32_fp8((int)old, 0);
        w[1] += beta * __builtin_amdgcn_cvt_f32_fp8((int)old, 1);
        w[2] += beta * __builtin_amdgcn_cvt_f32_fp8((int)old, 2);
        w[3] += beta * __builtin_amdgcn_cvt_f32_fp8((int)old, 3);
      }
      *cp = e4m3x4_from_f32(w[0], w[1], w[2], w[3]);
    } else {
      uint16_t* cp = (uint16_t*)a.C + base;
      if (beta != 0.f) {
        u16x4 old = *(const u16x4*)cp;
#pragma unroll
        for (int e = 0; e < 4; ++e) w[e] += beta * bf16_bits_to_f32(old[e]);
      }
      *(u16x4*)cp = (u16x4){f32_to_bf16_bits(w[0]), f32_to_bf16_bits(w[1]), f32_to_bf16_bits(w[2]),
                            f32_to_bf16_bits(w[3])};
    }
  } else {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      if (n + e >= a.N) break;
      if (a.c_kind == C_F32) {
        float* cp = (float*)a.C + base + e;
        *cp = w[e] + (beta != 0.f ? beta * *cp : 0.f);
      } else if (a.c_kind == C_E4M3) {
        uint8_t* cp = (uint8_t*)a.C + base + e;
        *cp = (uint8_t)e4m3x4_from_f32(w[e] + (beta != 0.f ? beta * __builtin_amdgcn_cvt_f32_fp8(*cp, 0) : 0.f),
                                       0.f, 0.f, 0.f);
      } else {
        uint16_t* cp = (uint16_t*)a.C + base + e;
        *cp = f32_to_bf16_bits(w[e] + (beta != 0.f ? beta * bf16_bits_to_f32(*cp) : 0.f));
      }
    }
  }
}

// alpha*acc + beta*C_old -> C for one wave's accumulator tile whose first row is
// row0 and first column col0.  The MFMA ran with the B fragment as first operand, so
// a lane holds, for row row0 + i*MT + lane%MT, groups of four consecutive columns.
template <class C>
__device__ __forceinline__ void store_tile(const GemmArgs& a, const typename AccOf<C::MT>::T (&acc)[C::FM][C::FN],
                                  int row0, int col0, int lane) {
  // compile-time indices (not a loop left to the unroller), so acc stays in registers
  static_for<C::FM * C::FN * (C::ACC / 4)>([&](auto pc) {
    constexpr int p = decltype(pc)::value;
    constexpr int q = p % (C::ACC / 4), j = (p / (C::ACC / 4)) % C::FN, i = p / (C::ACC / 4) / C::FN;
    store_group<C>(a, (f32x4){acc[i][j][4 * q], acc[i][j][4 * q + 1], acc[i][j][4 * q + 2], acc[i][j][4 * q + 3]},
                   p, row0, col0, lane);
  });
}

// Split-K partial tiles.  A partial is kept in register order: float4 number p of
// thread t sits at p * THREADS + t, so both the write and the read-back are fully
// coalesced and need no index math beyond the thread id.
template <class C>
__device__ inline void store_partial(float* blk, const typename AccOf<C::MT>::T (&acc)[C::FM][C::FN], int t) {
  f32x4* dst = (f32x4*)blk;
#pragma unroll
  for (int i = 0; i < C::FM; ++i)
#pragma unroll
    for (int j = 0; j < C::FN; ++j)
#pragma unroll
      for (int q = 0; q < C::ACC / 4; ++q)
        dst[((i * C::FN + j) * (C::ACC / 4) + q) * C::THREADS + t] =
            (f32x4){acc[i][j][4 * q], acc[i][j][4 * q + 1], acc[i][j][4 * q + 2], acc[i][j][4 * q + 3]};
}

}  // namespace
}  // namespace dbgemm
