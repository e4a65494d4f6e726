// Ping-pong MFMA GEMM kernel for gfx950 (large tiles, bf16 operands).
//
// Same operation, LDS layout (XOR-swizzled 16-byte chunks), fragment reads, MFMA and
// epilogue as the other MFMA kernels (mfma_common.h), and the same direct-to-LDS
// operand staging as the ring kernel; what differs is how the eight waves of a
// workgroup share each SIMD's matrix core.
//
// A CU has four SIMDs and a 256x256 workgroup tile keeps two waves on each.  In the
// ring kernel both waves of a SIMD run the same instruction mix at the same time:
// MFMAs with their share of fragment reads between them, and all eight waves meet at
// one barrier per K tile, where the matrix cores drain.  Here the waves form two
// groups of four, one wave of each group per SIMD, and the groups take turns:
//
//   * while group 0 runs one K tile's MFMAs (one uninterrupted cluster of 64
//     16x16x32 MFMAs per wave, at raised wave priority) group 1 reads its fragments
//     of the same K tile from LDS, and the other way round in the next phase;
//   * every phase ends at a workgroup barrier, and a group that arrives from its
//     memory phase has its fragments in registers, so the matrix core of each SIMD
//     passes from one wave's cluster straight to the other's;
//   * the operand tiles sit in two LDS slots.  K tile t + 2 is loaded into the slot of
//     tile t as soon as both groups have read tile t (the barrier after group 1's read
//     of it): group 0 issues its share of the copies in its memory phase, group 1
//     between its MFMAs; every wave waits for its own copies (vmcnt) before the
//     barrier after which they are read, two phases after they were issued.
//
// Barrier schedule (B_i is the i-th barrier of the main loop; C(t) = MFMAs of tile t,
// M(t) = fragment reads of tile t):
//
//   group 0:  M(0) | C(0) B1 M(1) B2 | C(1) B3 M(2) B4 | ... | C(n-1) B(2n-1)
//   group 1:       | M(0) B1 C(0) B2 | M(1) B3 C(1) B4 | ... | M(n-1) B(2n-1) C(n-1)
//
// Both groups execute the same number of barriers.  This is the gfx950 form of the
// pages' producer/consumer split of a CTA ("cp.async / ldmatrix ablation", sections 0.2
// and 1: asynchronous copies running ahead of the matrix instructions, per-stage
// completion tracking), with the roles taken by two groups of waves that alternate
// rather than by dedicated producer warps.
//
// E4M3 operands stay E4M3 bytes in LDS and are widened exactly to bf16 in registers after
// each fragment read.  Block-scaled E4M3 (one UE8M0 byte per row and 32 elements of K)
// adds a third stream: the scale bytes are copied to LDS ahead of their operands, each
// lane reads the scale words of its fragments' rows once per K tile, and each fragment is
// widened with its block's scale code placed in the exponent field of the conversion's
// scale operand.
#include "mfma_common.h"

namespace dbgemm {
namespace {

typedef unsigned short u16x8 __attribute__((ext_vector_type(8)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));

// 64 lanes x 4 bytes from buffer `rsrc` at per-lane byte offset `voff` into LDS bytes
// [lds_base, lds_base + 256) (lane i -> lds_base + 4*i); an offset past the buffer's size
// reads zeros.  M0 carries the LDS address: it is saved and restored inside the statement
// (the compiler reserves M0 and does not honour it as a clobber), and one wait state
// separates its write from the load that reads it.  The compiler neither sees nor waits
// for these loads or the 16-byte copies below; every wait on them is explicit.
__device__ __forceinline__ void pp_load_to_lds_dword(uint32_t lds_base, uint32_t voff, __amdgpu_buffer_rsrc_t rsrc) {
  uint32_t saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %1\n\t"
      "s_nop 0\n\t"
      "buffer_load_dword %2, %3, 0 offen lds\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(saved)
      : "s"(lds_base), "v"(voff), "s"(rsrc)
      : "memory");
}

// N copies of 1 KiB from one buffer into the LDS blocks at l, l + 1024, ... in one
// statement (M0 saved once, written before each load, one wait state after each write).
// TAIL only changes the statement's text (a ragged-K tile), so that the compiler keeps the
// full-tile and the ragged-tile forms apart instead of merging them with per-copy selects.
template <int N, bool TAIL>
__device__ __forceinline__ void pp_copies(uint32_t l, const uint32_t (&o)[N], __amdgpu_buffer_rsrc_t r) {
  uint32_t saved;
  if constexpr (N == 1) {
    asm volatile(
        "s_mov_b32 %0, m0\n\ts_mov_b32 m0, %1\n\ts_nop 0\n\tbuffer_load_dwordx4 %2, %3, 0 offen lds\n\t"
        "s_mov_b32 m0, %0 ; %4"
        : "=&s"(saved)
        : "s"(l), "v"(o[0]), "s"(r), "i"(TAIL ? 1 : 0)
        : "memory");
  } else if constexpr (N == 2) {
    asm volatile(
        "s_mov_b32 %0, m0\n\t"
        "s_mov_b32 m0, %1\n\ts_nop 0\n\tbuffer_load_dwordx4 %2, %4, 0 offen lds\n\t"
        "s_add_u32 m0, m0, 0x400\n\ts_nop 0\n\tbuffer_load_dwordx4 %3, %4, 0 offen lds\n\t"
        "s_mov_b32 m0, %0 ; %5"
        : "=&s"(saved)
        : "s"(l), "v"(o[0]), "v"(o[1]), "s"(r), "i"(TAIL ? 1 : 0)
        : "memory");
  } else if constexpr (N == 3) {
    asm volatile(
        "s_mov_b32 %0, m0\n\t"
        "s_mov_b32 m0, %1\n\ts_nop 0\n\tbuffer_load_dwordx4 %2, %5, 0 offen lds\n\t"
        "s_add_u32 m0, m0, 0x400\n\ts_nop 0\n\tbuffer_load_dwordx4 %3, %5, 0 offen lds\n\t"
        "s_add_u32 m0, m0, 0x400\n\ts_nop 0\n\tbuffer_load_dwordx4 %4, %5, 0 offen lds\n\t"
        "s_mov_b32 m0, %0 ; %6"
        : "=&s"(saved)
        : "s"(l), "v"(o[0]), "v"(o[1]), "v"(o[2]), "s"(r), "i"(TAIL ? 1 : 0)
        : "memory");
  } else {
    static_assert(N == 4, "1 to 4 copies per statement");
    asm volatile(
        "s_mov_b32 %0, m0\n\t"
        "s_mov_b32 m0, %1\n\ts_nop 0\n\tbuffer_load_dwordx4 %2, %6, 0 offen lds\n\t"
        "s_add_u32 m0, m0, 0x400\n\ts_nop 0\n\tbuffer_load_dwordx4 %3, %6, 0 offen lds\n\t"
        "s_add_u32 m0, m0, 0x400\n\ts_nop 0\n\tbuffer_load_dwordx4 %4, %6, 0 offen lds\n\t"
        "s_add_u32 m0, m0, 0x400\n\ts_nop 0\n\tbuffer_load_dwordx4 %5, %6, 0 offen lds\n\t"
        "s_mov_b32 m0, %0 ; %7"
        : "=&s"(saved)
        : "s"(l), "v"(o[0]), "v"(o[1]), "v"(o[2]), "v"(o[3]), "s"(r), "i"(TAIL ? 1 : 0)
        : "memory");
  }
}

// Waits for this wave's LDS reads only (its copies stay in flight), then the barrier.
__device__ __forceinline__ void pp_wait_lds_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

template <int N>
__device__ __forceinline__ void pp_wait_vm_barrier() {
  asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)\n\ts_barrier" : : "n"(N) : "memory");
}

// E4M3 bytes in LDS, widened to bf16 after each fragment read (with or without block scales)
template <class C>
constexpr bool pp_e8 = C::IN == IN_E4M3_LDS || C::IN == IN_MX_LDS;

template <class C>
struct PingPong {
  static_assert(C::THREADS == 512 && C::WM == 2 && C::WN == 4, "two groups of four waves");
  static_assert(C::STAGES >= 2 && C::STAGES <= 5, "two to five LDS slots");
  static_assert((C::IN == IN_BF16 || pp_e8<C>) && C::GES == C::ES,
                "bf16 or E4M3 operands, LDS holds the global format");
  static_assert(!pp_e8<C> || C::MT == 16, "E4M3 tiles feed the 16x16x32 fragment map");
  static constexpr bool E8 = pp_e8<C>;
  // block scales: per K tile, one dword per operand row (its four UE8M0 bytes, one per K
  // step) copied to LDS
  static constexpr bool MXS = C::IN == IN_MX_LDS;
  static constexpr int NW = 8, S = C::STAGES;
  static_assert(!MXS || (C::A_KC && C::B_KC && C::BK == 128 && C::KT == 32 && C::BM == 256 && C::BN == 256 && S == 2),
                "block-scaled tiles: A [M][K] and B [N][K], one 32-element scale block per K step, 512 rows "
                "(one scale dword per thread), two slots");
  static_assert(C::A_BYTES % (1024 * NW) == 0 && C::B_BYTES % (1024 * NW) == 0,
                "each wave copies whole 1 KiB blocks of both tiles");
  static constexpr int A_IPW = C::A_BYTES / 1024 / NW;  // copy instructions per wave per K tile
  static constexpr int B_IPW = C::B_BYTES / 1024 / NW;
  static constexpr int DATA_IPW = A_IPW + B_IPW;
  // the scale dwords of a K tile (4-byte scale rows): 256 bytes per wave; 16-byte rows take
  // one 1 KiB copy per wave with every fourth K tile instead
  static constexpr int SC_IPW = MXS ? 1 : 0;
  static constexpr int IPW = DATA_IPW + SC_IPW;
  static_assert((S - 1) * IPW <= 63, "vmcnt range");
  static_assert((C::A_KC || (C::A_CPR & (C::A_CPR - 1)) == 0) && (C::B_KC || (C::B_CPR & (C::B_CPR - 1)) == 0),
                "M/N-contiguous rows of a power of two of chunks (the XOR swizzle stays in the row)");
  static constexpr int NMF = C::FM * C::FN * C::KSTEPS;  // MFMAs per wave per K tile
  static_assert(NMF >= IPW, "one copy per MFMA at most");
  // LDS: the A tiles of the S slots, then the B tiles; with block scales, 32 KiB of scale
  // bytes.  Scale position p holds one row, and a K tile's scale words are read from
  // [p * 4, + 4) of a 2 KiB table.  Scale rows aligned to 16 bytes are copied 16 bytes
  // (four K tiles) at a time, with the copies of the K tile two before the first of the
  // four, into two 8 KiB slots (position p at p * 16), and each thread later moves its
  // position's four words into four tables (two sets of four, after the copy area).
  // Otherwise a K tile's 4 bytes ride with the copies of the tile before it, straight into
  // one of four tables in the copy area, the bytes of K tile kt in table kt % 4.  Positions
  // are ordered so that the rows of a lane's fragments (16 apart) sit at consecutive
  // positions, four at a time, and the sixteen lanes of a row of a wave read consecutive
  // runs (no bank conflicts): A rows wm * 128 + 16 i + l at p = wm * 128 + (i / 4) * 64 +
  // 4 l + i % 4, B rows wn * 64 + 16 j + l at p = 256 + wn * 64 + 4 l + j.
  static constexpr int A_OFF = 0, B_OFF = S * C::A_BYTES;
  static constexpr int SC_TABLE = 4 * (C::BM + C::BN);              // one K tile's words
  static constexpr int SCB_REGION = MXS ? 2 * 4 * SC_TABLE : 0;       // the copy area
  static constexpr int SCB_OFF = S * (C::A_BYTES + C::B_BYTES);
  static constexpr int SCR_OFF = SCB_OFF + SCB_REGION;               // the tables of 16-byte rows
  static constexpr int LDS_BYTES = SCR_OFF + SCB_REGION;
  static_assert(LDS_BYTES <= 160 * 1024, "LDS of one CU");
  // LDS reads per fragment (transposing bf16 reads take two 8-byte reads per fragment; an
  // E4M3 fragment is 8 bytes, one read either way)
  static constexpr int A_RD = (C::A_KC || E8) ? 1 : 2, B_RD = (C::B_KC || E8) ? 1 : 2;
};

// XOR swizzle of the 16-byte chunk index of LDS row r.  bf16 tiles use the shared layout
// (swz).  E4M3 tiles are read 8 bytes per lane; measured conflict-free with the LDS bank
// counter on gfx950: K-contiguous rows (ds_read_b64) xor by (r >> 2) for 64-byte rows and
// (r >> 1) for 128-byte rows, M/N-contiguous rows (ds_read_b64_tr_b8) by the row itself.
template <class C, bool KC, int CPR>
__device__ __forceinline__ int pp_swz(int r) {
  if constexpr (pp_e8<C>) {
    if constexpr (KC)
      return (r >> (CPR == 4 ? 2 : 1)) & (CPR - 1);
    else
      return r & (CPR - 1);
  } else {
    return swz<KC, false, CPR, C::MT>(r);
  }
}

// Byte offset, inside one operand tile in LDS, of this lane's part of fragment read h of
// the MT-row block starting at x0 (M or N index) and K step starting at kbase: the
// addresses that load_frag computes for bf16 tiles in the XOR-swizzled layout, and the
// 8-byte reads of E4M3 tiles (lane l: row or column l % 16, K values 8 (l / 16) .. + 7).
template <class C, bool KC, int RB>
__device__ __forceinline__ uint32_t pp_frag_off(int x0, int kbase, int lane, int h) {
  constexpr int CPR = RB / 16;
  if constexpr (pp_e8<C>) {
    if constexpr (KC) {
      const int r = x0 + lane % 16;
      const int kb = kbase + (lane / 16) * 8;  // bytes = elements
      return (uint32_t)(r * RB + ((((kb >> 4) ^ pp_swz<C, true, CPR>(r)) << 4) | (kb & 15)));
    } else {
      // ds_read_b64_tr_b8: within each group of 16 lanes, lane t gives row t / 2 of eight and
      // the 8 bytes at column (t % 2) * 8 of a 16-column block; lane i receives column i
      const int g = lane >> 4, t = lane & 15;
      const int k = kbase + g * 8 + t / 2;
      const int xb = x0 + (t % 2) * 8;
      return (uint32_t)(k * RB + ((((xb >> 4) ^ pp_swz<C, false, CPR>(k)) << 4) | (xb & 15)));
    }
  } else if constexpr (KC) {
    const int r = x0 + lane % C::MT;
    const int c = (kbase + (lane / C::MT) * C::KPL) * 2 / 16;
    return (uint32_t)(r * RB + ((c ^ swz<true, false, CPR, C::MT>(r)) << 4));
  } else {
    const int g = lane >> 4, s = lane & 15;
    const int coloff = (C::MT == 32) ? 16 * (g & 1) : 0;
    const int kgrp = (C::MT == 32) ? (g >> 1) : g;
    const int xb = (x0 + coloff + (s % 4) * 4) * 2;
    const int k = kbase + kgrp * C::KPL + h * 4 + s / 4;
    return (uint32_t)(k * RB + ((((xb >> 4) ^ swz<false, false, CPR, C::MT>(k)) << 4) | (xb & 15)));
  }
}

// 8 E4M3 values (bytes in K order) -> 8 bf16 values times `scale`, with the gfx950 packed
// conversion: exact at unit scale (every E4M3 number, subnormals included, is a bf16
// number).  The conversion takes its scale as a UE8M0 code: only the exponent field (bits
// 23-30) of the operand counts, sign and mantissa are ignored, code 0 scales by 2^-127 and
// code 255 gives NaN (measured on gfx950, and pinned by the block-scaled GPU tests, which
// compare with a kernel that passes 2^(e - 127) as a float).
__device__ __forceinline__ bf16x8 pp_widen8(i32x2 v, float scale = 1.0f) {
  const int w0 = __builtin_bit_cast(int, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(v[0], scale, false));
  const int w1 = __builtin_bit_cast(int, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(v[0], scale, true));
  const int w2 = __builtin_bit_cast(int, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(v[1], scale, false));
  const int w3 = __builtin_bit_cast(int, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(v[1], scale, true));
  return __builtin_bit_cast(bf16x8, (i32x4){w0, w1, w2, w3});
}

// Stream-K: bound on the tries of an owner's wait for one partial (each try sleeps a few
// hundred cycles after a device-scope load, about a microsecond, so the bound is a few
// seconds).  Every workgroup the owner waits for is resident or next in line once the
// grid's data-parallel part has run, so a wait only runs out if the device is held by
// other work for that long; then the tile gets NaN instead of a hang.
constexpr int kStreamKSpins = 1 << 22;

// Stream-K partial tiles in register order (as store_partial): float4 number p of thread
// t sits at byte (p * THREADS + t) * 16 of the slot.  Buffer instructions take the
// thread's offset in one VGPR and each p's offset as a scalar, so no per-p address is
// held in registers.
template <class C>
__device__ __forceinline__ void pp_store_partial(float* slot, const typename AccOf<C::MT>::T (&acc)[C::FM][C::FN],
                                                 uint32_t voff) {
  const __amdgpu_buffer_rsrc_t r = make_rsrc(slot, C::BM * C::BN * 4);
  static_for<C::FM * C::FN * (C::ACC / 4)>([&](auto pc) {
    constexpr int p = decltype(pc)::value;
    constexpr int q = p % (C::ACC / 4), j = (p / (C::ACC / 4)) % C::FN, i = p / (C::ACC / 4) / C::FN;
    const f32x4 v = {acc[i][j][4 * q], acc[i][j][4 * q + 1], acc[i][j][4 * q + 2], acc[i][j][4 * q + 3]};
    __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, v), r, voff, p * C::THREADS * 16, 0);
  });
}

// Adds such a partial into acc, half of the fragment rows at a time (the scheduling
// barrier keeps the second half's loads from being hoisted above the first half's
// additions, which bounds the registers in flight).
template <class C>
__device__ __forceinline__ void pp_add_partial(const float* slot, typename AccOf<C::MT>::T (&acc)[C::FM][C::FN],
                                               uint32_t voff) {
  const __amdgpu_buffer_rsrc_t r = make_rsrc(slot, C::BM * C::BN * 4);
  constexpr int NP = C::FM * C::FN * (C::ACC / 4);
  static_assert(NP % 2 == 0, "two halves");
  static_for<2>([&](auto hc) {
    constexpr int h = decltype(hc)::value;
    static_for<NP / 2>([&](auto pc) {
      constexpr int p = h * (NP / 2) + decltype(pc)::value;
      constexpr int q = p % (C::ACC / 4), j = (p / (C::ACC / 4)) % C::FN, i = p / (C::ACC / 4) / C::FN;
      const f32x4 v =
          __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(r, voff, p * C::THREADS * 16, 0));
#pragma unroll
      for (int e = 0; e < 4; ++e) acc[i][j][4 * q + e] += v[e];
    });
    __builtin_amdgcn_sched_barrier(0);
  });
}

// Epilogue through LDS.  Written straight from the accumulators, a 16x16 fragment store
// puts 16 rows x 32 bytes in one instruction; here the tile goes out in whole rows instead.
// Two passes, one per row of waves (wave group g holds tile rows [g*WTM, (g+1)*WTM)): the
// group writes alpha*acc as fp32 into a row-major image of its rows in LDS (16-byte chunks
// XOR-swizzled by row, so that the sixteen rows of a fragment store and the two rows of a
// wave's chunk reads spread over all banks), then all threads take 8 consecutive columns
// each, 32 threads per 256-column row, add beta*C_old, round to C's type once and store
// 16 bytes (bf16), 32 (fp32) or 8 (E4M3) per thread.  The same arithmetic as store_group.
// The whole-vector stores are non-temporal: C is not read again by the kernel, and
// streaming it past the caches cut 4096^2 at K = 256 from 18.0 to 16.0 us.
template <class C>
__device__ __forceinline__ void pp_store_tile_lds(const GemmArgs& a, const typename AccOf<C::MT>::T (&acc)[C::FM][C::FN],
                                                  int m0, int n0, int grp, int xb0, int lane, int t, uint32_t lds0) {
  static_assert(C::MT == 16 && C::BN == 256 && C::THREADS == 512, "16x16 fragments, 256 columns, 8 waves");
  static_assert(C::WTM * C::BN * 4 <= PingPong<C>::LDS_BYTES, "one row of waves' fp32 image fits the LDS");
  constexpr int RB = C::BN * 4;  // bytes per staged row
  const float alpha = a.alpha, beta = a.beta;
  // every wave's copies have landed (the last ones, past K, write zeros into LDS)
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  if (a.c_kind == C_BF16 && beta == 0.f) {
    // beta = 0 into bf16: both groups stage alpha*acc already rounded to bf16 (the rounding
    // the store makes), 16-byte chunks XOR-swizzled by row as above, then one pass of row
    // stores
    constexpr int RB2 = C::BN * 2;
    static_assert(C::BM * RB2 <= PingPong<C>::LDS_BYTES, "the tile's bf16 image fits the LDS");
    __syncthreads();  // the LDS is free: the K loop's reads are done
    static_for<C::FM * C::FN>([&](auto pc) {
      constexpr int p = decltype(pc)::value;
      constexpr int i = p / C::FN, j = p % C::FN;
      const int r = grp * C::WTM + i * 16 + lane % 16;
      const int c = xb0 + j * 16 + 4 * (lane / 16);  // a multiple of 4: half a chunk
      const int chunk = (c >> 3) ^ (r & 15);
      const u16x4 v = {f32_to_bf16_bits(alpha * acc[i][j][0]), f32_to_bf16_bits(alpha * acc[i][j][1]),
                       f32_to_bf16_bits(alpha * acc[i][j][2]), f32_to_bf16_bits(alpha * acc[i][j][3])};
      *(__attribute__((address_space(3))) u16x4*)(uintptr_t)(lds0 + (uint32_t)(r * RB2 + chunk * 16 + (c & 7) * 2)) = v;
    });
    __syncthreads();
    constexpr int RPS = C::THREADS / 32;  // rows per step: 32 threads of 8 columns per row
#pragma unroll 2
    for (int s = 0; s < C::BM / RPS; ++s) {
      const int r = s * RPS + t / 32, ch = t % 32;
      const int m = m0 + r, n = n0 + ch * 8;
      if (m >= a.M || n >= a.N) continue;
      const u16x8 v = *(__attribute__((address_space(3))) u16x8*)(uintptr_t)(lds0 + (uint32_t)(r * RB2 + (ch ^ (r & 15)) * 16));
      uint16_t* cp = (uint16_t*)a.C + (int64_t)m * a.ldc + n;
      if (n + 8 <= a.N) {
        __builtin_nontemporal_store(v, (u16x8*)cp);
      } else {
#pragma unroll
        for (int e = 0; e < 8; ++e)
          if (n + e < a.N) cp[e] = v[e];
      }
    }
    return;
  }
#pragma unroll
  for (int g = 0; g < 2; ++g) {
    __syncthreads();  // the LDS is free: the K loop's reads, or the previous pass's
    if (grp == g) {
      static_for<C::FM * C::FN>([&](auto pc) {
        constexpr int p = decltype(pc)::value;
        constexpr int i = p / C::FN, j = p % C::FN;
        const int r = i * 16 + lane % 16;                 // row within the pass
        const int c = xb0 + j * 16 + 4 * (lane / 16);     // column, a multiple of 4
        const int chunk = (c >> 2) ^ (r & 15);
        const f32x4 v = {alpha * acc[i][j][0], alpha * acc[i][j][1], alpha * acc[i][j][2], alpha * acc[i][j][3]};
        *(__attribute__((address_space(3))) f32x4*)(uintptr_t)(lds0 + (uint32_t)(r * RB + chunk * 16)) = v;
      });
    }
    __syncthreads();
    constexpr int RPS = C::THREADS / 32;  // rows per step
#pragma unroll 2
    for (int s = 0; s < C::WTM / RPS; ++s) {
      const int r = s * RPS + t / 32, ch = (t % 32) * 2;  // 8 columns: chunks ch, ch + 1
      const int m = m0 + g * C::WTM + r, n = n0 + ch * 4;
      if (m >= a.M || n >= a.N) continue;
      const uint32_t row = lds0 + (uint32_t)(r * RB);
      const f32x4 lo = *(__attribute__((address_space(3))) f32x4*)(uintptr_t)(row + ((ch ^ (r & 15)) * 16));
      const f32x4 hi = *(__attribute__((address_space(3))) f32x4*)(uintptr_t)(row + (((ch + 1) ^ (r & 15)) * 16));
      float w[8] = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
      const int64_t base = (int64_t)m * a.ldc + n;
      if (n + 8 <= a.N) {
        if (a.c_kind == C_F32) {
          f32x4* cp = (f32x4*)((float*)a.C + base);
          if (beta != 0.f) {
            const f32x4 o0 = cp[0], o1 = cp[1];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              w[e] += beta * o0[e];
              w[4 + e] += beta * o1[e];
            }
          }
          __builtin_nontemporal_store((f32x4){w[0], w[1], w[2], w[3]}, cp);
          __builtin_nontemporal_store((f32x4){w[4], w[5], w[6], w[7]}, cp + 1);
        } else if (a.c_kind == C_E4M3) {
          uint32_t* cp = (uint32_t*)((uint8_t*)a.C + base);
          if (beta != 0.f) {
            const uint32_t o0 = cp[0], o1 = cp[1];
            static_for<4>([&](auto ec) {
              constexpr int e = decltype(ec)::value;
              w[e] += beta * __builtin_amdgcn_cvt_f32_fp8((int)o0, e);
              w[4 + e] += beta * __builtin_amdgcn_cvt_f32_fp8((int)o1, e);
            });
          }
          __builtin_nontemporal_store(
              (u32x2){e4m3x4_from_f32(w[0], w[1], w[2], w[3]), e4m3x4_from_f32(w[4], w[5], w[6], w[7])}, (u32x2*)cp);
        } else {
          uint16_t* cp = (uint16_t*)a.C + base;
          if (beta != 0.f) {
            const u16x8 o = *(const u16x8*)cp;
#pragma unroll
            for (int e = 0; e < 8; ++e) w[e] += beta * bf16_bits_to_f32(o[e]);
          }
          u16x8 v;
#pragma unroll
          for (int e = 0; e < 8; ++e) v[e] = f32_to_bf16_bits(w[e]);
          __builtin_nontemporal_store(v, (u16x8*)cp);
        }
      } else {  // the last columns of C
#pragma unroll
        for (int e = 0; e < 8; ++e) {
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
  }
}

// SK = false: one workgroup per output tile, its whole K loop.  SK = true: the stream-K
// grid of GemmArgs (sk_dp whole tiles, then sk_grid workgroups sharing the K loops of the
// other sk_tiles tiles).  Each workgroup runs its segments (a tile and a range [k0, k1) of
// its K tiles) one after the other, each through the same two-group pipeline.
template <class C, bool SK>
__global__ __launch_bounds__(512) void gemm_pp_kernel(GemmArgs a) {
  using P = PingPong<C>;
  constexpr int S = P::S;
  __shared__ __attribute__((aligned(1024))) char lds[P::LDS_BYTES];
  using Acc = typename AccOf<C::MT>::T;

  const int t = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(t >> 6);
  // waves are dealt to the four SIMDs in turn: waves w and w + 4 share a SIMD
  const int grp = wave >> 2;
  const int wn = wave & 3;
  const int wm = grp;
  const int nk = (a.K + C::BK - 1) / C::BK;
  const int nkb = (a.K + 31) / 32;  // 32-element K blocks (block scales)

  // ---- this workgroup's work: K tiles [it, it_end) of the sequence that lays the K loops
  // of the stream-K tiles end to end (tile ts of that part holds [ts*nk, (ts+1)*nk)), or
  // one whole tile.  `slot` is the stream-K workgroup's index: consecutive indices share
  // tiles, and they are grouped by XCD (ids b run on XCD b % xcd) so that a tile's owner
  // and the workgroups that hand it partials mostly share one L2.
  int it = 0, it_end = nk, slot = 0;
  int tm0 = 0, tn0 = 0;
  bool whole = true;
  if constexpr (SK) {
    const int b = blockIdx.x;
    if (b < a.sk_dp) {
      raster_tile(xcd_remap(b, a.sk_dp, a.xcd), a, tm0, tn0);
    } else {
      const int q = b - a.sk_dp, G = a.sk_grid;
      slot = (a.xcd > 1 && G % a.xcd == 0) ? ((q + a.sk_dp) % a.xcd) * (G / a.xcd) + q / a.xcd : q;
      it = slot * a.sk_iters;
      it_end = min(it + a.sk_iters, a.sk_tiles * nk);
      whole = false;
      if (it >= it_end) return;  // an empty range (uniform over the workgroup)
    }
  } else {
    int split_unused;  // unsplit
    tile_of(blockIdx.x, a, tm0, tn0, split_unused);
  }

  const uint32_t a_rows = C::A_KC ? a.M : a.K;
  const uint32_t b_rows = C::B_KC ? a.N : a.K;
  // 32-bit offsets: every operand spans less than 2^31 bytes with 256 rows (of K for an
  // M/N-contiguous operand) to spare, more than the S tiles issued past the end
  const uint32_t a_kstep = C::A_KC ? C::BK * C::ES : (uint32_t)(C::BK * a.lda * C::ES);
  const uint32_t b_kstep = C::B_KC ? C::BK * C::ES : (uint32_t)(C::BK * a.ldb * C::ES);
  const uint32_t a_total = (uint32_t)(a_rows * a.lda * C::ES), b_total = (uint32_t)(b_rows * a.ldb * C::ES);
  const uint32_t lds0 = (uint32_t)(uintptr_t)(lds_char*)lds;

  for (;;) {
    // ---- the segment: tile (tm, tn), K tiles [k0, k1)
    int tm = tm0, tn = tn0, k0 = 0, k1 = nk;
    if (!whole) {
      const int ts = it / nk;
      k0 = it - ts * nk;
      k1 = min(nk, k0 + (it_end - it));
      raster_tile(a.sk_dp + ts, a, tm, tn);
    }
    const int m0 = tm * C::BM, n0 = tn * C::BN;
    // The thread index through an opaque copy: everything derived from it below (fragment
    // addresses, copy offsets, partial-tile offsets) is computed again for each segment
    // instead of being hoisted out of the segment loop and held in registers across the
    // K loop.
    int lane_t = t;
    asm volatile("" : "+v"(lane_t));
    lane_t &= C::THREADS - 1;
    const int lane = lane_t & 63;

    // ---- fragment addresses of this lane, computed once for slot 0.  For a K-contiguous
    // operand fragments MT rows apart share their swizzle, so fragment f of K step kk sits
    // at base[kk] + f*MT rows; for an M/N-contiguous operand the K step and the second
    // transposing read only add whole rows (the swizzle depends on bits 0, 1 and 3 of the
    // row, which neither touches), so it sits at base[f] + (kk*KT + h*4) rows.  A slot
    // adds its offset; all of these constants become the reads' immediate offsets.
    const int xa0 = wm * C::WTM, xb0 = wn * C::WTN;
    constexpr int A_NB = C::A_KC ? C::KSTEPS : C::FM, B_NB = C::B_KC ? C::KSTEPS : C::FN;
    uint32_t a_base[A_NB], b_base[B_NB];
  #pragma unroll
    for (int v = 0; v < A_NB; ++v)
      a_base[v] = lds0 + P::A_OFF +
                  (C::A_KC ? pp_frag_off<C, true, C::A_RB>(xa0, v * C::KT, lane, 0)
                           : pp_frag_off<C, false, C::A_RB>(xa0 + v * C::MT, 0, lane, 0));
  #pragma unroll
    for (int v = 0; v < B_NB; ++v)
      b_base[v] = lds0 + P::B_OFF +
                  (C::B_KC ? pp_frag_off<C, true, C::B_RB>(xb0, v * C::KT, lane, 0)
                           : pp_frag_off<C, false, C::B_RB>(xb0 + v * C::MT, 0, lane, 0));
    // LDS address of read h of fragment f (K step kk) of an operand in slot u
    auto a_addr = [&](int u, int kk, int f, int h) -> uint32_t {
      return C::A_KC ? a_base[kk] + (uint32_t)(u * C::A_BYTES + f * C::MT * C::A_RB)
                     : a_base[f] + (uint32_t)(u * C::A_BYTES + (kk * C::KT + h * 4) * C::A_RB);
    };
    auto b_addr = [&](int u, int kk, int f, int h) -> uint32_t {
      return C::B_KC ? b_base[kk] + (uint32_t)(u * C::B_BYTES + f * C::MT * C::B_RB)
                     : b_base[f] + (uint32_t)(u * C::B_BYTES + (kk * C::KT + h * 4) * C::B_RB);
    };

    bf16x8 fa[C::FM], fb[C::FN];
    // E4M3: the raw 8-byte A fragments, widened by the compute phase that uses them
    i32x2 ra8[P::E8 ? C::FM : 1];
    // block scales: the scale words of a K tile for the rows of the A fragments (rows
    // xa0 + 16 i + lane % 16) and of the B fragments, byte kk the code of K step kk; set b
    // serves the tile in slot b, and is read during the tile before it (in the memory
    // phase of its second K step, one of the lighter ones)
    constexpr int NSW = P::MXS ? S : 1;
    uint32_t swa[NSW][P::MXS ? C::FM : 1], swb[NSW][P::MXS ? C::FN : 1];
    float soa[P::MXS ? C::FM : 1], sob[P::MXS ? C::FN : 1];  // one K step's scale operands
    static_assert(!P::MXS || (C::FM == 8 && C::FN == 4 && C::WTM == 128 && C::WTN == 64),
                  "a lane's A scale rows are 8 positions in two runs of 4, its B rows one run");
    // the conversion's scale operand for K step kk: code kk of word w in the exponent field
    // (the bits shifted in below and above it are ignored)
    auto scale_op = [](uint32_t w, int kk) -> float {
      return __builtin_bit_cast(float, kk == 3 ? w >> 1 : w << (23 - 8 * kk));
    };
    // ---- block scales.  Wave w copies positions [64 w, 64 w + 64) (waves 0-3: rows of A,
    // 4-7: rows of B); the dword of a row at K tile kt is its bytes [4 kt, 4 kt + 4), the
    // scales of K blocks 4 kt .. 4 kt + 3 (whole dwords: scale rows are 4-byte aligned),
    // and its 16 bytes at 16 q those of K tiles 4 q .. 4 q + 3 (with 16-byte aligned rows,
    // whose length covers them).  A row past M or N reads zeros.
    const bool sc_quad = P::MXS && ((((uintptr_t)a.sa | (uintptr_t)a.sb) & 15u) | ((a.ldsa | a.ldsb) & 15)) == 0;
    uint32_t sc_goff = kOOB;
    __amdgpu_buffer_rsrc_t sc_rsrc = make_rsrc(nullptr, 0u);
    if constexpr (P::MXS) {
      const int pos = (wave & 3) * 64 + lane;  // position within the operand's 256
      if (wave < 4) {
        const int r = (pos >> 7) * 128 + (((pos >> 6) & 1) * 4 + (pos & 3)) * 16 + ((pos >> 2) & 15);
        sc_goff = m0 + r < a.M ? (uint32_t)((m0 + r) * a.ldsa) : kOOB;
        sc_rsrc = make_rsrc(a.sa, (uint32_t)(a.M * a.ldsa));
      } else {
        const int r = (pos >> 6) * 64 + (pos & 3) * 16 + ((pos >> 2) & 15);
        sc_goff = n0 + r < a.N ? (uint32_t)((n0 + r) * a.ldsb) : kOOB;
        sc_rsrc = make_rsrc(a.sb, (uint32_t)(a.N * a.ldsb));
      }
    }
    // the scale bytes that ride with the copies of K tile kt: the next tile's dwords, or
    // (16-byte rows) the 16 bytes of K tiles kt + 2 .. kt + 5 with every fourth tile
    auto scale_copy = [&](int kt) {
      if (sc_quad) {
        if ((kt & 3) != 2) return;
        const int q = (kt + 2) >> 2;
        const uint32_t l = lds0 + P::SCB_OFF + (uint32_t)((q & 1) * 4 * P::SC_TABLE + wave * 1024);
        const uint32_t o[1] = {sc_goff + (uint32_t)q * 16u};
        pp_copies<1, false>(__builtin_amdgcn_readfirstlane(l), o, sc_rsrc);
      } else {
        const uint32_t l = lds0 + P::SCB_OFF + (uint32_t)(((kt + 1) & 3) * 2 * P::SC_TABLE + wave * 256);
        pp_load_to_lds_dword(__builtin_amdgcn_readfirstlane(l), sc_goff + (uint32_t)(kt + 1) * 4u, sc_rsrc);
      }
    };
    // This lane's scale words of K tile kt (its 8 A rows and 4 B rows) into set bc, with the
    // codes of K blocks past K (whose operands read zeros) replaced by 127 (scale 1) in the
    // last K tile: the bytes there may be row padding, and code 255 would give NaN even on
    // zeros.
    const int sc_l = lane & 15;
    auto read_scales = [&](int kt, auto bc) {
      constexpr int sb = P::MXS ? decltype(bc)::value : 0;
      const uint32_t pa = (uint32_t)(wm * 128 + sc_l * 4), pb = (uint32_t)(256 + wn * 64 + sc_l * 4);
      // K tile kt's table: four per 16-byte copy, or one per copy of 4 bytes
      const uint32_t base = lds0 + (sc_quad ? (uint32_t)(P::SCR_OFF + (((kt >> 2) & 1) * 4 + (kt & 3)) * P::SC_TABLE)
                                            : (uint32_t)(P::SCB_OFF + (kt & 3) * 2 * P::SC_TABLE));
      const u32x4 a0 = *(__attribute__((address_space(3))) u32x4*)(uintptr_t)(base + pa * 4);
      const u32x4 a1 = *(__attribute__((address_space(3))) u32x4*)(uintptr_t)(base + (pa + 64) * 4);
      const u32x4 b0 = *(__attribute__((address_space(3))) u32x4*)(uintptr_t)(base + pb * 4);
  #pragma unroll
      for (int e = 0; e < 4; ++e) {
        swa[sb][e] = a0[e];
        swa[sb][4 + e] = a1[e];
        swb[sb][P::MXS ? e : 0] = b0[e];
      }
      const int nvalid = nkb - kt * 4;  // blocks of this tile inside K (uniform)
      if (nvalid < 4) {
        const uint32_t keep = nvalid <= 0 ? 0u : (1u << (8 * nvalid)) - 1u;
  #pragma unroll
        for (int i = 0; i < 8; ++i) swa[sb][i] = (swa[sb][i] & keep) | (0x7F7F7F7Fu & ~keep);
  #pragma unroll
        for (int j = 0; j < 4; ++j) swb[sb][P::MXS ? j : 0] = (swb[sb][P::MXS ? j : 0] & keep) | (0x7F7F7F7Fu & ~keep);
      }
    };
    // 16-byte scale rows: thread t moves position t of the copy of K tiles 4q .. 4q + 3
    // into the four tables of set q % 2 (run during K tile 4q - 2, after that copy has
    // landed and after the tables' previous K tiles, 4q - 8 .. 4q - 5, were read)
    auto scale_spread = [&](int q) {
      const u32x4 w = *(__attribute__((address_space(3))) u32x4*)(uintptr_t)(
          lds0 + P::SCB_OFF + (uint32_t)((q & 1) * 4 * P::SC_TABLE + lane_t * 16));
      const uint32_t d = lds0 + P::SCR_OFF + (uint32_t)((q & 1) * 4 * P::SC_TABLE + lane_t * 4);
  #pragma unroll
      for (int e = 0; e < 4; ++e) *(__attribute__((address_space(3))) uint32_t*)(uintptr_t)(d + e * P::SC_TABLE) = w[e];
    };

    auto rd = [&](uint32_t addr) -> u16x4 {
      return __builtin_bit_cast(u16x4, __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                                           (__attribute__((address_space(3))) s16x4*)(uintptr_t)addr));
    };
    // (The plain 8-byte reads are volatile so that the compiler does not pair the reads of
    // two fragments 16 rows apart into one ds_read2st64_b64: the two addresses of a lane
    // then fall in the same banks; the LDS read probe's paired form, kind 5, runs 2.3x the
    // time per fragment of single ds_read_b64, with bank conflicts where those have none.)
    auto rd8 = [&](uint32_t addr, bool tr) -> i32x2 {
      if (tr) return __builtin_amdgcn_ds_read_tr8_b64_v2i32((__attribute__((address_space(3))) i32x2*)(uintptr_t)addr);
      return *(volatile __attribute__((address_space(3))) i32x2*)(uintptr_t)addr;
    };
    // Memory phase: the fragments of K step kk of the tile in slot u (E4M3 tiles: all reads
    // first, then the widening, so that the reads are in flight together).
    auto read_step = [&](auto uc, auto kc, int rkt) {
      constexpr int u = decltype(uc)::value, kk = decltype(kc)::value;
      if constexpr (P::E8) {
        // B fragments and the first A fragment are widened here; the other A fragments in
        // the compute phase, between the MFMAs (the conversions share the issue port with
        // the MFMAs of the wave computing next to this one)
        i32x2 rb8[C::FN];
  #pragma unroll
        for (int i = 0; i < C::FM; ++i) ra8[i] = rd8(a_addr(u, kk, i, 0), !C::A_KC);
  #pragma unroll
        for (int j = 0; j < C::FN; ++j) rb8[j] = rd8(b_addr(u, kk, j, 0), !C::B_KC);
        if constexpr (P::MXS) {
          // this step's scale operands, formed while the reads are in flight (a shift
          // right before the conversion that reads it would stall it)
          constexpr int sb = P::MXS ? u : 0;
          __builtin_amdgcn_sched_barrier(0);
  #pragma unroll
          for (int i = 0; i < C::FM; ++i) soa[P::MXS ? i : 0] = scale_op(swa[sb][P::MXS ? i : 0], kk);
  #pragma unroll
          for (int j = 0; j < C::FN; ++j) sob[P::MXS ? j : 0] = scale_op(swb[sb][P::MXS ? j : 0], kk);
          __builtin_amdgcn_sched_barrier(0);
  #pragma unroll
          for (int j = 0; j < C::FN; ++j) fb[j] = pp_widen8(rb8[j], sob[P::MXS ? j : 0]);
          fa[0] = pp_widen8(ra8[0], soa[0]);
          // the next tile's scale words (its bytes landed before this tile began)
          if constexpr (kk == 1) read_scales(rkt + 1, std::integral_constant<int, (u + 1) % S>{});
          if constexpr (kk == 2)
            if (sc_quad && (rkt & 3) == 2) scale_spread((rkt + 2) >> 2);
        } else {
  #pragma unroll
          for (int j = 0; j < C::FN; ++j) fb[j] = pp_widen8(rb8[j]);
          fa[0] = pp_widen8(ra8[0]);
        }
        return;
      }
  #pragma unroll
      for (int i = 0; i < C::FM; ++i) {
        if constexpr (C::A_KC) {
          fa[i] = *(__attribute__((address_space(3))) bf16x8*)(uintptr_t)a_addr(u, kk, i, 0);
        } else {
          const u16x4 lo = rd(a_addr(u, kk, i, 0)), hi = rd(a_addr(u, kk, i, 1));
          fa[i] = __builtin_bit_cast(bf16x8, (u16x8){lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]});
        }
      }
  #pragma unroll
      for (int j = 0; j < C::FN; ++j) {
        if constexpr (C::B_KC) {
          fb[j] = *(__attribute__((address_space(3))) bf16x8*)(uintptr_t)b_addr(u, kk, j, 0);
        } else {
          const u16x4 lo = rd(b_addr(u, kk, j, 0)), hi = rd(b_addr(u, kk, j, 1));
          fb[j] = __builtin_bit_cast(bf16x8, (u16x8){lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]});
        }
      }
    };
    Acc acc[C::FM][C::FN];
    // Compute phase: the MFMA cluster of one K step, at raised wave priority.  With E4M3
    // tiles the MFMAs of A row i are followed by the four conversions of A fragment i + 1.
    static_assert(!P::E8 || C::FN == 4, "four conversions per A fragment, one after each MFMA of a row");
    int wpart[4];
    auto compute_step = [&]() {
      __builtin_amdgcn_s_setprio(1);
      static_for<C::FM * C::FN>([&](auto ic) {
        constexpr int i = decltype(ic)::value;
        constexpr int row = i / C::FN, col = i % C::FN;
        mma(acc[row][col], fb[col], fa[row]);
        if constexpr (P::E8 && row + 1 < C::FM) {
          const float sc = P::MXS ? soa[P::MXS ? row + 1 : 0] : 1.0f;
          wpart[col] = __builtin_bit_cast(int, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(ra8[row + 1][col >> 1], sc,
                                                                                         (col & 1) != 0));
          if constexpr (col == 3)
            fa[row + 1] = __builtin_bit_cast(bf16x8, (i32x4){wpart[0], wpart[1], wpart[2], wpart[3]});
        }
        __builtin_amdgcn_sched_barrier(0);
      });
      __builtin_amdgcn_s_setprio(0);
    };
    // copies allowed in flight at the barrier before a tile's first K step is read: those
    // of the S - 2 tiles issued after it
    constexpr int VM = (S - 2) * P::IPW;
    constexpr int KS = C::KSTEPS;


    // ---- this wave's copy instructions: instruction i fills LDS block wave*IPW + i of the
    // tile (A blocks, then B); this lane fills chunk p = blk*64 + lane of its operand, row
    // p / CPR, physical chunk p % CPR, which holds logical chunk (p % CPR) ^ swizzle(row).
    // The per-lane offsets are relative to the start of a K tile, and fixed: each K tile
    // gets its own buffer descriptor (base moved to the tile, size cut by as much), built
    // with scalar arithmetic.  A chunk in a row or column past M or N gets an offset past
    // every buffer.  Rows at or past the segment's end in K of an M/N-contiguous operand
    // then lie past the tile's buffer and read zeros; a K-contiguous operand's chunks
    // there (a ragged last tile, or a tile past the segment) are sent past the buffer in
    // copy_tile.
    uint32_t a_off[P::A_IPW], b_off[P::B_IPW];
    auto chunk_k = [&](int blk, int CPR, int VEC, auto swzc) {  // K index of a K-contiguous chunk
      const int p = blk * 64 + lane;
      return ((p % CPR) ^ swzc(p / CPR)) * VEC;
    };
#pragma unroll
    for (int i = 0; i < P::A_IPW; ++i) {
      const int p = (wave * P::A_IPW + i) * 64 + lane;
      const int r = p / C::A_CPR;
      const int c = (p % C::A_CPR) ^ pp_swz<C, C::A_KC, C::A_CPR>(r);
      if constexpr (C::A_KC)
        a_off[i] = (m0 + r) < a.M ? (uint32_t)((m0 + r) * a.lda + c * C::VEC) * C::ES : kOOB;
      else
        a_off[i] = (m0 + c * C::VEC) < a.M ? (uint32_t)(r * a.lda + m0 + c * C::VEC) * C::ES : kOOB;
    }
#pragma unroll
    for (int i = 0; i < P::B_IPW; ++i) {
      const int p = (wave * P::B_IPW + i) * 64 + lane;
      const int r = p / C::B_CPR;
      const int c = (p % C::B_CPR) ^ pp_swz<C, C::B_KC, C::B_CPR>(r);
      if constexpr (C::B_KC)
        b_off[i] = (n0 + r) < a.N ? (uint32_t)((n0 + r) * a.ldb + c * C::VEC) * C::ES : kOOB;
      else
        b_off[i] = (n0 + c * C::VEC) < a.N ? (uint32_t)(r * a.ldb + n0 + c * C::VEC) * C::ES : kOOB;
    }
    // the segment's end in K (elements), and the bytes of each operand before it: all of
    // a K-contiguous operand, the rows before it of an M/N-contiguous one
    const int kend = min(a.K, k1 * C::BK);
    const uint32_t a_lim = C::A_KC || !SK ? a_total : min(a_total, (uint32_t)(kend * a.lda * C::ES));
    const uint32_t b_lim = C::B_KC || !SK ? b_total : min(b_total, (uint32_t)(kend * a.ldb * C::ES));

    // Copies of K tile kt into slot u: A blocks first, then B.  Tiles past the segment are
    // still issued (all their chunks read zeros), so that every wave has the same number
    // of copies in flight at every barrier and the waits can count them.
    auto copy_tile = [&](int u, int kt) {
      const uint32_t ao = (uint32_t)kt * a_kstep, bo = (uint32_t)kt * b_kstep;
      // the tile's buffer: base moved to the tile, size cut by as much (none left past the
      // end).  The sizes go through readfirstlane: the saturating subtraction is a VALU
      // instruction, and a descriptor built from a VGPR would not be a scalar operand.
      const uint32_t an = __builtin_amdgcn_readfirstlane(a_lim - min(ao, a_lim));
      const uint32_t bn = __builtin_amdgcn_readfirstlane(b_lim - min(bo, b_lim));
      const __amdgpu_buffer_rsrc_t rta = make_rsrc((const char*)a.A + ao, an);
      const __amdgpu_buffer_rsrc_t rtb = make_rsrc((const char*)a.B + bo, bn);
      // this wave's first LDS block of each operand tile (its blocks are consecutive)
      const uint32_t la = lds0 + P::A_OFF + u * C::A_BYTES + (uint32_t)(wave * P::A_IPW) * 1024u;
      const uint32_t lb = lds0 + P::B_OFF + u * C::B_BYTES + (uint32_t)(wave * P::B_IPW) * 1024u;
      const int kleft = kend - kt * C::BK;  // K elements left from this tile's start
      if ((!C::A_KC && !C::B_KC) || kleft >= C::BK) {
        pp_copies<P::A_IPW, false>(la, a_off, rta);
        pp_copies<P::B_IPW, false>(lb, b_off, rtb);
      } else {  // a ragged last tile or a tile past the segment: K-contiguous chunks there read zeros
        uint32_t oa[P::A_IPW], ob[P::B_IPW];
#pragma unroll
        for (int q = 0; q < P::A_IPW; ++q)
          oa[q] = !C::A_KC || chunk_k(wave * P::A_IPW + q, C::A_CPR, C::VEC,
                                      [](int r) { return pp_swz<C, true, C::A_CPR>(r); }) < kleft ? a_off[q] : kOOB;
#pragma unroll
        for (int q = 0; q < P::B_IPW; ++q)
          ob[q] = !C::B_KC || chunk_k(wave * P::B_IPW + q, C::B_CPR, C::VEC,
                                      [](int r) { return pp_swz<C, true, C::B_CPR>(r); }) < kleft ? b_off[q] : kOOB;
        pp_copies<P::A_IPW, true>(la, oa, rta);
        pp_copies<P::B_IPW, true>(lb, ob, rtb);
      }
      if constexpr (P::MXS) scale_copy(kt);
    };

#pragma unroll
    for (int i = 0; i < C::FM; ++i)
#pragma unroll
      for (int j = 0; j < C::FN; ++j) acc[i][j] = Acc{};

    // ---- prologue: K tiles k0 .. k0+S-1 into slots 0 .. S-1; wait for the first.  With
    // block scales (one segment per workgroup: k0 = 0), the first scale bytes go first (the
    // others ride with the copies of the tiles before them).  With 16-byte rows, tiles k0
    // and k0 + 1 carry none, so the wait counts the data copies of tile k0 + 1 alone.
    if constexpr (P::MXS) scale_copy(sc_quad ? k0 - 2 : k0 - 1);
    static_for<S>([&](auto uc) { copy_tile(decltype(uc)::value, k0 + decltype(uc)::value); });
    if constexpr (P::MXS) {
      if (sc_quad)
        pp_wait_vm_barrier<(S - 1) * P::DATA_IPW>();
      else
        pp_wait_vm_barrier<(S - 1) * P::IPW>();
      if (sc_quad) {
        scale_spread(k0 >> 2);
        pp_wait_lds_barrier();
      }
      read_scales(k0, std::integral_constant<int, 0>{});
    } else {
      pp_wait_vm_barrier<(S - 1) * P::IPW>();
    }

    // ---- main loop over K steps h = (tile t, step kk), S tiles per iteration so that slots
    // are compile-time constants: tile t sits in slot (t - k0) % S.  Group 0 computes step h
    // while group 1 reads it, then group 1 computes h while group 0 reads h + 1; barriers
    // B(2h+1) and B(2h+2) separate the phases.  Once both groups have read the last step of
    // tile t (B(2h+1) of that step) tile t + S replaces it: group 0 issues its copies right
    // after that barrier, group 1 at the start of its next memory phase.  Before the
    // barrier after which the first step of tile t + 1 is read, every wave waits for its
    // copies of tile t + 1.  Both groups run 2 (k1 - k0) KS barriers in all.
    if (grp == 0) {
      read_step(std::integral_constant<int, 0>{}, std::integral_constant<int, 0>{}, k0);
      __builtin_amdgcn_sched_barrier(0);
      pp_wait_lds_barrier();  // B0
      for (int kt0 = k0; kt0 < k1; kt0 += S) {
        static_for<S>([&](auto uc) {
          constexpr int u = decltype(uc)::value;
          const int kt = kt0 + u;
          if (kt < k1) {
            static_for<KS>([&](auto kc) {
              constexpr int kk = decltype(kc)::value;
              constexpr bool last = kk == KS - 1;
              compute_step();
              if constexpr (last) {
                pp_wait_vm_barrier<VM>();  // B(2h+1): tile t + 1 complete, slot u free
              } else {
                pp_wait_lds_barrier();  // B(2h+1)
              }
              // the fragment reads go out first, then the copies (whose issue can wait on a
              // full address queue)
              if (!last || kt + 1 < k1)
                read_step(std::integral_constant<int, last ? (u + 1) % S : u>{},
                          std::integral_constant<int, last ? 0 : kk + 1>{}, last ? kt + 1 : kt);
              if constexpr (last) copy_tile(u, kt + S);
              __builtin_amdgcn_sched_barrier(0);
              if (!last || kt + 1 < k1) pp_wait_lds_barrier();  // B(2h+2)
            });
          }
        });
      }
    } else {
      pp_wait_lds_barrier();  // B0
      for (int kt0 = k0; kt0 < k1; kt0 += S) {
        static_for<S>([&](auto uc) {
          constexpr int u = decltype(uc)::value;
          const int kt = kt0 + u;
          if (kt < k1) {
            static_for<KS>([&](auto kc) {
              constexpr int kk = decltype(kc)::value;
              constexpr bool last = kk == KS - 1;
              read_step(uc, kc, kt);
              // the slot of tile t - 1, left by both groups at the last B(2h+1) of that tile
              if (kk == 0 && kt > k0) copy_tile((u + S - 1) % S, kt - 1 + S);
              __builtin_amdgcn_sched_barrier(0);
              if constexpr (last) {
                pp_wait_vm_barrier<VM>();  // B(2h+1)
              } else {
                pp_wait_lds_barrier();
              }
              compute_step();
              if (!last || kt + 1 < k1) {
                pp_wait_lds_barrier();  // B(2h+2)
              }
            });
          }
        });
      }
    }
    // the last copies (past the segment) land before the LDS is reused or released
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");

    if constexpr (SK) {
      if (k0 != 0) {
        // Not the tile's first K tile: leave the partial sum in this workgroup's slot and
        // raise its flag.  Every wave waits for its stores to complete (to this XCD's L2)
        // before the workgroup barrier; then one thread raises the flag with release
        // semantics at device scope, which first writes the L2's dirty lines back, so the
        // owner (perhaps on another XCD, behind another L2) reads the partial from memory.
        // This is always the workgroup's first segment.
        pp_store_partial<C>(a.ws + (size_t)slot * (C::BM * C::BN), acc, (uint32_t)lane_t * 16u);
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        __syncthreads();
        if (t == 0) __hip_atomic_store(a.flags + slot, a.epoch, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
      } else {
        if (k1 < nk) {
          // The tile's first K tiles: the rest of its K loop was summed by the next
          // workgroups of the sequence, each starting inside this tile.  Wait for their
          // flags, then add their partials in K order and clear the flags for the next call.
          // The flag loads have acquire semantics at device scope (they invalidate this
          // XCD's L2 and the CU's cache), and the barrier orders every wave's partial loads
          // after them.
          __shared__ int sk_ok;
          const int ts = it / nk;
          const int last_slot = ((ts + 1) * nk - 1) / a.sk_iters;
          if (t == 0) {
            int ok = 1;
            for (int s2 = slot + 1; s2 <= last_slot && ok; ++s2) {
              int n = 0;
              while (__hip_atomic_load(a.flags + s2, __ATOMIC_ACQUIRE, __HIP_MEMORY_SCOPE_AGENT) != a.epoch) {
                if (++n >= kStreamKSpins) {
                  ok = 0;
                  break;
                }
                __builtin_amdgcn_s_sleep(8);
              }
            }
            sk_ok = ok;
          }
          __syncthreads();
          if (sk_ok) {
            for (int s2 = slot + 1; s2 <= last_slot; ++s2)
              pp_add_partial<C>(a.ws + (size_t)s2 * (C::BM * C::BN), acc, (uint32_t)lane_t * 16u);
          } else {
#pragma unroll
            for (int i = 0; i < C::FM; ++i)
#pragma unroll
              for (int j = 0; j < C::FN; ++j)
#pragma unroll
                for (int e = 0; e < C::ACC; ++e) acc[i][j][e] = __builtin_nanf("");
          }
          if (t == 0)
            for (int s2 = slot + 1; s2 <= last_slot; ++s2)
              __hip_atomic_store(a.flags + s2, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
        pp_store_tile_lds<C>(a, acc, m0, n0, grp, xb0, lane, t, lds0);
      }
      it += k1 - k0;
      if (whole || it >= it_end) break;
      // the next segment's waits count its copies with vmcnt, which also counts this
      // segment's stores, and stores may complete after later loads: drain them first; and
      // its copies overwrite the LDS, which the epilogue may still be reading
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
      __syncthreads();
    } else {
      pp_store_tile_lds<C>(a, acc, m0, n0, grp, xb0, lane, t, lds0);
      break;
    }
  }
}

template <class C>
hipError_t launch_pp(const GemmArgs& a, hipStream_t s) {
  if (a.splits != 1 || a.tri != TRI_NONE || a.kband != KBAND_NONE || a.dual) return hipErrorInvalidConfiguration;
  if constexpr (PingPong<C>::MXS) {
    // scale rows of whole dwords, at least one byte per 32-element block of K
    if (!a.mx || !a.sa || !a.sb || ((uintptr_t)a.sa & 3u) || ((uintptr_t)a.sb & 3u) || (a.ldsa & 3) ||
        (a.ldsb & 3) || a.ldsa < (a.K + 31) / 32 || a.ldsb < (a.K + 31) / 32)
      return hipErrorInvalidConfiguration;
  }
  if (a.sk_tiles > 0) {
    // no stream-K form of the 128-deep E4M3 tiles (the host never plans one: they would
    // spill), so none is instantiated
    if constexpr ((C::IN == IN_E4M3_LDS && C::BK > 64) || C::IN == IN_MX_LDS) {
      return hipErrorInvalidConfiguration;
    } else {
      if (!a.ws || !a.flags || a.sk_grid < 1 || a.sk_iters < 1 || a.epoch == 0 ||
          (int64_t)a.sk_grid * a.sk_iters < (int64_t)a.sk_tiles * ((a.K + C::BK - 1) / C::BK) ||
          a.sk_dp + a.sk_tiles != a.tiles_m * a.tiles_n)
        return hipErrorInvalidConfiguration;
      hipLaunchKernelGGL((gemm_pp_kernel<C, true>), dim3(a.sk_dp + a.sk_grid), dim3(C::THREADS), 0, s, a);
    }
  } else {
    hipLaunchKernelGGL((gemm_pp_kernel<C, false>), dim3(grid_tiles(a)), dim3(C::THREADS), 0, s, a);
  }
  return hipGetLastError();
}

#if !defined(DBGEMM_DMA_TA) || !defined(DBGEMM_DMA_TB)
#error "compile with -DDBGEMM_DMA_TA=0|1 -DDBGEMM_DMA_TB=0|1"
#endif

}  // namespace

#define DBGEMM_PP_CAT2(a, b) launch_mfma_pp_##a##b
#define DBGEMM_PP_CAT(a, b) DBGEMM_PP_CAT2(a, b)

// pipe 2 entries of the policy table; a tile edge whose M/N-contiguous rows would not be
// a power of two of chunks is not instantiated for that transpose case (the policy code
// does not choose it there)
constexpr bool pp_pow2(int x) { return (x & (x - 1)) == 0; }

hipError_t DBGEMM_PP_CAT(DBGEMM_DMA_TA, DBGEMM_DMA_TB)(const Policy& p, const GemmArgs& a, hipStream_t s) {
#define DBGEMM_SIMT(name, eff)
#define DBGEMM_MFMA(name_, pipe_, in_, bm_, bn_, bk_, wm_, wn_, mt_, st_, grp_, rn_, xcd_, sw_, eff_)        \
  if constexpr (pipe_ == 2 && pp_pow2(DBGEMM_DMA_TA ? (bm_) : 16) && pp_pow2(DBGEMM_DMA_TB ? 16 : (bn_)) &&  \
                (in_ != IN_MX_LDS || (DBGEMM_DMA_TA == 0 && DBGEMM_DMA_TB == 1)))                           \
    if (p.BM == bm_ && p.BN == bn_ && p.BK == bk_ && p.WM == wm_ && p.WN == wn_ && p.MT == mt_ &&          \
        p.stages == st_ && p.in_mode == in_)                                                               \
      return launch_pp<Cfg<bm_, bn_, bk_, wm_, wn_, mt_, st_, in_, DBGEMM_DMA_TA != 0, DBGEMM_DMA_TB != 0>>(a, s);
#include "policies_pp.inc"
#undef DBGEMM_SIMT
#undef DBGEMM_MFMA
  return hipErrorInvalidConfiguration;
}

}  // namespace dbgemm
