// MFMA GEMM kernels for gfx950 with direct-to-LDS operand staging.
//
// Same operation, LDS layout, fragment reads, MFMA and epilogue as the register-
// staged kernels (mfma_common.h), but the global -> LDS copy goes through the
// gfx950 buffer-load-to-LDS path: one `buffer_load_dwordx4 ... lds` moves 64 x 16
// bytes from 64 independently addressed global chunks into 1 KiB of contiguous LDS
// (lane i -> M0 + 16*i), without passing through vector registers.  This is the
// CDNA4 counterpart of the pages' asynchronous global->shared copies (the
// "cp.async / ldmatrix ablation" plan, sections 0.2 and 1: copy groups, per-stage
// completion tracking, multi-stage buffering), re-designed around what gfx950 has:
//
//   * a ring of STAGES LDS buffers; stage t+STAGES is loaded while stage t is
//     consumed, so loads run STAGES-1 K tiles ahead of the matrix cores;
//   * the LDS XOR swizzle is applied on the load side: the lane that fills LDS
//     chunk p fetches the global chunk that the swizzle maps to p;
//   * completion is tracked per wave with `s_waitcnt vmcnt(N)` counting the
//     loads still in flight, followed by one workgroup barrier per K tile;
//   * the barrier of tile t+1 is taken before the last K step of tile t, so the
//     first fragments of tile t+1 are read while tile t's last MFMAs execute.
//
// The cross-wave wait is explicit (`s_waitcnt vmcnt` + `s_barrier`); within a wave the
// compiler also orders each LDS read after the loads into the same ring slot.
#include "mfma_common.h"

namespace dbgemm {
namespace {

// 64 lanes x 16 bytes from buffer `rsrc` at per-lane byte offset `voff` into LDS
// bytes [lds_base, lds_base + 1024) (lane i -> lds_base + 16*i); an offset past the
// buffer's size reads zeros.  Issued as assembly: the compiler neither sees nor waits
// for these loads (it could not tell them apart from the LDS reads of other ring
// slots), so every wait on them below is explicit.  M0 carries the LDS address: the
// statement saves and restores it (the compiler reserves M0 and does not honour it as
// a clobber), and one wait state separates its write from the load that reads it.
__device__ __forceinline__ void load_to_lds(uint32_t lds_base, uint32_t voff, __amdgpu_buffer_rsrc_t rsrc) {
  uint32_t saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %1\n\t"
      "s_nop 0\n\t"
      "buffer_load_dwordx4 %2, %3, 0 offen lds\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(saved)
      : "s"(lds_base), "v"(voff), "s"(rsrc)
      : "memory");
}

// 64 lanes x 4 bytes from buffer `rsrc` at per-lane byte offset `voff` into LDS bytes
// [lds_base, lds_base + 256) (lane i -> lds_base + 4*i); an offset past the buffer reads 0.
// M0 as in load_to_lds.
__device__ __forceinline__ void load_to_lds_dword(uint32_t lds_base, uint32_t voff, __amdgpu_buffer_rsrc_t rsrc) {
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

// Waits until at most N of this wave's buffer loads are in flight and all its LDS
// reads have returned, then joins the workgroup barrier.
template <int N>
__device__ __forceinline__ void wait_loads_and_barrier() {
  asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)\n\ts_barrier" : : "n"(N) : "memory");
}

template <class C>
struct Dma {
  static_assert(C::IN != IN_E4M3, "widening needs the register-staged pipeline");
  static_assert(C::GES == C::ES, "LDS holds the global format");
  static constexpr int NW = C::THREADS / 64;
  static_assert(C::A_BYTES % (1024 * NW) == 0 && C::B_BYTES % (1024 * NW) == 0,
                "each wave loads whole 1 KiB blocks of both tiles");
  static constexpr int A_IPW = C::A_BYTES / 1024 / NW;  // load instructions per wave per tile
  static constexpr int B_IPW = C::B_BYTES / 1024 / NW;
  // scaled native E4M3: each wave also loads the scale words of 64 tile rows
  static_assert(!C::MXN || (C::BM + C::BN) / 64 == NW, "one 64-row block of scale words per wave");
  static constexpr int SC_IPW = C::MXN ? 1 : 0;
  static constexpr int IPW = A_IPW + B_IPW + SC_IPW;
  static_assert(C::STAGES >= 2 && C::STAGES <= 4, "two to four LDS stages");
  static_assert((C::STAGES - 1) * IPW <= 63, "vmcnt range");
  static_assert(C::KSTEPS >= 2 && C::KSTEPS % 2 == 0,
                "an even number (>= 2) of K steps per tile: loads ride on the first steps");
  // the loads of one tile are spread over the first KSTEPS-1 steps of the tile before
  static constexpr int LOAD_STEPS = C::KSTEPS - 1;
  static constexpr int loads_before(int kk) { return IPW * kk / LOAD_STEPS; }
};

template <class C>
__global__ __launch_bounds__(C::THREADS) void gemm_dma_kernel(GemmArgs a) {
  using D = Dma<C>;
  // One LDS object per ring slot: the compiler tracks the loads into each slot on
  // its own, so its automatic waits before LDS reads wait for that slot only.
  __shared__ __attribute__((aligned(1024))) char lds_s0[C::STAGE_BYTES];
  __shared__ __attribute__((aligned(1024))) char lds_s1[C::STAGE_BYTES];
  __shared__ __attribute__((aligned(1024))) char lds_s2[C::STAGES > 2 ? C::STAGE_BYTES : 16];
  __shared__ __attribute__((aligned(1024))) char lds_s3[C::STAGES > 3 ? C::STAGE_BYTES : 16];
  auto slot = [&](auto sc) -> lds_char* {
    constexpr int s = decltype(sc)::value;
    if constexpr (s == 0) return (lds_char*)lds_s0;
    else if constexpr (s == 1) return (lds_char*)lds_s1;
    else if constexpr (s == 2) return (lds_char*)lds_s2;
    else return (lds_char*)lds_s3;
  };
  using Frag = typename FragOf<C::FP8>::T;
  using Acc = typename AccOf<C::MT>::T;

  if (a.batch_y > 1 || a.batch_z > 1) {  // this workgroup's product of the batch
    const int64_t y = blockIdx.y, z = blockIdx.z;
    const int c_es = a.c_kind == C_F32 ? 4 : a.c_kind == C_BF16 ? 2 : 1;
    a.A = (const char*)a.A + (y * a.bsA[0] + z * a.bsA[1]) * C::ES;
    a.B = (const char*)a.B + (y * a.bsB[0] + z * a.bsB[1]) * C::ES;
    a.C = (char*)a.C + (y * a.bsC[0] + z * a.bsC[1]) * c_es;
  }
  int tm, tn, split;
  tile_of(blockIdx.x, a, tm, tn, split);
  const int m0 = tm * C::BM, n0 = tn * C::BN;
  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  const int wm = wave / C::WN, wn = wave % C::WN;
  const int sw_on = a.swizzle;

  const uint32_t a_rows = C::A_KC ? a.M : a.K;
  const uint32_t b_rows = C::B_KC ? a.N : a.K;
  const __amdgpu_buffer_rsrc_t ra = make_rsrc(a.A, (uint32_t)(a_rows * a.lda * C::ES));
  const __amdgpu_buffer_rsrc_t rb = make_rsrc(a.B, (uint32_t)(b_rows * a.ldb * C::ES));
  // Two products in one sum (the rank-2K update), in the bf16 A [M][K], B [N][K]
  // instantiations only: their register budget has room for the second pair of buffer
  // descriptors, which pushed the transposed-A 256 x 256 tile (and the scaled-E4M3 one) into
  // scratch.  Same strides as (A, B).
  constexpr bool kDual = !C::TA && C::TB && C::IN == IN_BF16;
  const __amdgpu_buffer_rsrc_t ra2 = kDual ? make_rsrc(a.dual ? a.A2 : a.A, (uint32_t)(a_rows * a.lda * C::ES)) : ra;
  const __amdgpu_buffer_rsrc_t rb2 = kDual ? make_rsrc(a.dual ? a.B2 : a.B, (uint32_t)(b_rows * a.ldb * C::ES)) : rb;

  // ---- per-lane sources of the load instructions (fixed over the K loop).
  // Instruction i of this wave fills LDS block blk = wave*IPW + i of the tile; this
  // lane fills chunk p = blk*64 + lane, i.e. row p / CPR and physical chunk p % CPR,
  // which holds logical chunk (p % CPR) ^ swizzle(row).
  uint32_t a_goff[D::A_IPW], b_goff[D::B_IPW];
  int a_kc[D::A_IPW], b_kc[D::B_IPW];  // K index of this lane's chunk within a tile
  bool a_ok[D::A_IPW], b_ok[D::B_IPW];
#pragma unroll
  for (int i = 0; i < D::A_IPW; ++i) {
    const int p = (wave * D::A_IPW + i) * 64 + lane;
    const int r = p / C::A_CPR;
    const int c = (p % C::A_CPR) ^ (sw_on ? swz<C::A_KC, C::FP8, C::A_CPR, C::MT>(r) : 0);
    if constexpr (C::A_KC) {  // rows = m, chunks along k
      a_goff[i] = (uint32_t)((m0 + r) * a.lda + c * C::VEC) * C::ES;
      a_ok[i] = (m0 + r) < a.M;
      a_kc[i] = c * C::VEC;
    } else {  // rows = k, chunks along m
      a_goff[i] = (uint32_t)(r * a.lda + m0 + c * C::VEC) * C::ES;
      a_ok[i] = (m0 + c * C::VEC) < a.M;
      a_kc[i] = r;
    }
  }
#pragma unroll
  for (int i = 0; i < D::B_IPW; ++i) {
    const int p = (wave * D::B_IPW + i) * 64 + lane;
    const int r = p / C::B_CPR;
    const int c = (p % C::B_CPR) ^ (sw_on ? swz<C::B_KC, C::FP8, C::B_CPR, C::MT>(r) : 0);
    if constexpr (C::B_KC) {  // rows = n, chunks along k
      b_goff[i] = (uint32_t)((n0 + r) * a.ldb + c * C::VEC) * C::ES;
      b_ok[i] = (n0 + r) < a.N;
      b_kc[i] = c * C::VEC;
    } else {  // rows = k, chunks along n
      b_goff[i] = (uint32_t)(r * a.ldb + n0 + c * C::VEC) * C::ES;
      b_ok[i] = (n0 + c * C::VEC) < a.N;
      b_kc[i] = r;
    }
  }
  const uint32_t a_kstep = C::A_KC ? C::BK * C::ES : (uint32_t)(C::BK * a.lda * C::ES);
  const uint32_t b_kstep = C::B_KC ? C::BK * C::ES : (uint32_t)(C::BK * a.ldb * C::ES);

  // ---- scaled native E4M3: this wave's scale words (rows wave*64 + lane of A's tile, or
  // of B's for the upper waves); K tile kt reads the word at byte kt*4 of the row.  Rows
  // past M or N read zeros; tiles past K read whatever follows, all of it masked below.
  const int wave_u = __builtin_amdgcn_readfirstlane(wave);
  const bool sc_is_a = wave_u < C::BM / 64;
  const int sc_w = sc_is_a ? wave_u : wave_u - C::BM / 64;
  const int sc_r = (sc_is_a ? m0 : n0) + sc_w * 64 + lane;
  const uint32_t sc_goff =
      !C::MXN || sc_r >= (sc_is_a ? a.M : a.N) ? kOOB : (uint32_t)(sc_r * (sc_is_a ? a.ldsa : a.ldsb));
  const uint32_t sc_lds = (uint32_t)C::SC_OFF + (uint32_t)((sc_is_a ? 0 : C::A_SC_BYTES) + sc_w * 256);
  const __amdgpu_buffer_rsrc_t rsa = make_rsrc(C::MXN ? a.sa : nullptr, C::MXN ? (uint32_t)(a.M * a.ldsa) : 0u);
  const __amdgpu_buffer_rsrc_t rsb = make_rsrc(C::MXN ? a.sb : nullptr, C::MXN ? (uint32_t)(a.N * a.ldsb) : 0u);
  const int nb = (a.K + 31) / 32;  // scale blocks along K

  // Loads instructions [lo, hi) of K tile kt (A blocks first, then B) into slot sb.
  // Past the end of K every offset is out of range: the loads read zeros and touch no
  // memory.
  const uint32_t a_blk = (uint32_t)(wave * D::A_IPW) * 1024u;
  const uint32_t b_blk = C::A_BYTES + (uint32_t)(wave * D::B_IPW) * 1024u;
  // K tiles of this workgroup: [kbeg, kbeg + nk) of the nk_all tiles of K.  A dual call
  // walks 2 * nk_k tiles, the second nk_k on (A2, B2).  A K band keeps only the tiles that
  // meet the band (the rest multiply zeros).
  const int nk_k = (a.K + C::BK - 1) / C::BK;
  const int nk_all = kDual && a.dual ? 2 * nk_k : nk_k;
  int kbeg = split * a.kt_per_split;
  int nk = a.splits > 1 ? min(nk_all - kbeg, a.kt_per_split) : nk_all;
  if (C::IN == IN_BF16 && a.kband != KBAND_NONE) {  // K bands: bf16 calls only
    int lo = 0, hi = a.K;  // elements of K
    if (a.kband == KBAND_A_LOWER) hi = min(a.K, a.band_off + (tm + 1) * C::BM);
    if (a.kband == KBAND_A_UPPER) lo = min(a.K, a.band_off + tm * C::BM);
    if (a.kband == KBAND_B_LOWER) lo = min(a.K, a.band_off + tn * C::BN);
    if (a.kband == KBAND_B_UPPER) hi = min(a.K, a.band_off + (tn + 1) * C::BN);
    kbeg = lo / C::BK;
    nk = max(0, (hi + C::BK - 1) / C::BK - kbeg);
  }
  // K-loop rotation: with krot set, the workgroups of XCD x (ids x, x+8, ...) walk K
  // starting at tile x*nk/8 and wrap around, so the eight XCDs stream different parts
  // of A and B at any moment instead of the same power-of-two-strided addresses.  The
  // workgroups of one XCD stay in step and keep sharing its L2.  (This changes only
  // the order of the K tiles in each sum.)
  const int krot = a.krot && a.splits == 1 ? (int)((blockIdx.x % 8) * nk / 8) : 0;
  // Load instruction q (A blocks first, then B) of logical K tile u into slot sb;
  // logical tiles past the end stay past the end (zeros).
  auto issue_one = [&](const lds_char* sb, int u, auto qc) {
    constexpr int q = decltype(qc)::value;
    int kt = u < nk ? kbeg + u : nk_all;  // past this workgroup's range: past K (zeros)
    if (krot != 0 && u < nk) kt = u + krot < nk ? u + krot : u + krot - nk;
    // a dual call's second product: tiles nk_k .. 2*nk_k - 1 are K tiles of (A2, B2); the
    // past-the-end marker 2*nk_k becomes K tile nk_k, past K as well
    const bool second = kDual && a.dual && kt >= nk_k;
    if (second) kt -= nk_k;
    const int k0 = kt * C::BK;
    const uint32_t base = (uint32_t)(uintptr_t)sb;
    if constexpr (C::MXN && q == D::IPW - 1) {
      load_to_lds_dword(base + sc_lds, sc_goff + (uint32_t)kt * 4u, sc_is_a ? rsa : rsb);
    } else if constexpr (q < D::A_IPW) {
      const bool ok = a_ok[q] & (k0 + a_kc[q] < a.K);
      load_to_lds(__builtin_amdgcn_readfirstlane(base + a_blk + q * 1024u),
                  ok ? a_goff[q] + (uint32_t)kt * a_kstep : kOOB, second ? ra2 : ra);
    } else {
      constexpr int i = q - D::A_IPW;
      const bool ok = b_ok[i] & (k0 + b_kc[i] < a.K);
      load_to_lds(__builtin_amdgcn_readfirstlane(base + b_blk + i * 1024u),
                  ok ? b_goff[i] + (uint32_t)kt * b_kstep : kOOB, second ? rb2 : rb);
    }
  };

  Acc acc[C::FM][C::FN];
#pragma unroll
  for (int i = 0; i < C::FM; ++i)
#pragma unroll
    for (int j = 0; j < C::FN; ++j) acc[i][j] = Acc{};

  const int xa0 = wm * C::WTM, xb0 = wn * C::WTN;

  Frag fa[2][C::FM], fb[2][C::FN];
  // Fragment r of K step kk, in the order the MFMAs first use them (the MFMAs run
  // A-fragment-major): A0, B0 .. B(FN-1), then A1 .. A(FM-1).
  auto read_one = [&](const lds_char* sb, int kk, Frag* xa, Frag* xb, auto rc) {
    constexpr int r = decltype(rc)::value;
    constexpr bool is_b = r >= 1 && r <= C::FN;
    constexpr int idx = r == 0 ? 0 : (is_b ? r - 1 : r - C::FN);
    if constexpr (!is_b)
      xa[idx] = load_frag<C, C::A_KC, C::A_RB>(sb, xa0 + idx * C::MT, kk * C::KT, lane, sw_on);
    else
      xb[idx] = load_frag<C, C::B_KC, C::B_RB>(sb + C::A_BYTES, xb0 + idx * C::MT, kk * C::KT, lane, sw_on);
  };
  auto read_step = [&](const lds_char* sb, int kk, Frag* xa, Frag* xb) {
#pragma unroll
    for (int i = 0; i < C::FM; ++i)
      xa[i] = load_frag<C, C::A_KC, C::A_RB>(sb, xa0 + i * C::MT, kk * C::KT, lane, sw_on);
#pragma unroll
    for (int j = 0; j < C::FN; ++j)
      xb[j] = load_frag<C, C::B_KC, C::B_RB>(sb + C::A_BYTES, xb0 + j * C::MT, kk * C::KT, lane, sw_on);
  };

  // Scaled native E4M3: the scale bytes this lane's MFMAs take, one register per two
  // fragments and one set per tile parity (two LDS stages).  A tile row's LDS word holds
  // its four 32-wide K blocks; the lane's K half h takes blocks h (step 0) and 2 + h
  // (step 1), so fragment f of a pair sits at bytes 2f (step 0) and 2f + 1 (step 1).
  // Blocks past K, which meet zero-filled elements, read as 127 (x1), so that whatever
  // the caller left in the scale rows' padding cannot bring a NaN or an overflow.
  static_assert(!C::MXN || (C::FM % 2 == 0 && C::FN % 2 == 0), "fragments pair up for the scales");
  constexpr int SCA = C::MXN ? C::FM / 2 : 1, SCB = C::MXN ? C::FN / 2 : 1;
  int scA[2][SCA], scB[2][SCB];
  auto read_scales = [&](const lds_char* sb, int u, auto bc) {
    if constexpr (C::MXN) {
      constexpr int b = decltype(bc)::value;
      int kt = u < nk ? kbeg + u : nk_all;  // the K tile issue_one loaded for u
      if (krot != 0 && u < nk) kt = u + krot < nk ? u + krot : u + krot - nk;
      const int blk = kt * 4 + (lane >> 5);
      const uint32_t m = (blk >= nb ? 0x00FF00FFu : 0u) | (blk + 2 >= nb ? 0xFF00FF00u : 0u);
      const uint32_t sh = 8u * (uint32_t)(lane >> 5);
      auto pair = [&](int off) {
        const uint32_t w0 = *LDS_PTR(uint32_t, sb, off) >> sh;
        const uint32_t w1 = *LDS_PTR(uint32_t, sb, off + C::MT * 4) >> sh;
        const uint32_t v = __builtin_amdgcn_perm(w1, w0, 0x06040200u);  // w0.b0 w0.b2 w1.b0 w1.b2
        return (int)((v & ~m) | (0x7F7F7F7Fu & m));
      };
#pragma unroll
      for (int i = 0; i < SCA; ++i) scA[b][i] = pair(C::SC_OFF + (xa0 + 2 * i * C::MT + (lane & 31)) * 4);
#pragma unroll
      for (int j = 0; j < SCB; ++j)
        scB[b][j] = pair(C::SC_OFF + C::A_SC_BYTES + (xb0 + 2 * j * C::MT + (lane & 31)) * 4);
    }
  };

  // ---- prologue: tiles 0 .. STAGES-2 into slots 0 .. STAGES-2; wait for tile 0
  static_for<C::STAGES - 1>([&](auto sc) {
    static_for<D::IPW>([&](auto qc) { issue_one(slot(sc), decltype(sc)::value, qc); });
  });
  wait_loads_and_barrier<(C::STAGES - 2) * D::IPW>();
  read_step(slot(std::integral_constant<int, 0>{}), 0, fa[0], fb[0]);
  read_scales(slot(std::integral_constant<int, 0>{}), 0, std::integral_constant<int, 0>{});

  // ---- main loop.  Tile u lives in slot u % STAGES.  During tile u's first K steps
  // the loads of tile u+STAGES-1 go into slot (u-1) % STAGES, which every wave left at
  // the barrier of tile u-1.  In tile u's last step each wave waits for its loads of
  // tile u+1, the barrier makes all of them visible, and the first fragments of tile
  // u+1 are read while tile u's last MFMAs run.  The loop runs over whole rings;
  // tiles past the end of K are all zeros and add nothing.
  for (int kt0 = 0; kt0 < nk; kt0 += C::STAGES) {
    static_for<C::STAGES>([&](auto sc) {
      constexpr int s = decltype(sc)::value;
      const int u = kt0 + s;
      const lds_char* cur = slot(sc);
      const lds_char* nxt = slot(std::integral_constant<int, (s + 1) % C::STAGES>{});
      lds_char* fill = slot(std::integral_constant<int, (s + C::STAGES - 1) % C::STAGES>{});
      static_for<C::KSTEPS>([&](auto kkc) {
        constexpr int kk = decltype(kkc)::value;
        constexpr bool last = kk + 1 == C::KSTEPS;
        constexpr int NMF = C::FM * C::FN;
        constexpr int NRF = C::FM + C::FN;
        // the barrier of the last step comes after its first quarter of MFMAs, which
        // keep the matrix core busy while the workgroup gathers
        constexpr int BAR_AT = last ? (NMF + 3) / 4 : -1;
        constexpr int RD0 = last ? BAR_AT : 0;  // reads start after the barrier
        constexpr int LD0 = kk < D::LOAD_STEPS ? D::loads_before(kk) : 0;
        constexpr int NLD = kk < D::LOAD_STEPS ? D::loads_before(kk + 1) - LD0 : 0;
        Frag* ra_next = fa[(kk + 1) & 1];
        Frag* rb_next = fb[(kk + 1) & 1];
        const lds_char* rsrc_slot = last ? nxt : cur;
        const int rkk = last ? 0 : kk + 1;
        // Explicit order: MFMA i, then its share of the fragment reads for the next
        // step and of the loads for tile u+STAGES-1; nothing is moved across a group.
        static_for<NMF>([&](auto ic) {
          constexpr int i = decltype(ic)::value;
          if constexpr (i == BAR_AT) {
            wait_loads_and_barrier<(C::STAGES - 2) * D::IPW>();
            read_scales(nxt, u + 1, std::integral_constant<int, (s + 1) & 1>{});
          }
          if constexpr (C::MXN)
            mma_mx<2 * (i % C::FN % 2) + kk, 2 * (i / C::FN % 2) + kk>(
                acc[i / C::FN][i % C::FN], fb[kk & 1][i % C::FN], fa[kk & 1][i / C::FN],
                scB[s & 1][i % C::FN / 2], scA[s & 1][i / C::FN / 2]);
          else
            mma(acc[i / C::FN][i % C::FN], fb[kk & 1][i % C::FN], fa[kk & 1][i / C::FN]);
          if constexpr (i >= RD0) {
            constexpr int r0 = NRF * (i - RD0) / (NMF - RD0), r1 = NRF * (i + 1 - RD0) / (NMF - RD0);
            static_for<r1 - r0>([&](auto jc) {
              read_one(rsrc_slot, rkk, ra_next, rb_next, std::integral_constant<int, r0 + decltype(jc)::value>{});
            });
          }
          constexpr int l0 = LD0 + NLD * i / NMF, l1 = LD0 + NLD * (i + 1) / NMF;
          static_for<l1 - l0>([&](auto qc) {
            issue_one(fill, u + C::STAGES - 1, std::integral_constant<int, l0 + decltype(qc)::value>{});
          });
          __builtin_amdgcn_sched_barrier(0);
        });
      });
    });
  }
  // drain the loads of the tiles past the end before the workgroup's LDS is released
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");

  if (a.splits > 1) {  // split-K: this split's fp32 partial, summed by split_reduce_kernel
    const int tile = tm * a.tiles_n + tn;
    store_partial<C>(a.ws + ((size_t)tile * a.splits + split) * (C::BM * C::BN), acc, t);
    return;
  }
  store_tile<C>(a, acc, m0 + xa0, n0 + xb0, lane);
}

// Split-K, second launch on the same stream: C <- alpha * (P_0 + ... + P_{S-1}) +
// beta * C with the partials added in split order, so the result does not depend on
// which split finished first.  Workgroup (tile, c) handles float4 groups
// [c*CH, (c+1)*CH) of every thread of the tile's partials; the kernel boundary
// makes the first launch's partials visible, whichever XCD wrote them.
template <class C>
struct Reduce {
  static constexpr int NP = C::FM * C::FN * C::ACC / 4;  // float4 groups per thread
  static constexpr int CH = NP < 2 ? NP : 2;
  static constexpr int CHUNKS = NP / CH;
  static_assert(NP % CH == 0, "whole chunks");
};

template <class C>
__global__ __launch_bounds__(C::THREADS) void split_reduce_kernel(GemmArgs a) {
  using Rd = Reduce<C>;
  const int tile = blockIdx.x / Rd::CHUNKS, c0 = (blockIdx.x % Rd::CHUNKS) * Rd::CH;
  const int tm = tile / a.tiles_n, tn = tile % a.tiles_n;
  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  const int wm = wave / C::WN, wn = wave % C::WN;
  const f32x4* src = (const f32x4*)(a.ws + (size_t)tile * a.splits * (C::BM * C::BN));
  const size_t stride = (size_t)Rd::NP * C::THREADS;  // float4s per partial
  f32x4 v[Rd::CH];
#pragma unroll
  for (int c = 0; c < Rd::CH; ++c) v[c] = src[(c0 + c) * C::THREADS + t];
  for (int s = 1; s < a.splits; ++s) {
#pragma unroll
    for (int c = 0; c < Rd::CH; ++c) v[c] += src[s * stride + (c0 + c) * C::THREADS + t];
  }
#pragma unroll
  for (int c = 0; c < Rd::CH; ++c)
    store_group<C>(a, v[c], c0 + c, tm * C::BM + wm * C::WTM, tn * C::BN + wn * C::WTN, lane);
}

template <class C>
hipError_t launch_cfg(const GemmArgs& a, hipStream_t s) {
  const int ntiles = a.tiles_m * a.tiles_n;
  const unsigned by = a.batch_y > 1 ? (unsigned)a.batch_y : 1u, bz = a.batch_z > 1 ? (unsigned)a.batch_z : 1u;
  hipLaunchKernelGGL(gemm_dma_kernel<C>, dim3(grid_tiles(a), by, bz), dim3(C::THREADS), 0, s, a);
  if (a.splits > 1) {
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(split_reduce_kernel<C>, dim3(ntiles * Reduce<C>::CHUNKS), dim3(C::THREADS), 0, s, a);
  }
  return hipGetLastError();
}

// This file is compiled once per transpose case (DBGEMM_DMA_TA, DBGEMM_DMA_TB) and half of
// the policy table (DBGEMM_DMA_PART: the entries on even or odd lines of policies.inc), so
// the eight groups of kernel instantiations build in parallel.
#if !defined(DBGEMM_DMA_TA) || !defined(DBGEMM_DMA_TB) || !defined(DBGEMM_DMA_PART)
#error "compile with -DDBGEMM_DMA_TA=0|1 -DDBGEMM_DMA_TB=0|1 -DDBGEMM_DMA_PART=0|1"
#endif

}  // namespace

#define DBGEMM_DMA_CAT2(a, b, c) launch_mfma_dma_##a##b##_p##c
#define DBGEMM_DMA_CAT(a, b, c) DBGEMM_DMA_CAT2(a, b, c)

// Launches policy p if this part of the table instantiates its geometry (*err is the launch
// status); returns false, with nothing enqueued, otherwise.
bool DBGEMM_DMA_CAT(DBGEMM_DMA_TA, DBGEMM_DMA_TB, DBGEMM_DMA_PART)(const Policy& p, const GemmArgs& a, hipStream_t s,
                                                                   hipError_t* err) {
#define DBGEMM_SIMT(name, eff)
#define DBGEMM_MFMA(name_, pipe_, in_, bm_, bn_, bk_, wm_, wn_, mt_, st_, grp_, rn_, xcd_, sw_, eff_)       \
  if constexpr (pipe_ == 1 && __LINE__ % 2 == DBGEMM_DMA_PART &&                                          \
                ((in_ != 4 && !(((sw_) >> 3) & 1)) || (DBGEMM_DMA_TA == 0 && DBGEMM_DMA_TB == 1)))        \
    if (p.BM == bm_ && p.BN == bn_ && p.BK == bk_ && p.WM == wm_ && p.WN == wn_ && p.MT == mt_ &&         \
        p.stages == st_ && p.in_mode == in_ && p.read_mode == ((((sw_) >> 2) & 1) ? 0 : 1)) {             \
      *err = launch_cfg<Cfg<bm_, bn_, bk_, wm_, wn_, mt_, st_, in_, DBGEMM_DMA_TA != 0, DBGEMM_DMA_TB != 0,  \
                            (((sw_) >> 2) & 1) ? 0 : 1>>(a, s);                                           \
      return true;                                                                                        \
    }
#include "policies.inc"
#undef DBGEMM_SIMT
#undef DBGEMM_MFMA
  return false;
}

}  // namespace dbgemm
