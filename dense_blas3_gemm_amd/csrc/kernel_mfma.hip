// MFMA GEMM kernels for gfx950 (MI355X).
//
// C = alpha * op(A) * op(B) + beta * C with bf16 or E4M3 operands and fp32
// accumulation.  The steps follow the hot path of the pages' hgemm kernels (the
// "cp.async / ldmatrix ablation" plan, sections 2 and 3: pipelined global->shared
// staging, a bank-conflict-free XOR-swizzled shared layout, shared->register
// fragment loads with an optional transpose, tensor-core MMA into a register
// accumulator tile, and grid swizzle), re-designed for CDNA4:
//
//   * one workgroup computes a BM x BN tile with WM x WN waves of 64 lanes;
//   * global -> LDS: 16-byte buffer loads (bounds handled by the buffer unit:
//     an out-of-range offset reads zeros) into registers, written to one of
//     STAGES LDS buffers while the previous stage feeds the matrix cores;
//   * LDS keeps every operand in its global layout (the contiguous dimension
//     innermost), in 16-byte chunks XOR-swizzled by row;
//   * K-contiguous operands reach the MFMA through ds_read_b128; M- or
//     N-contiguous ones through ds_read_b64_tr_b16 / ds_read_b64_tr_b8, the
//     gfx950 transposing LDS reads, so a transposed operand is never copied;
//   * v_mfma_f32_{32x32x16,16x16x32}_bf16 or v_mfma_f32_{32x32x64,16x16x128}_f8f6f4
//     (E4M3, unit scale) accumulate into fp32 registers;
//   * the epilogue computes alpha*acc + beta*C_old in fp32 and stores bf16 (RNE)
//     or fp32, four consecutive columns per lane.
//
// The MFMA is issued with the B fragment as its first operand, so each lane ends
// up holding four consecutive columns of one row of C (a row-major friendly store).
#include "mfma_common.h"

namespace dbgemm {
namespace {

// Register-staged pipeline: chunk geometry of the global -> register -> LDS copy.
template <class C>
struct Staged {
  static_assert(C::STAGES == 2, "register-staged pipeline: two LDS stages");
  static_assert(C::A_ROWS * C::A_GCPR % C::THREADS == 0 && C::B_ROWS * C::B_GCPR % C::THREADS == 0,
                "chunks per thread");
  static_assert(C::THREADS % C::A_GCPR == 0 && C::THREADS % C::B_GCPR == 0, "a load pass covers whole rows");
};

template <class C>
__global__ __launch_bounds__(C::THREADS) void gemm_mfma_kernel(GemmArgs a) {
  (void)sizeof(Staged<C>);
  __shared__ __attribute__((aligned(1024))) char smem[C::STAGES * C::STAGE_BYTES];
  using Frag = typename FragOf<C::FP8>::T;
  using Acc = typename AccOf<C::MT>::T;

  int tm, tn;
  int split_unused;  // the register-staged kernels run with splits == 1
  tile_of(blockIdx.x, a, tm, tn, split_unused);
  const int m0 = tm * C::BM, n0 = tn * C::BN;
  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  const int wm = wave / C::WN, wn = wave % C::WN;
  const int sw_on = a.swizzle;

  // ---- buffer resources over the whole operands (host guarantees < 2^31 bytes)
  const uint32_t a_rows = C::A_KC ? a.M : a.K;
  const uint32_t b_rows = C::B_KC ? a.N : a.K;
  const __amdgpu_buffer_rsrc_t ra = make_rsrc(a.A, (uint32_t)(a_rows * a.lda * C::GES));
  const __amdgpu_buffer_rsrc_t rb = make_rsrc(a.B, (uint32_t)(b_rows * a.ldb * C::GES));

  // ---- per-thread global chunk coordinates (fixed over the K loop)
  // A global chunk i: tile row t / GCPR + i * (THREADS / GCPR), chunk column t % GCPR;
  // it lands in LDS chunk column (t % GCPR) * WIDEN (and the next one when widened).
  const int a_c = t % C::A_GCPR, a_r0 = t / C::A_GCPR;
  const int b_c = t % C::B_GCPR, b_r0 = t / C::B_GCPR;
  constexpr int A_RSTEP = C::THREADS / C::A_GCPR, B_RSTEP = C::THREADS / C::B_GCPR;

  uint32_t a_goff[C::A_CH], b_goff[C::B_CH];
  uint32_t a_soff[C::A_CH], b_soff[C::B_CH];
  bool a_fixed_ok[C::A_CH], b_fixed_ok[C::B_CH];
#pragma unroll
  for (int i = 0; i < C::A_CH; ++i) {
    const int r = a_r0 + i * A_RSTEP;
    if constexpr (C::A_KC) {  // rows = m, cols = k
      a_goff[i] = (uint32_t)((m0 + r) * a.lda + a_c * C::VEC) * C::GES;
      a_fixed_ok[i] = (m0 + r) < a.M;
    } else {  // rows = k, cols = m
      a_goff[i] = (uint32_t)(r * a.lda + m0 + a_c * C::VEC) * C::GES;
      a_fixed_ok[i] = (m0 + a_c * C::VEC) < a.M;
    }
    const int s = sw_on ? swz<C::A_KC, C::FP8, C::A_CPR, C::MT>(r) : 0;
    a_soff[i] = r * C::A_RB + (((a_c * C::WIDEN) ^ s) << 4);
  }
#pragma unroll
  for (int i = 0; i < C::B_CH; ++i) {
    const int r = b_r0 + i * B_RSTEP;
    if constexpr (C::B_KC) {  // rows = n, cols = k
      b_goff[i] = (uint32_t)((n0 + r) * a.ldb + b_c * C::VEC) * C::GES;
      b_fixed_ok[i] = (n0 + r) < a.N;
    } else {  // rows = k, cols = n
      b_goff[i] = (uint32_t)(r * a.ldb + n0 + b_c * C::VEC) * C::GES;
      b_fixed_ok[i] = (n0 + b_c * C::VEC) < a.N;
    }
    const int s = sw_on ? swz<C::B_KC, C::FP8, C::B_CPR, C::MT>(r) : 0;
    b_soff[i] = C::A_BYTES + r * C::B_RB + (((b_c * C::WIDEN) ^ s) << 4);
  }
  // byte advance of one K tile
  const uint32_t a_kstep = C::A_KC ? C::BK * C::GES : (uint32_t)(C::BK * a.lda * C::GES);
  const uint32_t b_kstep = C::B_KC ? C::BK * C::GES : (uint32_t)(C::BK * a.ldb * C::GES);

  i32x4 a_reg[C::A_CH], b_reg[C::B_CH];
  // block-scaled E4M3: the UE8M0 byte of each chunk (a 16-element chunk of a row lies in
  // one 32-element block); both operands are K-contiguous here
  constexpr bool MX = C::IN == IN_MX;
  static_assert(!MX || (C::A_KC && C::B_KC && C::VEC == 16), "block-scaled operands are K-contiguous E4M3");
  static_assert(!MX || C::A_CH + C::B_CH <= 4, "scale bytes of a tile fit one register");
  static_assert(!MX || C::BK % 32 == 0, "whole scale blocks per K tile");
  uint32_t sc_packed = 0;  // byte i: scale of A chunk i, then of B chunk i - A_CH
  // byte offsets of this thread's scale bytes in K tile 0 (32-bit: the host keeps each
  // scale array below 2^31 bytes); K tile kt adds kt * BK / 32
  uint32_t a_sco[MX ? C::A_CH : 1], b_sco[MX ? C::B_CH : 1];
  if constexpr (MX) {
#pragma unroll
    for (int i = 0; i < C::A_CH; ++i)
      a_sco[i] = (uint32_t)(m0 + a_r0 + i * A_RSTEP) * (uint32_t)a.ldsa + (uint32_t)(a_c * C::VEC / 32);
#pragma unroll
    for (int i = 0; i < C::B_CH; ++i)
      b_sco[i] = (uint32_t)(n0 + b_r0 + i * B_RSTEP) * (uint32_t)a.ldsb + (uint32_t)(b_c * C::VEC / 32);
  }
  const __amdgpu_buffer_rsrc_t rsa = make_rsrc(MX ? a.sa : nullptr, MX ? (uint32_t)(a.M * a.ldsa) : 0u);
  const __amdgpu_buffer_rsrc_t rsb = make_rsrc(MX ? a.sb : nullptr, MX ? (uint32_t)(a.N * a.ldsb) : 0u);

  auto global_load = [&](int kt) {
    const int k0 = kt * C::BK;
#pragma unroll
    for (int i = 0; i < C::A_CH; ++i) {
      const int r = a_r0 + i * A_RSTEP;
      const bool ok = a_fixed_ok[i] & (C::A_KC ? (k0 + a_c * C::VEC < a.K) : (k0 + r < a.K));
      const uint32_t off = ok ? a_goff[i] + (uint32_t)kt * a_kstep : kOOB;
      a_reg[i] = __builtin_amdgcn_raw_buffer_load_b128(ra, off, 0, 0);
      if constexpr (MX) {
        const uint32_t so = ok ? a_sco[i] + (uint32_t)(kt * (C::BK / 32)) : kOOB;
        const uint32_t v = __builtin_amdgcn_raw_buffer_load_b8(rsa, so, 0, 0);
        sc_packed = i == 0 ? v : (sc_packed | (v << (8 * i)));
      }
    }
#pragma unroll
    for (int i = 0; i < C::B_CH; ++i) {
      const int r = b_r0 + i * B_RSTEP;
      const bool ok = b_fixed_ok[i] & (C::B_KC ? (k0 + b_c * C::VEC < a.K) : (k0 + r < a.K));
      const uint32_t off = ok ? b_goff[i] + (uint32_t)kt * b_kstep : kOOB;
      b_reg[i] = __builtin_amdgcn_raw_buffer_load_b128(rb, off, 0, 0);
      if constexpr (MX) {
        const uint32_t so = ok ? b_sco[i] + (uint32_t)(kt * (C::BK / 32)) : kOOB;
        sc_packed |= (uint32_t)__builtin_amdgcn_raw_buffer_load_b8(rsb, so, 0, 0) << (8 * (C::A_CH + i));
      }
    }
  };
  lds_char* const sm = (lds_char*)smem;
  auto lds_store_to = [&](lds_char* sbase) {
#pragma unroll
    for (int i = 0; i < C::A_CH; ++i)
      put_chunk<C>(sbase, a_soff[i], a_reg[i], MX ? ue8m0_value((sc_packed >> (8 * i)) & 0xFFu) : 1.0f);
#pragma unroll
    for (int i = 0; i < C::B_CH; ++i)
      put_chunk<C>(sbase, b_soff[i], b_reg[i],
                   MX ? ue8m0_value((sc_packed >> (8 * (C::A_CH + i))) & 0xFFu) : 1.0f);
  };
  auto lds_store = [&](int stage) { lds_store_to(sm + stage * C::STAGE_BYTES); };

  Acc acc[C::FM][C::FN];
#pragma unroll
  for (int i = 0; i < C::FM; ++i)
#pragma unroll
    for (int j = 0; j < C::FN; ++j) acc[i][j] = Acc{};

  const int nk = (a.K + C::BK - 1) / C::BK;
  const int xa0 = wm * C::WTM, xb0 = wn * C::WTN;

  // ---- main loop.  Two LDS stages: while tile kt is consumed from stage kt&1, tile
  // kt+1 travels global -> registers -> stage (kt+1)&1.  Past the last tile the global
  // loads see only out-of-range offsets, read zeros and touch no memory, so the loop
  // body is one basic block that the instruction scheduling hints below can order.
  Frag fa[2][C::FM], fb[2][C::FN];
  auto read_step = [&](const lds_char* sb, int kk, Frag* xa, Frag* xb) {
#pragma unroll
    for (int i = 0; i < C::FM; ++i)
      xa[i] = load_frag<C, C::A_KC, C::A_RB>(sb, xa0 + i * C::MT, kk * C::KT, lane, sw_on);
#pragma unroll
    for (int j = 0; j < C::FN; ++j)
      xb[j] = load_frag<C, C::B_KC, C::B_RB>(sb + C::A_BYTES, xb0 + j * C::MT, kk * C::KT, lane, sw_on);
  };

  global_load(0);
  lds_store(0);
  __syncthreads();
  read_step(sm, 0, fa[0], fb[0]);

  for (int kt = 0; kt < nk; ++kt) {
    const lds_char* cur = sm + (kt & 1) * C::STAGE_BYTES;
    lds_char* nxt = sm + ((kt + 1) & 1) * C::STAGE_BYTES;
    global_load(kt + 1);
    static_for<C::KSTEPS>([&](auto kkc) {
      constexpr int kk = decltype(kkc)::value;
      // the reads of step kk+1 (or, in the last step, the writes of the next tile)
      // are issued between this step's MFMAs
      if constexpr (kk + 1 < C::KSTEPS) {
        read_step(cur, kk + 1, fa[(kk + 1) & 1], fb[(kk + 1) & 1]);
      } else {
        lds_store_to(nxt);
      }
#pragma unroll
      for (int i = 0; i < C::FM; ++i)
#pragma unroll
        for (int j = 0; j < C::FN; ++j) mma(acc[i][j], fb[kk & 1][j], fa[kk & 1][i]);
      constexpr int nmf = C::FM * C::FN;
      constexpr int nds = kk + 1 < C::KSTEPS ? C::DS_READS_PER_STEP : 0;
      constexpr int nvm = kk == 0 ? (C::A_CH + C::B_CH) * (MX ? 2 : 1) : 0;  // + the scale bytes
      constexpr int ndw = kk + 1 < C::KSTEPS ? 0 : (C::A_CH + C::B_CH) * C::WIDEN;
      interleave<nmf, nds, nvm, ndw>();
      __builtin_amdgcn_sched_barrier(0);  // nothing crosses a K-step boundary
    });
    __syncthreads();
    read_step(nxt, 0, fa[0], fb[0]);
  }

  store_tile<C>(a, acc, m0 + xa0, n0 + xb0, lane);
}

template <class C>
hipError_t launch_cfg(const GemmArgs& a, hipStream_t s) {
  hipLaunchKernelGGL(gemm_mfma_kernel<C>, dim3(grid_tiles(a)), dim3(C::THREADS), 0, s, a);
  return hipGetLastError();
}

#if !defined(DBGEMM_DMA_TA) || !defined(DBGEMM_DMA_TB)
#error "compile with -DDBGEMM_DMA_TA=0|1 -DDBGEMM_DMA_TB=0|1"
#endif

// This object's transpose case (the file is compiled once per case).
template <int BM, int BN, int BK, int WM, int WN, int MT, int ST, int IN>
hipError_t launch_trans(const GemmArgs& a, hipStream_t s) {
  constexpr bool TA = DBGEMM_DMA_TA != 0, TB = DBGEMM_DMA_TB != 0;
  if constexpr (IN == IN_MX && (TA || !TB)) {  // block-scaled operands: A [M][K] and B [N][K] only
    return hipErrorInvalidConfiguration;
  } else {
    return launch_cfg<Cfg<BM, BN, BK, WM, WN, MT, ST, IN, TA, TB>>(a, s);
  }
}

}  // namespace

#define DBGEMM_ST_CAT2(a, b) launch_mfma_staged_##a##b
#define DBGEMM_ST_CAT(a, b) DBGEMM_ST_CAT2(a, b)

hipError_t DBGEMM_ST_CAT(DBGEMM_DMA_TA, DBGEMM_DMA_TB)(const Policy& p, const GemmArgs& a, hipStream_t s) {
#define DBGEMM_SIMT(name, eff)
#define DBGEMM_MFMA(name_, pipe_, in_, bm_, bn_, bk_, wm_, wn_, mt_, st_, grp_, rn_, xcd_, sw_, eff_)       \
  if constexpr (pipe_ == 0)                                                                               \
    if (p.BM == bm_ && p.BN == bn_ && p.BK == bk_ && p.WM == wm_ && p.WN == wn_ && p.MT == mt_ &&         \
        p.stages == st_ && p.in_mode == in_ && p.read_mode == 1)                                          \
      return launch_trans<bm_, bn_, bk_, wm_, wn_, mt_, st_, in_>(a, s);
#include "policies.inc"
#undef DBGEMM_SIMT
#undef DBGEMM_MFMA
  return hipErrorInvalidConfiguration;
}

}  // namespace dbgemm
