// Shape-driven tile-policy table and its wave-time model.
//
// The fused profile protocol's GEMM policies (sections "fixed sampling flow" and the
// QKV command: tile policies named by BM x BN, a `wave_time_model` auto policy, raster
// m/n and swizzle 1/2/4/8 knobs, environment overrides used only to pin a policy for
// ablation) are the model here.  On MI355X a "wave" is one round of workgroups over
// the 256 CUs: a grid of T tiles with `occ` resident workgroups per CU takes
// ceil(T / (CUs * occ)) rounds, each as long as one CU needs for `occ` tiles.
#include <cstring>

#include "gemm_internal.h"

namespace dbgemm {
namespace {

const Policy kTable[] = {
#define DBGEMM_SIMT(name_, eff_) {name_, KIND_SIMT, 0, -1, 64, 64, 16, 1, 1, 0, 1, 1, 0, 1, 0, 0, 1, 256, eff_, 0, 0},
#define DBGEMM_MFMA(name_, pipe_, in_, bm_, bn_, bk_, wm_, wn_, mt_, st_, grp_, rn_, xcd_, sw_, eff_) \
  {name_, KIND_MFMA, pipe_, in_, bm_, bn_, bk_, wm_, wn_, mt_, st_, grp_, rn_, xcd_, (sw_) & 1,        \
   ((sw_) >> 1) & 1, ((sw_) >> 2) & 1 ? 0 : 1, (wm_) * (wn_) * 64, eff_, ((sw_) >> 3) & 1, ((sw_) >> 4) & 1},
#include "policies.inc"
#include "policies_pp.inc"
#undef DBGEMM_SIMT
#undef DBGEMM_MFMA
};
constexpr int kCount = sizeof(kTable) / sizeof(kTable[0]);

// Resident workgroups per CU: bounded by LDS (160 KiB) and by the unified register
// file (512 registers per lane per SIMD shared by the waves on that SIMD).
int occupancy(const Policy& p) {
  const int es = (p.in_mode == 2 || p.in_mode >= 4) ? 1 : 2;  // bytes per element in LDS
  const int lds = p.stages * (p.BM + p.BN) * p.BK * es;
  const int staging = p.pipe == 0 ? (p.BM + p.BN) * p.BK * (p.in_mode == 0 ? 2 : 1) / (p.WM * p.WN * 64) / 4 : 0;
  int occ_lds = (160 * 1024) / lds;
  const int acc = (p.BM / p.WM) * (p.BN / p.WN) / 64;  // fp32 accumulators per lane
  const int regs = acc + 96 + staging;                   // + fragments, addresses, load staging
  const int waves_per_simd = 512 / regs;
  const int wg_waves_per_simd = (p.WM * p.WN + 3) / 4;
  int occ_reg = waves_per_simd / wg_waves_per_simd;
  int occ = occ_lds < occ_reg ? occ_lds : occ_reg;
  if (occ < 1) occ = 1;
  if (occ > 8) occ = 8;
  return occ;
}

}  // namespace

int policy_count() { return kCount; }
const Policy& policy_at(int i) { return kTable[i]; }

int policy_find(const char* name) {
  if (!name) return -1;
  for (int i = 0; i < kCount; ++i)
    if (std::strcmp(kTable[i].name, name) == 0) return i;
  return -1;
}

bool policy_serves(const Policy& p, const Problem& pr) {
  if (p.kind == KIND_SIMT) return true;
  if (p.kind != KIND_MFMA || !pr.fast_ok) return false;
  if (p.k_contig_only && (pr.transA != 0 || pr.transB != 1)) return false;
  if (p.a_kc_only && pr.transA != 0) return false;
  if (pr.mx) return p.in_mode == 3 || ((p.in_mode == 4 || p.in_mode == 6) && pr.mx_words);
  if (pr.blas3)  // triangle, K band or dual product: the bf16 direct-to-LDS kernels
    return p.pipe == 1 && p.in_mode == 0 && !pr.in_fp8 && (!pr.square_tiles || p.BM == p.BN);
  return (p.in_mode < 3 || p.in_mode == 5) && (p.in_mode != 0) == (pr.in_fp8 != 0);
}

int64_t split_ws_floats(const Policy& p, const Problem& pr, int splits) {
  const int64_t tiles = ((pr.M + p.BM - 1) / p.BM) * ((pr.N + p.BN - 1) / p.BN);
  return tiles * splits * p.BM * p.BN;
}

// K tiles per split for `splits` ways, or 0 when that split is not a distinct,
// useful one (every split gets at least two K tiles and the last is not empty).
int64_t split_kt(const Policy& p, int64_t K, int splits) {
  const int64_t nk = (K + p.BK - 1) / p.BK;
  if (splits == 1) return nk;
  const int64_t per = (nk + splits - 1) / splits;
  if (per < 2 || (nk + per - 1) / per != splits) return 0;
  return per;
}

bool split_allowed(const Policy& p, const Problem& pr, int splits, int64_t ws_floats) {
  if (splits == 1) return true;
  if (p.pipe != 1 || split_kt(p, pr.K, splits) == 0) return false;  // direct-to-LDS ring kernels
  return split_ws_floats(p, pr, splits) <= ws_floats;
}

// Fewest K tiles a stream-K workgroup sums: below this the partial hand-offs cost more
// than the balance gains.
constexpr int kStreamKMinIters = 4;

StreamK stream_k_plan(const Policy& p, const Problem& pr, int cu_count, int grid) {
  StreamK s;
  // the ping-pong kernels on plain operands; the 128-deep E4M3 tile has no stream-K form
  // (its registers would spill)
  if (p.kind != KIND_MFMA || p.pipe != 2 || pr.blas3 || pr.mx || (p.in_mode == 5 && p.BK > 64)) return s;
  if (cu_count <= 0) cu_count = 256;
  const int64_t tiles = ((pr.M + p.BM - 1) / p.BM) * ((pr.N + p.BN - 1) / p.BN);
  const int64_t nk = (pr.K + p.BK - 1) / p.BK;
  // one workgroup per CU at a time (the ping-pong tiles fill the LDS), so a grid of at
  // most one per CU is resident at once: every owner's wait ends
  const int64_t G = grid > 0 ? (grid < cu_count ? grid : cu_count) : cu_count;
  if (tiles == 0 || nk < 2 || (grid == 0 && tiles % G == 0)) return s;
  const int64_t dp = (tiles / G) * G;
  const int64_t rest = tiles - dp;
  if (rest == 0) return s;
  int64_t iters = (rest * nk + G - 1) / G;
  if (iters < kStreamKMinIters) iters = nk < kStreamKMinIters ? nk : kStreamKMinIters;
  s.dp = (int)dp;
  s.tiles = (int)rest;
  s.iters = (int)iters;
  s.grid = (int)((rest * nk + iters - 1) / iters);
  return s;
}

int64_t stream_k_ws_floats(const Policy& p, const StreamK& s) { return (int64_t)s.grid * p.BM * p.BN; }

int policy_select(const Problem& pr, int cu_count, int64_t ws_floats, int* splits) {
  if (cu_count <= 0) cu_count = 256;
  int best = policy_find("simt_generic");
  *splits = 1;
  if (!pr.fast_ok) return best;
  double best_t = 0.0;
  bool have = false;
  const double K0 = 256.0;  // prologue + epilogue cost of a tile, in K-equivalents
  // Split-K adds a reduction launch: about 1.5 us plus 0.75 us per split on MI355X.
  // The model's unit is BM*BN*K/efficiency per CU; one us is about 2e6 of them (a
  // 64 x 64 tile at efficiency 0.5 advances about 265 K per us).
  const double kUnitsPerUs = 2.0e6;
  for (int i = 0; i < kCount; ++i) {
    const Policy& p = kTable[i];
    if (p.kind != KIND_MFMA || p.efficiency <= 0.f || !policy_serves(p, pr)) continue;
    const int occ = occupancy(p);
    double tiles = (double)((pr.M + p.BM - 1) / p.BM) * (double)((pr.N + p.BN - 1) / p.BN);
    if (pr.square_tiles) {  // a triangle of the T x T tile grid
      const double t = (double)((pr.M + p.BM - 1) / p.BM);
      tiles = t * (t + 1) / 2;
    }
    const double slots = (double)cu_count * occ;
    for (int sp = 1; sp <= 16; sp *= 2) {
      if (!split_allowed(p, pr, sp, ws_floats)) continue;
      const double wgs = tiles * sp;
      const double k_eff = (double)split_kt(p, pr.K, sp) * p.BK;
      const double rounds = (double)(int64_t)((wgs + slots - 1) / slots);
      // workgroups sharing a CU at a time: the occupancy, or fewer on a small grid
      const double per_cu = (double)(int64_t)((wgs + cu_count - 1) / cu_count);
      const double conc = per_cu < occ ? per_cu : occ;
      // (the four-slot ping-pong ring, measured at 4096^2 against the two-slot 64-deep one,
      // is as fast or faster from K = 256 up: 14.8-15.7 against 15.6-16.4 us at K = 256)
      double t = rounds * conc * (double)p.BM * p.BN * (k_eff + K0) / p.efficiency;
      // a K band, tiles walked from the longest K to the shortest: round r of R holds
      // tiles of about K (1 - r/R), so the rounds add up to (R + 1) / 2 full-K rounds
      if (pr.kband) t *= (rounds + 1.0) / (2.0 * rounds);
      if (sp > 1) t += (1.5 + 0.75 * sp) * kUnitsPerUs;
      if (!have || t < best_t * 0.999) {
        best = i;
        best_t = t;
        *splits = sp;
        have = true;
      }
    }
  }
  return best;
}

}  // namespace dbgemm
