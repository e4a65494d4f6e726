// Internal interfaces between the C-ABI layer, the policy table and the kernels.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

namespace dbgemm {

// Everything a kernel needs for one call.  Sizes are validated on the host before a
// launch: the fast kernels additionally require every operand span to stay below
// 2^31 bytes so that 32-bit buffer offsets cover it.
// C element types (GemmArgs::c_kind)
enum { C_BF16 = 0, C_F32 = 1, C_E4M3 = 2 };

struct GemmArgs {
  const void* A;
  const void* B;
  void* C;
  int64_t lda, ldb, ldc;
  int M, N, K;
  float alpha, beta;
  int c_kind;     // C's element type: C_BF16, C_F32 or C_E4M3
  int in_fp8;     // 1: A, B are E4M3, 0: bf16
  int transA, transB;
  int tiles_m, tiles_n;
  int group;      // raster group width (tiles) along the grouped dimension
  int raster_n;   // 0: groups of `group` tile-rows walked along N; 1: the transpose
  int xcd;        // XCDs to remap across (1 disables the remap; below -1: runs of four in turn)
  int swizzle;    // 1: XOR-swizzled LDS layout, 0: plain row-major LDS tiles
  int krot;       // 1: each XCD starts its K loop at its own eighth of K (see the DMA kernel)
  // Split-K (direct-to-LDS kernels): `splits` workgroups share each output tile, split
  // s summing K tiles [s*kt_per_split, (s+1)*kt_per_split).  Each writes its fp32
  // partial tile to `ws` (slot tile*splits + s, tile = tm*tiles_n + tn); a second
  // kernel adds the partials in split order and runs the epilogue.  splits == 1: no
  // workspace use.
  int splits;
  int kt_per_split;
  float* ws;
  // Stream-K (ping-pong kernel; sk_tiles == 0: off).  Workgroups 0 .. sk_dp-1 each run
  // one whole tile, the first sk_dp tiles of the raster order.  The other sk_tiles tiles
  // are shared by the next sk_grid workgroups: their K loops are laid end to end and
  // workgroup s sums K tiles [s*sk_iters, (s+1)*sk_iters) of that sequence (the last one
  // fewer).  A range that starts inside a tile leaves that part's sum in the workgroup's
  // slot of `ws` (BM*BN floats per slot) and sets flags[slot] to `epoch` (non-zero); the
  // workgroup holding the tile's first K tile waits for those flags, adds the partials in
  // K order, sets the flags back to zero and runs the epilogue.
  int sk_dp, sk_tiles, sk_grid, sk_iters;
  int* flags;
  int epoch;
  // Block-scaled E4M3 (mx = 1): one UE8M0 byte per row and 32-element K block, for A
  // (rows m) in sa[m * ldsa + k / 32] and for B (rows n) in sb[n * ldsb + k / 32].
  int mx;
  const uint8_t* sa;
  const uint8_t* sb;
  int64_t ldsa, ldsb;
  // Triangle of C (the symmetric rank-K updates): TRI_LOWER writes only elements with
  // row >= column, TRI_UPPER only row <= column, and the grid holds only the tiles that
  // meet that triangle (square tiles, M == N; see tile_of).  TRI_NONE: all of C.
  int tri;
  // K band of each tile (a triangular operand expanded with zeros outside its triangle):
  // the tile skips the K tiles that meet only zeros.  KBAND_A_LOWER: op(A) is lower, tile
  // row tm reads k < (tm+1)*BM; KBAND_A_UPPER: k >= tm*BM; KBAND_B_LOWER: op(B) is lower
  // (zero for k < n), tile column tn reads k >= tn*BN; KBAND_B_UPPER: k < (tn+1)*BN.
  // band_off is added to the tile's first row (A bands) or column (B bands): the index,
  // in the triangular operand, of this call's first row or column of C.
  int kband;
  int band_off;
  // Two products in one sum (the rank-2K update when its operands cannot be packed): with
  // dual set, the K loop runs over op(A)*op(B) and then over op(A2)*op(B2), same M, N, K and
  // transposes; A2 has leading dimension lda2, B2 ldb2.  Generic kernel only.
  int dual;
  const void* A2;
  const void* B2;
  int64_t lda2, ldb2;
  // A batch of equal products (direct-to-LDS kernels, unsplit, a K band at most): workgroup
  // (x, y, z) runs tile x of the product whose A, B and C start y * bs?[0] + z * bs?[1]
  // elements past the given ones.  batch_y, batch_z: the batch extents (0 or 1: none).
  int batch_y, batch_z;
  int64_t bsA[2], bsB[2], bsC[2];
};
enum { TRI_NONE = 0, TRI_LOWER = 1, TRI_UPPER = 2 };
enum { KBAND_NONE = 0, KBAND_A_LOWER = 1, KBAND_A_UPPER = 2, KBAND_B_LOWER = 3, KBAND_B_UPPER = 4 };

// Workgroups of a tile grid: every tile, or with a triangle the T(T+1)/2 tiles on and
// below (or above) the diagonal of the T x T tile grid; times the split-K factor.
__host__ __device__ inline int grid_tiles(const GemmArgs& a) {
  const int t = a.tri ? a.tiles_m * (a.tiles_m + 1) / 2 : a.tiles_m * a.tiles_n;
  return t * a.splits;
}

enum PolicyKind { KIND_SIMT = 0, KIND_MFMA = 1, KIND_SCALE = 2 };

struct Policy {
  const char* name;
  int kind;
  int pipe;        // 0: global -> registers -> LDS (two stages); 1: direct-to-LDS loads into a
                   // ring; 2: direct-to-LDS loads, two wave groups taking turns (ping-pong)
  int in_mode;     // 0: bf16 in, bf16 MFMA; 1: E4M3 in, widened to bf16 in LDS (exact
                   // fp32 accumulation); 2: E4M3 in, native f8f6f4 MFMA; 3: block-scaled
                   // E4M3 (MXFP8), widened with its scale; 4: block-scaled E4M3 on the
                   // scaled f8f6f4 MFMA; 5: E4M3 in, E4M3 in LDS, widened to bf16 in
                   // registers (ping-pong kernel); 6: block-scaled E4M3, bytes and scales in
                   // LDS, widened with the scale in registers (ping-pong kernel); -1: any
  int BM, BN, BK;  // workgroup tile
  int WM, WN;      // waves along M and N
  int MT;          // MFMA block edge (32 or 16)
  int stages;      // LDS stages
  int group, raster_n, xcd, swizzle;
  int krot;        // K-loop rotation per XCD (direct-to-LDS kernels only)
  int read_mode;   // 1: transposing LDS reads for M/N-contiguous operands; 0: one element per read
  int threads;
  float efficiency;  // relative per-CU throughput used by the wave-time model
  int k_contig_only;  // serves only A [M][K] with B [N][K] (transA = 0, transB = 1)
  int a_kc_only;      // serves only A [M][K] (transA = 0)
};

// Launchers (one per kernel family).  They return hipSuccess or the launch error.
hipError_t launch_simt(const GemmArgs& a, hipStream_t s);
hipError_t launch_scale(const GemmArgs& a, hipStream_t s);  // C <- beta*C (K == 0 or alpha == 0)
hipError_t launch_mfma_staged(const Policy& p, const GemmArgs& a, hipStream_t s);  // pipe 0
// pipe 0, one per (transA, transB) case, each in its own object
hipError_t launch_mfma_staged_00(const Policy& p, const GemmArgs& a, hipStream_t s);
hipError_t launch_mfma_staged_01(const Policy& p, const GemmArgs& a, hipStream_t s);
hipError_t launch_mfma_staged_10(const Policy& p, const GemmArgs& a, hipStream_t s);
hipError_t launch_mfma_staged_11(const Policy& p, const GemmArgs& a, hipStream_t s);
hipError_t launch_mfma_dma(const Policy& p, const GemmArgs& a, hipStream_t s);     // pipe 1
// pipe 1, one per (transA, transB) case and half of the policy table, each in its own
// object: true when that part launched p (*err = the launch status)
#define DBGEMM_DMA_DECL(ab)                                                                           \
  bool launch_mfma_dma_##ab##_p0(const Policy& p, const GemmArgs& a, hipStream_t s, hipError_t* err); \
  bool launch_mfma_dma_##ab##_p1(const Policy& p, const GemmArgs& a, hipStream_t s, hipError_t* err);
DBGEMM_DMA_DECL(00)
DBGEMM_DMA_DECL(01)
DBGEMM_DMA_DECL(10)
DBGEMM_DMA_DECL(11)
#undef DBGEMM_DMA_DECL
// pipe 2 (ping-pong), one per (transA, transB) case
hipError_t launch_mfma_pp(const Policy& p, const GemmArgs& a, hipStream_t s);
hipError_t launch_mfma_pp_00(const Policy& p, const GemmArgs& a, hipStream_t s);
hipError_t launch_mfma_pp_01(const Policy& p, const GemmArgs& a, hipStream_t s);
hipError_t launch_mfma_pp_10(const Policy& p, const GemmArgs& a, hipStream_t s);
hipError_t launch_mfma_pp_11(const Policy& p, const GemmArgs& a, hipStream_t s);

// LDS read microbenchmark: 8 reads per lane per iteration, offsets in bytes from the
// start of a 64 KiB LDS array, each a multiple of the read width and inside the array.
struct LdsProbeOffsets {
  uint32_t off[8][64];
};
constexpr int kLdsProbeBytes = 65536;
int lds_probe_width(int kind);  // bytes per lane of read kind 0..5, 0 for an unknown kind
int lds_probe_span(int kind);   // bytes from a lane's offset to the end of what its read touches
hipError_t launch_lds_probe(int kind, const LdsProbeOffsets& offs, int iters, int workgroups, hipStream_t s);

// Hardware microbenchmarks (gemm_hw_probe): kind 0 / 1 the 16x16x32 / 32x32x16 bf16 MFMA
// issue (param 1: the two wave groups take turns), kind 2 the direct-to-LDS copy of 256-row
// tiles of `param` bytes per row from a buffer of rows of kHwProbePitch bytes.
constexpr int64_t kHwProbePitch = 8192;
hipError_t launch_hw_probe(int kind, int param, int iters, int workgroups, const void* src, int64_t src_bytes,
                           unsigned long long* cycles, hipStream_t s);

// bf16 [rows][ld_src] -> E4M3 [rows][ld_dst] plus one UE8M0 byte per 32 elements of a row
// in scales [rows][ld_scales] (the MXFP8 quantisation; see gemm_quantize_mx).
constexpr int64_t kQuantizeMaxCols = (int64_t)65535 * 256 * 8;  // one grid row of 8-element chunks
hipError_t launch_quantize_mx(int64_t rows, int64_t cols, const void* src, int64_t ld_src, void* dst,
                              int64_t ld_dst, uint8_t* scales, int64_t ld_scales, hipStream_t s);

// Tile-policy table.
int policy_count();
const Policy& policy_at(int i);
int policy_find(const char* name);

struct Problem {
  int transA, transB;
  int64_t M, N, K;
  int in_fp8, c_kind;
  int mx;        // block-scaled E4M3 operands (gemm_run_mx)
  bool mx_words;  // scale rows 4-byte aligned (the scaled native MFMA reads 32-bit words)
  bool fast_ok;  // alignment / divisibility allow the MFMA kernels
  // BLAS3 calls with a triangle, K band or second product: direct-to-LDS bf16 kernels
  // only, unsplit, and square tiles for a triangle
  bool blas3 = false;
  bool square_tiles = false;
  bool kband = false;  // per-tile K band (wave model: longest tiles first)
};
// Stream-K plan of a ping-pong policy on a problem (the GemmArgs fields of that name);
// tiles == 0: none (the grid is whole rounds, or the policy has no stream-K form).
// `grid` > 0 asks for that many stream-K workgroups; 0 takes one per CU.
struct StreamK {
  int dp = 0, tiles = 0, grid = 0, iters = 0;
};
StreamK stream_k_plan(const Policy& p, const Problem& pr, int cu_count, int grid = 0);
int64_t stream_k_ws_floats(const Policy& p, const StreamK& s);  // partial slots
// Shape-driven selection; returns an index into the table and, in *splits, the
// split-K factor (1 unless a workspace of ws_floats fp32 values allows more).  Stream-K is
// never chosen here, only by name: on the grids it was built for (dX, dW) it measured
// slower than the plain grid, because its workgroups run at scattered K offsets and lose
// the L2 reuse of workgroups that step through K together.
int policy_select(const Problem& pr, int cu_count, int64_t ws_floats, int* splits);
// fp32 partials a split-K call of policy p with `splits` needs, K tiles per split
// (0: that split is not allowed), and whether the split fits a workspace.
int64_t split_ws_floats(const Policy& p, const Problem& pr, int splits);
int64_t split_kt(const Policy& p, int64_t K, int splits);
bool split_allowed(const Policy& p, const Problem& pr, int splits, int64_t ws_floats);
bool policy_serves(const Policy& p, const Problem& pr);

}  // namespace dbgemm
