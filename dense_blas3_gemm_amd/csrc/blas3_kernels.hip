// Device kernels of the single-GPU BLAS3 family that are not GEMMs ("BLASMp development
// notes", section 2: SYMM, TRMM and TRSM built on a GEMM core).  The products themselves
// run on the GEMM kernels; these kernels prepare their operands:
//
//   * expand_tri_kernel: a rectangle of the dense matrix a triangular operand stands for
//     (its stored triangle, zeros elsewhere, ones on a unit diagonal), so that TRMM is a
//     GEMM whose tiles skip the zero K band;
//   * expand_sym_kernel: a rectangle of the dense symmetric matrix a stored triangle
//     stands for, mirrored through LDS so that both the reads and the writes are
//     row-contiguous;
//   * invert_diag_kernel, combine_inverse_kernel: the inverses of the 256 x 256 diagonal
//     blocks of a triangular operand, from fp32 inverses of their 128 x 128 halves, stored as
//     bf16: TRSM then applies each diagonal block as a product.
//
// Every kernel reads the stored triangle only: the other triangle (and a unit diagonal)
// may hold anything, NaN included.
#include <type_traits>

#include "blas3_internal.h"

namespace dbgemm {
namespace {

__device__ inline float bf16f(uint16_t b) { return __builtin_bit_cast(float, (uint32_t)b << 16); }
__device__ inline uint16_t f2bf(float v) { return __builtin_bit_cast(uint16_t, static_cast<__bf16>(v)); }

__device__ inline bool referenced(int i, int j, int uplo) { return uplo == 0 ? i >= j : i <= j; }

// dst[r][c] (r < rows, c < cols, leading dimension ldd) = T[r0 + r][c0 + c] of the n x n
// triangular matrix T.  One thread per 8 consecutive columns of one row, written with one
// 16-byte store; a group inside the stored triangle (and off a unit diagonal) is read with
// one 16-byte load when `vec` (src 16-byte aligned, lds and c0 multiples of 8), the rest
// element by element, and groups outside it are not read.  Columns past `cols` up to the
// padded width are zeros.
__global__ __launch_bounds__(256) void expand_tri_kernel(const uint16_t* __restrict__ src, int64_t lds,
                                                         uint16_t* __restrict__ dst, int64_t ldd, int r0, int c0,
                                                         int rows, int cols, int cols_pad, int uplo, int unit,
                                                         int vec) {
  const int groups = cols_pad / 8;
  const int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (t >= (int64_t)rows * groups) return;
  const int r = (int)(t / groups), c8 = (int)(t % groups) * 8;
  const int i = r0 + r, j0 = c0 + c8;
  uint4 w;
  // the whole group strictly inside the triangle: i > j0 + 7 (lower) or i < j0 (upper)
  const bool inside = c8 + 8 <= cols && (uplo == 0 ? i > j0 + 7 : i < j0);
  const bool outside = uplo == 0 ? i < j0 : i > j0 + 7;
  if (vec && inside) {
    w = *(const uint4*)(src + (int64_t)i * lds + j0);
  } else if (outside) {
    w = make_uint4(0, 0, 0, 0);
  } else {
    uint16_t v[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int c = c8 + e, j = c0 + c;
      float x = 0.f;
      if (c < cols) {
        if (i == j && unit) x = 1.f;
        else if (referenced(i, j, uplo)) x = bf16f(src[(int64_t)i * lds + j]);
      }
      v[e] = f2bf(x);
    }
    w.x = v[0] | ((uint32_t)v[1] << 16);
    w.y = v[2] | ((uint32_t)v[3] << 16);
    w.z = v[4] | ((uint32_t)v[5] << 16);
    w.w = v[6] | ((uint32_t)v[7] << 16);
  }
  *(uint4*)(dst + (int64_t)r * ldd + c8) = w;
}

constexpr int SB = 64;  // block edge of the kernels that go through an LDS block
constexpr int kInvThreads = 512;  // threads of a 128-block inversion

// dst[r][c] = T^T[r0 + r][c0 + c] = T[c0 + c][r0 + r] of the n x n triangular T (stored
// triangle, zeros elsewhere, ones on a unit diagonal): the transposed operand written out, so
// that the product that follows reads it in the layout of an untransposed one.  Workgroup
// (bx, by) writes the 64 x 64 block at rows 64*by, columns 64*bx: the source block (rows
// c0 + 64*bx .., columns r0 + 64*by ..) is read row-wise into LDS (16-byte loads when `vec`)
// and written transposed, 8 columns per 16-byte store.  Columns past `cols` up to the padded
// width are zeros.
__global__ __launch_bounds__(256) void expand_tri_trans_kernel(const uint16_t* __restrict__ src, int64_t lds,
                                                               uint16_t* __restrict__ dst, int64_t ldd, int r0,
                                                               int c0, int rows, int cols, int cols_pad, int n,
                                                               int uplo, int unit, int vec) {
  __shared__ uint16_t tile[SB][SB + 2];  // tile[y][x] = src[sr0 + y][sc0 + x]; 33-word rows: column reads spread over the banks
  const int br = blockIdx.y * SB, bc = blockIdx.x * SB;
  const int sr0 = c0 + bc, sc0 = r0 + br;  // the source block
  for (int e = threadIdx.x; e < SB * SB / 8; e += 256) {
    const int y = e / (SB / 8), x8 = (e % (SB / 8)) * 8;
    const int si = sr0 + y, sj = sc0 + x8;
    uint16_t v[8];
    if (vec && si < n && sj + 7 < n) {
      const uint4 w = *(const uint4*)(src + (int64_t)si * lds + sj);
      v[0] = (uint16_t)w.x; v[1] = (uint16_t)(w.x >> 16); v[2] = (uint16_t)w.y; v[3] = (uint16_t)(w.y >> 16);
      v[4] = (uint16_t)w.z; v[5] = (uint16_t)(w.z >> 16); v[6] = (uint16_t)w.w; v[7] = (uint16_t)(w.w >> 16);
    } else {
#pragma unroll
      for (int k = 0; k < 8; ++k) v[k] = si < n && sj + k < n ? src[(int64_t)si * lds + sj + k] : (uint16_t)0;
    }
#pragma unroll
    for (int k = 0; k < 8; ++k) tile[y][x8 + k] = v[k];
  }
  __syncthreads();
  const uint16_t one = f2bf(1.f);
  for (int e = threadIdx.x; e < SB * SB / 8; e += 256) {
    const int y = e / (SB / 8), x8 = (e % (SB / 8)) * 8;
    const int r = br + y, c = bc + x8;
    if (r >= rows || c >= cols_pad) continue;
    const int i = r0 + r;  // row of T^T = column of T
    uint16_t v[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const int j = c0 + c + k;  // column of T^T = row of T: element T[j][i]
      uint16_t x = 0;
      if (c + k < cols && i < n && j < n) {
        if (i == j && unit) x = one;
        else if (referenced(j, i, uplo)) x = tile[x8 + k][y];
      }
      v[k] = x;
    }
    uint4 w;
    w.x = v[0] | ((uint32_t)v[1] << 16);
    w.y = v[2] | ((uint32_t)v[3] << 16);
    w.z = v[4] | ((uint32_t)v[5] << 16);
    w.w = v[6] | ((uint32_t)v[7] << 16);
    *(uint4*)(dst + (int64_t)r * ldd + c) = w;
  }
}

// dst[r][c] = S[r0 + r][c0 + c] of the symmetric matrix S whose uplo triangle is stored
// in src.  Workgroup (bx, by) writes the 64 x 64 output block at rows 64*by, columns
// 64*bx, 8 columns (16 bytes) per thread and store; its elements come from src directly
// where (i, j) is referenced and from the mirrored block elsewhere, which is read row-wise
// into LDS and read back transposed.  With `vec` (src 16-byte aligned, lds, r0 and c0
// multiples of 8) groups of 8 stored elements are read with one 16-byte load.  Columns
// past `cols` up to the padded width are zeros.
__global__ __launch_bounds__(256) void expand_sym_kernel(const uint16_t* __restrict__ src, int64_t lds,
                                                         uint16_t* __restrict__ dst, int64_t ldd, int r0, int c0,
                                                         int rows, int cols, int cols_pad, int n, int uplo, int vec) {
  __shared__ uint16_t mir[SB][SB + 2];  // mir[y][x] = src[gj0 + y][gi0 + x]; 33-word rows: column reads spread over the banks
  const int br = blockIdx.y * SB, bc = blockIdx.x * SB;  // output block origin
  const int gi0 = r0 + br, gj0 = c0 + bc;                  // in S
  // 8 stored elements of src row si from column sj, or fewer / none at the edges
  auto read8 = [&](int si, int sj, uint16_t* v) {
    const bool all = si < n && sj + 7 < n && (uplo == 0 ? si >= sj + 7 : si <= sj);
    if (vec && all) {
      const uint4 w = *(const uint4*)(src + (int64_t)si * lds + sj);
      v[0] = (uint16_t)w.x; v[1] = (uint16_t)(w.x >> 16); v[2] = (uint16_t)w.y; v[3] = (uint16_t)(w.y >> 16);
      v[4] = (uint16_t)w.z; v[5] = (uint16_t)(w.z >> 16); v[6] = (uint16_t)w.w; v[7] = (uint16_t)(w.w >> 16);
      return;
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int sje = sj + e;
      v[e] = si < n && sje < n && referenced(si, sje, uplo) ? src[(int64_t)si * lds + sje] : (uint16_t)0;
    }
  };
  // does the block need the mirror (any element outside the stored triangle)?
  const bool need_mirror = uplo == 0 ? (gi0 < gj0 + SB - 1) : (gi0 + SB - 1 > gj0);
  if (need_mirror) {
    for (int e = threadIdx.x; e < SB * SB / 8; e += 256) {
      const int y = e / (SB / 8), x8 = (e % (SB / 8)) * 8;
      uint16_t v[8];
      read8(gj0 + y, gi0 + x8, v);
#pragma unroll
      for (int k = 0; k < 8; ++k) mir[y][x8 + k] = v[k];
    }
  }
  __syncthreads();
  for (int e = threadIdx.x; e < SB * SB / 8; e += 256) {
    const int y = e / (SB / 8), x8 = (e % (SB / 8)) * 8;
    const int r = br + y, c = bc + x8;
    if (r >= rows || c >= cols_pad) continue;
    const int i = r0 + r, j = c0 + c;
    uint16_t v[8];
    read8(i, j, v);  // the referenced ones (zeros elsewhere)
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      if (c + k >= cols || i >= n || j + k >= n) v[k] = 0;
      else if (!referenced(i, j + k, uplo)) v[k] = mir[x8 + k][y];  // S[i][j+k] = src[j+k][i]
    }
    uint4 w;
    w.x = v[0] | ((uint32_t)v[1] << 16);
    w.y = v[2] | ((uint32_t)v[3] << 16);
    w.z = v[4] | ((uint32_t)v[5] << 16);
    w.w = v[6] | ((uint32_t)v[7] << 16);
    *(uint4*)(dst + (int64_t)r * ldd + c) = w;
  }
}

// The same expansion for a region of whole 64 x 64 blocks inside S (rows and columns 16-byte
// aligned), one wave per block and no LDS: lane (p, q) builds the 8 x 8 sub-block at rows
// 8q .., columns 8p .. of the output block, from eight 16-byte loads of the stored rows
// (where the sub-block meets the stored triangle) and eight 16-byte loads of the mirrored
// rows (where it meets the other one), those transposed in registers; a diagonal block
// takes each element from the right source.  Loads and stores of a wave cover 8 rows x
// 128 contiguous bytes each.
__global__ __launch_bounds__(256) void expand_sym_blocks_kernel(const uint16_t* __restrict__ src, int64_t lds,
                                                                uint16_t* __restrict__ dst, int64_t ldd, int r0,
                                                                int c0, int bcols, int nblocks, int uplo) {
  const int blk = (int)blockIdx.x * 4 + (int)(threadIdx.x >> 6), lane = threadIdx.x & 63;
  if (blk >= nblocks) return;
  const int by = blk / bcols, bx = blk % bcols;
  const int p = lane / 8, q = lane % 8;
  const int gi = r0 + by * SB + 8 * q, gj = c0 + bx * SB + 8 * p;  // S position of the sub-block
  const bool lower = uplo == 0;
  // sub-block rows gi .. gi+7, columns gj .. gj+7: stored where row >= column (lower)
  const bool any_direct = lower ? gi + 7 >= gj : gi <= gj + 7;
  const bool any_mirror = lower ? gi < gj + 7 : gi + 7 > gj;
  uint4 d[8], m[8];
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    d[k] = any_direct ? *(const uint4*)(src + (int64_t)(gi + k) * lds + gj) : make_uint4(0, 0, 0, 0);
    m[k] = any_mirror ? *(const uint4*)(src + (int64_t)(gj + k) * lds + gi) : make_uint4(0, 0, 0, 0);
  }
  // S[gi + k][gj + e] = src[gj + e][gi + k] = element k of m[e] where mirrored
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    const uint32_t dw[4] = {d[k].x, d[k].y, d[k].z, d[k].w};
    uint32_t w[4];
#pragma unroll
    for (int h = 0; h < 4; ++h) {
      const uint4 a = m[2 * h], b = m[2 * h + 1];
      const uint32_t ak = (k / 2 == 0 ? a.x : k / 2 == 1 ? a.y : k / 2 == 2 ? a.z : a.w);
      const uint32_t bk = (k / 2 == 0 ? b.x : k / 2 == 1 ? b.y : k / 2 == 2 ? b.z : b.w);
      const uint32_t mir = (k & 1) ? ((ak >> 16) | (bk & 0xFFFF0000u)) : ((ak & 0xFFFFu) | (bk << 16));
      if (!any_mirror) {
        w[h] = dw[h];
      } else if (!any_direct) {
        w[h] = mir;
      } else {  // a diagonal sub-block: element by element
        const int i = gi + k, j = gj + 2 * h;
        const uint32_t lo = referenced(i, j, uplo) ? (dw[h] & 0xFFFFu) : (mir & 0xFFFFu);
        const uint32_t hi = referenced(i, j + 1, uplo) ? (dw[h] & 0xFFFF0000u) : (mir & 0xFFFF0000u);
        w[h] = lo | hi;
      }
    }
    *(uint4*)(dst + (int64_t)(by * SB + 8 * q + k) * ldd + bx * SB + 8 * p) = make_uint4(w[0], w[1], w[2], w[3]);
  }
}

// Inverse of each diagonal block T_bb (rows and columns [b*NB, b*NB + nb), nb = NB except
// for a shorter last block) of the n x n triangular T, padded to NB x NB with the
// identity, in fp32, by recursive doubling: an upper block is handled as the transpose of
// a lower one, L = T_bb^T, inv(T_bb) = inv(L)^T.  For a lower block [A 0; C D],
//   inv = [inv(A) 0; -inv(D) (C inv(A))  inv(D)],
// so the inverses of the four 32 x 32 diagonal blocks (one column per thread, by
// substitution with the column in registers) give those of the two 64 x 64 blocks (two
// products of 32 x 32 matrices each), which give the 128 x 128 inverse (two products of
// 64 x 64 matrices).  The serial chain is 32 substitution steps plus four products,
// against 128 steps for substitution over the whole block.  L is kept transposed in LDS
// (column k one contiguous row); the inverse X is built in LDS, the products' first
// factor W = C inv(A) parked in X's upper triangle (zero in the result, cleared after
// use).  The result, zeros outside the triangle, is stored at dst + b*NB*NB, [NB][NB];
// blocks past n are the identity.  The first `whole` blocks (those of T's whole lf-blocks)
// are stored instead rounded to bf16 on the diagonals of bdst, [n / lf][lf][lf], and the
// lf-blocks' 128-blocks outside the triangle are zeroed: products double them up to lf x lf.
template <bool UPPER>
__global__ __launch_bounds__(kInvThreads) void invert_diag_kernel(const uint16_t* __restrict__ src, int64_t lds, int n,
                                                          int unit, int vec, float* __restrict__ dst,
                                                          uint16_t* __restrict__ bdst, int lf, int whole) {
  constexpr int NB = kTrsmNB, LD = NB + 4, SB = 32;  // row stride: float4-aligned rows
  static_assert(NB == 128, "three doubling levels from 32");
  __shared__ __attribute__((aligned(16))) float Lt[NB * LD];  // Lt[k * LD + r] = L[r][k]
  __shared__ __attribute__((aligned(16))) float X[NB * LD];   // X[r * LD + c] = inv(L)[r][c]
  __shared__ float dinv[NB];                                  // 1 / L[k][k]
  const int b = blockIdx.x, o = b * NB;
  const int nb = n - o < NB ? n - o : NB;
  const int t = threadIdx.x;
  // ---- L (lower: L[i][j] = T[o+i][o+j]; upper: T[o+j][o+i]), j <= i; the identity past
  // nb and on a unit diagonal; zeros above the diagonal.  Element (p, q) of the stored
  // block is L[i][j] with (i, j) = (p, q) for a lower block and (q, p) for an upper one.
  auto put = [&](int p, int q, uint16_t bits) {
    const int i = UPPER ? q : p, j = UPPER ? p : q;
    float v = 0.f;
    if (i == j && (unit || i >= nb)) v = 1.f;
    else if (j <= i && i < nb && j < nb) v = bf16f(bits);
    Lt[j * LD + i] = v;
  };
  constexpr int TH = kInvThreads, PARTS = TH / NB;  // threads per row of the block
  if (vec && nb == NB) {
    // a whole block with 16-byte aligned rows: thread t reads part t % PARTS of row t / PARTS
    // as independent 16-byte loads issued together (the other triangle is read and dropped)
    const int p = t / PARTS, q0 = (t % PARTS) * (NB / PARTS);
    const uint4* rp = (const uint4*)(src + (int64_t)(o + p) * lds + o + q0);
    uint4 w[NB / PARTS / 8];
#pragma unroll
    for (int qq = 0; qq < NB / PARTS / 8; ++qq) w[qq] = rp[qq];
#pragma unroll
    for (int qq = 0; qq < NB / PARTS / 8; ++qq) {
      const uint32_t u[4] = {w[qq].x, w[qq].y, w[qq].z, w[qq].w};
#pragma unroll
      for (int hh = 0; hh < 4; ++hh) {
        put(p, q0 + 8 * qq + 2 * hh, (uint16_t)u[hh]);
        put(p, q0 + 8 * qq + 2 * hh + 1, (uint16_t)(u[hh] >> 16));
      }
    }
  } else {
    // element by element, the referenced ones only (consecutive threads, consecutive
    // elements of a row of T)
    for (int e = t; e < NB * NB; e += TH) {
      const int p = e / NB, q = e % NB;
      const bool ref = (UPPER ? p <= q : q <= p) && p < nb && q < nb;
      put(p, q, ref ? src[(int64_t)(o + p) * lds + o + q] : (uint16_t)0);
    }
  }
  for (int e = t; e < NB * NB; e += TH) X[(e / NB) * LD + e % NB] = 0.f;
  __syncthreads();
  if (t < NB) dinv[t] = 1.f / Lt[t * LD + t];
  __syncthreads();
  // ---- the four 32 x 32 diagonal inverses: thread t < 128 solves column t % 32 of block
  // t / 32 (x_k = b_k / L_kk, then b_r -= L_rk x_k for r > k)
  if (t < NB) {
    const int s0 = (t / SB) * SB, c = t % SB;
    float x[SB];
#pragma unroll
    for (int r = 0; r < SB; ++r) x[r] = r == c ? 1.f : 0.f;
#pragma unroll
    for (int k = 0; k < SB; ++k) {
      x[k] *= dinv[s0 + k];
      const float* col = Lt + (s0 + k) * LD + s0;  // L[s0 + r][s0 + k], r = 0 .. 31
#pragma unroll
      for (int r4 = (k + 1) / 4; r4 < SB / 4; ++r4) {
        const float4 l = *(const float4*)(col + 4 * r4);
        const float lv[4] = {l.x, l.y, l.z, l.w};
#pragma unroll
        for (int e = 0; e < 4; ++e)
          if (4 * r4 + e > k) x[4 * r4 + e] -= lv[e] * x[k];
      }
    }
#pragma unroll
    for (int r = 0; r < SB; ++r) X[(s0 + r) * LD + s0 + c] = x[r];
  }
  __syncthreads();
  // ---- doubling: for each block [A 0; C D] of edge 2h at offset o2, W = C inv(A) into
  // X[o2 .. o2+h)[o2+h .. o2+2h), then the lower-left quadrant -inv(D) W, then W cleared.
  // h = 32: two blocks, 256 threads each, 4 outputs per thread; h = 64: one block, 8.
  auto level = [&](auto hc) {
    constexpr int h = decltype(hc)::value, TPB = TH / (NB / (2 * h));  // threads per block
    constexpr int PER = h * h / TPB;                                      // outputs per thread
    const int blk = t / TPB, lt = t % TPB, o2 = blk * 2 * h;
    const int i = lt / (h / PER), j0 = (lt % (h / PER)) * PER;           // row i, columns j0 ..
    float w[PER];
#pragma unroll
    for (int e = 0; e < PER; ++e) w[e] = 0.f;
    // (the loops are unrolled so that the LDS reads of several k are in flight together)
#pragma unroll 8
    for (int k = 0; k < h; ++k) {
      const float cv = Lt[(o2 + k) * LD + o2 + h + i];  // C[i][k] = L[o2+h+i][o2+k]
      const float* ar = X + (o2 + k) * LD + o2 + j0;    // inv(A)[k][j0 ..]
#pragma unroll
      for (int e4 = 0; e4 < PER / 4; ++e4) {
        const float4 a4 = *(const float4*)(ar + 4 * e4);
        w[4 * e4] += cv * a4.x;
        w[4 * e4 + 1] += cv * a4.y;
        w[4 * e4 + 2] += cv * a4.z;
        w[4 * e4 + 3] += cv * a4.w;
      }
    }
    float* wr = X + (o2 + i) * LD + o2 + h + j0;  // W[i][j0 ..], in the upper-right quadrant
#pragma unroll
    for (int e = 0; e < PER; ++e) wr[e] = w[e];
    __syncthreads();
#pragma unroll
    for (int e = 0; e < PER; ++e) w[e] = 0.f;
#pragma unroll 4
    for (int k = 0; k <= i; ++k) {
      const float dv = X[(o2 + h + i) * LD + o2 + h + k];  // inv(D)[i][k], zero for k > i
      const float* wk = X + (o2 + k) * LD + o2 + h + j0;    // W[k][j0 ..]
#pragma unroll
      for (int e4 = 0; e4 < PER / 4; ++e4) {
        const float4 w4 = *(const float4*)(wk + 4 * e4);
        w[4 * e4] -= dv * w4.x;
        w[4 * e4 + 1] -= dv * w4.y;
        w[4 * e4 + 2] -= dv * w4.z;
        w[4 * e4 + 3] -= dv * w4.w;
      }
    }
    float* qr = X + (o2 + h + i) * LD + o2 + j0;  // the lower-left quadrant
#pragma unroll
    for (int e = 0; e < PER; ++e) qr[e] = w[e];
    __syncthreads();
#pragma unroll
    for (int e = 0; e < PER; ++e) wr[e] = 0.f;
    __syncthreads();
  };
  level(std::integral_constant<int, 32>{});
  level(std::integral_constant<int, 64>{});
  // ---- out: inv(T_bb) = X (lower) or X^T (upper), row-major, coalesced rows
  if (b >= whole) {  // for the combination into 256-blocks
    float* out = dst + (int64_t)b * NB * NB;
    for (int e = t; e < NB * NB; e += TH) {
      const int r = e / NB, c = e % NB;
      out[e] = UPPER ? X[c * LD + r] : X[r * LD + c];
    }
  } else {
    const int per = lf / NB, p = b % per;  // 128-blocks per lf-block; this one's position
    uint16_t* base = bdst + (int64_t)(b / per) * lf * lf;
    uint16_t* bo = base + (int64_t)p * NB * (lf + 1);
    for (int e = t; e < NB * NB / 2; e += TH) {  // two elements per 4-byte store
      const int r = e / (NB / 2), c = 2 * (e % (NB / 2));
      const float v0 = UPPER ? X[c * LD + r] : X[r * LD + c];
      const float v1 = UPPER ? X[(c + 1) * LD + r] : X[r * LD + c + 1];
      *(uint32_t*)(bo + (int64_t)r * lf + c) = (uint32_t)f2bf(v0) | ((uint32_t)f2bf(v1) << 16);
    }
    // the per (per - 1) / 2 128-blocks of the lf-block outside the triangle, dealt out to its
    // per workgroups in turn: zero block z is (row i, column j), i < j, j (j - 1) / 2 + i = z
    // (lower; the transpose for upper).  16-byte stores: lf and the offsets are multiples of 8.
    for (int zb = p; zb < per * (per - 1) / 2; zb += per) {
      int j = 1;
      while ((j + 1) * j / 2 <= zb) ++j;
      const int i = zb - j * (j - 1) / 2;
      uint16_t* z = base + (int64_t)(UPPER ? j : i) * NB * lf + (UPPER ? i : j) * NB;
      for (int e = t; e < NB * NB / 8; e += TH)
        *(uint4*)(z + (int64_t)(e / (NB / 8)) * lf + 8 * (e % (NB / 8))) = make_uint4(0, 0, 0, 0);
    }
  }
}

// Inverse of each 2 x 2 block of the 128-block inverses: the 256 x 256 diagonal block
// b of T, [A 0; C D] (lower) or [A C; 0 D] (upper), has the inverse
//   lower: [inv(A) 0; -inv(D) C inv(A)  inv(D)],   upper: [inv(A)  -inv(A) C inv(D); 0 inv(D)],
// i.e. Q = -P (C R) with (P, R) = (inv(D), inv(A)) or (inv(A), inv(D)).  Workgroup (b, s)
// computes columns [32s, 32s + 32) of Q in fp32 (W = C R[:, cols], then Q = -P W, each
// thread a 4 x 4 register tile) and writes columns 32s .. 32s + 31 of both halves of the
// block, rounded once to bf16.  inv holds the fp32 128-block inverses, block 2b = inv(A),
// 2b + 1 = inv(D).  dst holds the inverses of T's lf x lf diagonal blocks, [n / lf][lf][lf]
// (lf a multiple of 256): the 256-block b sits on the diagonal of lf-block b / (lf / 256),
// and the same workgroups write zeros in the 256-blocks of that lf-block outside its
// triangle, in their slab of columns (the products that double the inverses up to lf x lf
// fill the blocks inside the triangle).
constexpr int CB = 2 * kTrsmNB;  // the combined block edge
template <bool UPPER>
__global__ __launch_bounds__(256) void combine_inverse_kernel(const uint16_t* __restrict__ src, int64_t lds, int n,
                                                              int vec, const float* __restrict__ inv,
                                                              uint16_t* __restrict__ dst, int lf, int b0) {
  constexpr int NB = kTrsmNB, SW = 32, LD = NB + 4;
  __shared__ __attribute__((aligned(16))) float Xt[NB * LD];  // C^T, then P^T: Xt[k*LD + i] = X[i][k]
  __shared__ __attribute__((aligned(16))) float Rs[NB * SW];  // R[:, cols]
  __shared__ __attribute__((aligned(16))) float Ws[NB * SW];  // W = C R[:, cols]
  const int b = b0 + (int)blockIdx.x, s0 = blockIdx.y * SW, t = threadIdx.x;
  const int o = b * CB;
  const float* Ai = inv + (int64_t)(2 * b) * NB * NB;
  const float* Di = Ai + NB * NB;
  const float* P = UPPER ? Ai : Di;
  const float* R = UPPER ? Di : Ai;
  // C: rows o+128.., columns o.. (lower) or rows o.., columns o+128.. (upper) of T
  const int cr = UPPER ? o : o + NB, cc = UPPER ? o + NB : o;
  // C: thread t reads half t % 2 of row t / 2 (64 elements), as 8 independent 16-byte
  // loads when `vec` and the block is inside T, else element by element
  {
    const int i = t / 2, k0 = (t % 2) * (NB / 2);
    const int gi = cr + i;
    uint16_t row[NB / 2];
    if (vec && cr + NB <= n && cc + NB <= n) {
      const uint4* rp = (const uint4*)(src + (int64_t)gi * lds + cc + k0);
      uint4 w[NB / 16];
#pragma unroll
      for (int q = 0; q < NB / 16; ++q) w[q] = rp[q];
#pragma unroll
      for (int q = 0; q < NB / 16; ++q) {
        const uint32_t u[4] = {w[q].x, w[q].y, w[q].z, w[q].w};
#pragma unroll
        for (int h = 0; h < 4; ++h) {
          row[8 * q + 2 * h] = (uint16_t)u[h];
          row[8 * q + 2 * h + 1] = (uint16_t)(u[h] >> 16);
        }
      }
    } else {
#pragma unroll
      for (int k = 0; k < NB / 2; ++k)
        row[k] = gi < n && cc + k0 + k < n ? src[(int64_t)gi * lds + cc + k0 + k] : (uint16_t)0;
    }
#pragma unroll
    for (int k = 0; k < NB / 2; ++k) Xt[(k0 + k) * LD + i] = bf16f(row[k]);
  }
  {  // R[:, s0 .. s0 + 32): 1024 float4, four per thread
    float4 w[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int e = (t + 256 * q) * 4;
      w[q] = *(const float4*)(R + (e / SW) * NB + s0 + e % SW);
    }
#pragma unroll
    for (int q = 0; q < 4; ++q) *(float4*)(Rs + (t + 256 * q) * 4) = w[q];
  }
  __syncthreads();
  const int i0 = (t / 8) * 4, j0 = (t % 8) * 4;
  float acc[4][4] = {};
  for (int k = 0; k < NB; ++k) {
    const float4 a = *(const float4*)(Xt + k * LD + i0);
    const float4 w = *(const float4*)(Rs + k * SW + j0);
    const float av[4] = {a.x, a.y, a.z, a.w}, wv[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
    for (int ii = 0; ii < 4; ++ii)
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) acc[ii][jj] += av[ii] * wv[jj];
  }
#pragma unroll
  for (int ii = 0; ii < 4; ++ii)
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) Ws[(i0 + ii) * SW + j0 + jj] = acc[ii][jj];
  __syncthreads();  // W complete; C^T no longer needed
  {  // P: thread t reads half t % 2 of row t / 2 as 16 independent float4 loads
    const int i = t / 2, k0 = (t % 2) * (NB / 2);
    const float4* rp = (const float4*)(P + i * NB + k0);
    float4 w[NB / 8];
#pragma unroll
    for (int q = 0; q < NB / 8; ++q) w[q] = rp[q];
#pragma unroll
    for (int q = 0; q < NB / 8; ++q) {
      Xt[(k0 + 4 * q) * LD + i] = w[q].x;
      Xt[(k0 + 4 * q + 1) * LD + i] = w[q].y;
      Xt[(k0 + 4 * q + 2) * LD + i] = w[q].z;
      Xt[(k0 + 4 * q + 3) * LD + i] = w[q].w;
    }
  }
  __syncthreads();
  float q[4][4] = {};
  for (int k = 0; k < NB; ++k) {
    const float4 a = *(const float4*)(Xt + k * LD + i0);
    const float4 w = *(const float4*)(Ws + k * SW + j0);
    const float av[4] = {a.x, a.y, a.z, a.w}, wv[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
    for (int ii = 0; ii < 4; ++ii)
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) q[ii][jj] -= av[ii] * wv[jj];
  }
  const int per = lf / CB, p = b % per;  // 256-blocks per lf-block; this one's position
  uint16_t* out = dst + (int64_t)(b / per) * lf * lf + (int64_t)p * CB * (lf + 1);
  // Q's quadrant: rows 128.., columns s0.. (lower) or rows 0.., columns 128 + s0.. (upper)
  const int qr = UPPER ? 0 : NB, qc = UPPER ? NB + s0 : s0;
#pragma unroll
  for (int ii = 0; ii < 4; ++ii)
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) out[(int64_t)(qr + i0 + ii) * lf + qc + j0 + jj] = f2bf(q[ii][jj]);
  // the other three quadrants' columns of this slab: inv(A) at (0, 0), inv(D) at (128, 128),
  // zeros in the quadrant opposite Q
  for (int e = t; e < NB * SW; e += 256) {
    const int i = e / SW, j = s0 + e % SW;
    out[(int64_t)i * lf + j] = f2bf(Ai[i * NB + j]);
    out[(int64_t)(NB + i) * lf + NB + j] = f2bf(Di[i * NB + j]);
    out[(int64_t)(UPPER ? NB + i : i) * lf + (UPPER ? j : NB + j)] = 0;
  }
  // the same two slabs of columns (s0 .., 128 + s0 ..) of the 256-blocks of this column
  // outside the triangle: above the diagonal (lower), below it (upper)
  const int q0 = UPPER ? p + 1 : 0, q1 = UPPER ? per : p;
  for (int qb = q0; qb < q1; ++qb) {  // 16-byte stores: lf, s0 and the block offsets are multiples of 8
    uint16_t* z = out + (int64_t)(qb - p) * CB * lf;
    for (int e = t; e < CB * (SW / 8); e += 256) {
      const int64_t r = (int64_t)(e / (SW / 8)) * lf + s0 + 8 * (e % (SW / 8));
      *(uint4*)(z + r) = make_uint4(0, 0, 0, 0);
      *(uint4*)(z + r + NB) = make_uint4(0, 0, 0, 0);
    }
  }
}

// dst[r][c] = src[r][c] for an rows x cols bf16 block (both row-major with their own
// leading dimensions), and zeros in dst columns cols .. cols_pad - 1; with `vec` (both
// 16-byte aligned, leading dimensions and cols multiples of 8, no padding) 8 elements per
// 16-byte load and store.
__global__ __launch_bounds__(256) void copy2d_kernel(const uint16_t* __restrict__ src, int64_t lds,
                                                     uint16_t* __restrict__ dst, int64_t ldd, int rows, int cols,
                                                     int cols_pad, int vec) {
  if (vec) {
    const int g = cols / 8;
    const int64_t total = (int64_t)rows * g;
    for (int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x; e < total; e += (int64_t)gridDim.x * 256) {
      const int r = (int)(e / g), c = (int)(e % g) * 8;
      *(uint4*)(dst + (int64_t)r * ldd + c) = *(const uint4*)(src + (int64_t)r * lds + c);
    }
    return;
  }
  const int64_t total = (int64_t)rows * cols_pad;
  for (int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x; e < total; e += (int64_t)gridDim.x * 256) {
    const int r = (int)(e / cols_pad), c = (int)(e % cols_pad);
    dst[(int64_t)r * ldd + c] = c < cols ? src[(int64_t)r * lds + c] : (uint16_t)0;
  }
}

// dst[c][r] = src[r][c] for an rows x cols bf16 matrix: 64 x 64 blocks through LDS, rows
// read and written as 16-byte vectors when `vec` (both 16-byte aligned, leading dimensions
// multiples of 8), else element by element.  dst rows are padded with zeros up to a
// multiple of 8 columns (dst columns rows .. round_up(rows, 8) - 1).
__global__ __launch_bounds__(256) void transpose_kernel(const uint16_t* __restrict__ src, int64_t lds,
                                                       uint16_t* __restrict__ dst, int64_t ldd, int rows, int cols,
                                                       int vec) {
  __shared__ uint16_t tile[SB][SB + 2];  // tile[y][x] = src[r0 + y][c0 + x]; 33-word rows: column reads spread over the banks
  const int r0 = blockIdx.y * SB, c0 = blockIdx.x * SB;
  for (int e = threadIdx.x; e < SB * SB / 8; e += 256) {
    const int y = e / (SB / 8), x8 = (e % (SB / 8)) * 8;
    const int r = r0 + y, c = c0 + x8;
    uint16_t v[8];
    if (vec && r < rows && c + 7 < cols) {
      const uint4 w = *(const uint4*)(src + (int64_t)r * lds + c);
      v[0] = (uint16_t)w.x; v[1] = (uint16_t)(w.x >> 16); v[2] = (uint16_t)w.y; v[3] = (uint16_t)(w.y >> 16);
      v[4] = (uint16_t)w.z; v[5] = (uint16_t)(w.z >> 16); v[6] = (uint16_t)w.w; v[7] = (uint16_t)(w.w >> 16);
    } else {
#pragma unroll
      for (int k = 0; k < 8; ++k) v[k] = r < rows && c + k < cols ? src[(int64_t)r * lds + c + k] : (uint16_t)0;
    }
#pragma unroll
    for (int k = 0; k < 8; ++k) tile[y][x8 + k] = v[k];
  }
  __syncthreads();
  const int rows_pad = (rows + 7) / 8 * 8;
  for (int e = threadIdx.x; e < SB * SB / 8; e += 256) {
    const int x = e / (SB / 8), y8 = (e % (SB / 8)) * 8;  // dst row c0 + x, columns r0 + y8 ..
    const int dr = c0 + x, dc = r0 + y8;
    if (dr >= cols || dc >= rows_pad) continue;
    uint16_t v[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) v[k] = tile[y8 + k][x];  // zero past `rows` (filled above)
    if (vec) {
      uint4 w;
      w.x = v[0] | ((uint32_t)v[1] << 16);
      w.y = v[2] | ((uint32_t)v[3] << 16);
      w.z = v[4] | ((uint32_t)v[5] << 16);
      w.w = v[6] | ((uint32_t)v[7] << 16);
      *(uint4*)(dst + (int64_t)dr * ldd + dc) = w;
    } else {
#pragma unroll
      for (int k = 0; k < 8; ++k) dst[(int64_t)dr * ldd + dc + k] = v[k];
    }
  }
}

unsigned blocks_for(int64_t work) {
  int64_t b = (work + 255) / 256;
  if (b < 1) b = 1;
  return (unsigned)b;
}

}  // namespace

hipError_t launch_expand_tri(const void* src, int64_t lds, void* dst, int64_t ldd, int r0, int c0, int rows, int cols,
                             int cols_pad, int uplo, int unit, hipStream_t s) {
  const int vec = ((uintptr_t)src % 16 == 0) && lds % 8 == 0 && c0 % 8 == 0;
  hipLaunchKernelGGL(expand_tri_kernel, dim3(blocks_for((int64_t)rows * (cols_pad / 8))), dim3(256), 0, s,
                     (const uint16_t*)src, lds, (uint16_t*)dst, ldd, r0, c0, rows, cols, cols_pad, uplo, unit, vec);
  return hipGetLastError();
}

hipError_t launch_expand_tri_trans(const void* src, int64_t lds, void* dst, int64_t ldd, int r0, int c0, int rows,
                                   int cols, int cols_pad, int n, int uplo, int unit, hipStream_t s) {
  const int vec = ((uintptr_t)src % 16 == 0) && lds % 8 == 0 && r0 % 8 == 0;
  dim3 grid((unsigned)((cols_pad + SB - 1) / SB), (unsigned)((rows + SB - 1) / SB));
  hipLaunchKernelGGL(expand_tri_trans_kernel, grid, dim3(256), 0, s, (const uint16_t*)src, lds, (uint16_t*)dst, ldd,
                     r0, c0, rows, cols, cols_pad, n, uplo, unit, vec);
  return hipGetLastError();
}

hipError_t launch_expand_sym(const void* src, int64_t lds, void* dst, int64_t ldd, int r0, int c0, int rows, int cols,
                             int cols_pad, int n, int uplo, hipStream_t s) {
  const int vec = ((uintptr_t)src % 16 == 0) && lds % 8 == 0 && r0 % 8 == 0 && c0 % 8 == 0;
  if (vec && (uintptr_t)dst % 16 == 0 && ldd % 8 == 0 && rows % SB == 0 && cols % SB == 0 && cols_pad == cols &&
      r0 + rows <= n && c0 + cols <= n && rows > 0 && cols > 0) {
    const int bcols = cols / SB, nblocks = (rows / SB) * bcols;
    hipLaunchKernelGGL(expand_sym_blocks_kernel, dim3((unsigned)((nblocks + 3) / 4)), dim3(256), 0, s,
                       (const uint16_t*)src, lds, (uint16_t*)dst, ldd, r0, c0, bcols, nblocks, uplo);
    return hipGetLastError();
  }
  dim3 grid((unsigned)((cols_pad + SB - 1) / SB), (unsigned)((rows + SB - 1) / SB));
  hipLaunchKernelGGL(expand_sym_kernel, grid, dim3(256), 0, s, (const uint16_t*)src, lds, (uint16_t*)dst, ldd, r0, c0,
                     rows, cols, cols_pad, n, uplo, vec);
  return hipGetLastError();
}

hipError_t launch_invert_diag(const void* src, int64_t lds, int n, int uplo, int unit, float* inv128, void* dst,
                              int lf, hipStream_t s) {
  if (lf < kTrsmLeaf || lf % kTrsmLeaf != 0) return hipErrorInvalidValue;
  const int blocks = (n + kTrsmLeaf - 1) / kTrsmLeaf;  // 256-blocks; two 128-blocks each
  // with lf > 256, the 128-blocks of T's whole lf-blocks go to dst in bf16 for the doubling
  // products; the 256-blocks of the rest are combined here
  const int whole256 = lf > kTrsmLeaf ? (n / lf) * (lf / kTrsmLeaf) : 0;
  // rows of T readable as 16-byte vectors
  const int vec = ((uintptr_t)src % 16 == 0) && lds % 8 == 0;
  if (uplo == 0)
    hipLaunchKernelGGL(invert_diag_kernel<false>, dim3((unsigned)(2 * blocks)), dim3(kInvThreads), 0, s,
                       (const uint16_t*)src, lds, n, unit, vec, inv128, (uint16_t*)dst, lf, 2 * whole256);
  else
    hipLaunchKernelGGL(invert_diag_kernel<true>, dim3((unsigned)(2 * blocks)), dim3(kInvThreads), 0, s,
                       (const uint16_t*)src, lds, n, unit, vec, inv128, (uint16_t*)dst, lf, 2 * whole256);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || whole256 == blocks) return e;
  const dim3 grid((unsigned)(blocks - whole256), kTrsmNB / 32);
  if (uplo == 0)
    hipLaunchKernelGGL(combine_inverse_kernel<false>, grid, dim3(256), 0, s, (const uint16_t*)src, lds, n, vec,
                       (const float*)inv128, (uint16_t*)dst, lf, whole256);
  else
    hipLaunchKernelGGL(combine_inverse_kernel<true>, grid, dim3(256), 0, s, (const uint16_t*)src, lds, n, vec,
                       (const float*)inv128, (uint16_t*)dst, lf, whole256);
  return hipGetLastError();
}

hipError_t launch_transpose(const void* src, int64_t lds, void* dst, int64_t ldd, int rows, int cols, hipStream_t s) {
  const int vec = (uintptr_t)src % 16 == 0 && (uintptr_t)dst % 16 == 0 && lds % 8 == 0 && ldd % 8 == 0;
  dim3 grid((unsigned)((cols + SB - 1) / SB), (unsigned)((rows + SB - 1) / SB));
  hipLaunchKernelGGL(transpose_kernel, grid, dim3(256), 0, s, (const uint16_t*)src, lds, (uint16_t*)dst, ldd, rows,
                     cols, vec);
  return hipGetLastError();
}

hipError_t launch_copy2d(const void* src, int64_t lds, void* dst, int64_t ldd, int rows, int cols, hipStream_t s,
                         int cols_pad) {
  if (cols_pad < cols) cols_pad = cols;
  int64_t b = ((int64_t)rows * cols_pad + 255) / 256;
  if (b > 8192) b = 8192;
  if (b < 1) b = 1;
  const int vec = (uintptr_t)src % 16 == 0 && (uintptr_t)dst % 16 == 0 && lds % 8 == 0 && ldd % 8 == 0 &&
                  cols % 8 == 0 && cols_pad == cols;
  hipLaunchKernelGGL(copy2d_kernel, dim3((unsigned)b), dim3(256), 0, s, (const uint16_t*)src, lds, (uint16_t*)dst, ldd,
                     rows, cols, cols_pad, vec);
  return hipGetLastError();
}

}  // namespace dbgemm
