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

// Items of the block inversion below: item it = s * (NB / G) + g is row group g of step s,
// which updates rows r > k (lower) or r < k (upper) with k = s or NB - 1 - s.
template <bool UPPER, int NB, int G>
constexpr bool item_has_work(int it) {
  const int s = it / (NB / G), g = it % (NB / G), k = UPPER ? NB - 1 - s : s;
  return UPPER ? g * G < k : g * G + G - 1 > k;
}
template <bool UPPER, int NB, int G>
constexpr int next_item(int it) {  // the next item with work after it, or -1
  for (int j = it + 1; j < NB * (NB / G); ++j)
    if (item_has_work<UPPER, NB, G>(j)) return j;
  return -1;
}
template <bool UPPER, int NB, int G>
constexpr int item_slot(int it) {  // register buffer of item it: alternates over the items with work
  int n = 0;
  for (int j = 0; j < it; ++j) n += item_has_work<UPPER, NB, G>(j) ? 1 : 0;
  return n & 1;
}

// f(integral_constant<int, 0>) ... f(integral_constant<int, N - 1>), expanded at compile time
template <int N, int I = 0, class F>
__device__ __forceinline__ void cfor(F&& f) {
  if constexpr (I < N) {
    f(std::integral_constant<int, I>{});
    cfor<N, I + 1>(f);
  }
}

// dst[r][c] (r < rows, c < cols, leading dimension ldd) = T[r0 + r][c0 + c] of the n x n
// triangular matrix T.  One thread per 8 consecutive columns of one row; columns past
// `cols` up to the padded width are written as zeros.
__global__ __launch_bounds__(256) void expand_tri_kernel(const uint16_t* __restrict__ src, int64_t lds,
                                                         uint16_t* __restrict__ dst, int64_t ldd, int r0, int c0,
                                                         int rows, int cols, int cols_pad, int uplo, int unit) {
  const int groups = cols_pad / 8;
  const int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (t >= (int64_t)rows * groups) return;
  const int r = (int)(t / groups), c8 = (int)(t % groups) * 8;
  const int i = r0 + r;
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
  uint4 w;
  w.x = v[0] | ((uint32_t)v[1] << 16);
  w.y = v[2] | ((uint32_t)v[3] << 16);
  w.z = v[4] | ((uint32_t)v[5] << 16);
  w.w = v[6] | ((uint32_t)v[7] << 16);
  *(uint4*)(dst + (int64_t)r * ldd + c8) = w;
}

// dst[r][c] = S[r0 + r][c0 + c] of the symmetric matrix S whose uplo triangle is stored
// in src.  Workgroup (bx, by) writes the 64 x 64 output block at rows 64*by, columns
// 64*bx; its elements come from src directly where (i, j) is referenced and from the
// mirrored block (read row-wise, transposed in LDS) elsewhere.  Columns past `cols` up to
// the padded width are zeros.
constexpr int SB = 64;
__global__ __launch_bounds__(256) void expand_sym_kernel(const uint16_t* __restrict__ src, int64_t lds,
                                                         uint16_t* __restrict__ dst, int64_t ldd, int r0, int c0,
                                                         int rows, int cols, int cols_pad, int n, int uplo) {
  __shared__ uint16_t mir[SB][SB + 2];
  const int br = blockIdx.y * SB, bc = blockIdx.x * SB;  // output block origin
  const int gi0 = r0 + br, gj0 = c0 + bc;                  // in S
  // does the block need the mirror (any element outside the stored triangle)?
  const bool need_mirror = uplo == 0 ? (gi0 < gj0 + SB - 1) : (gi0 + SB - 1 > gj0);
  if (need_mirror) {
    // mir[x][y] = src[gj0 + y][gi0 + x] (row gj0 + y of src, read along its columns)
    for (int e = threadIdx.x; e < SB * SB; e += 256) {
      const int y = e / SB, x = e % SB;
      const int si = gj0 + y, sj = gi0 + x;
      uint16_t v = 0;
      if (si < n && sj < n && referenced(si, sj, uplo)) v = src[(int64_t)si * lds + sj];
      mir[x][y] = v;
    }
  }
  __syncthreads();
  for (int e = threadIdx.x; e < SB * SB; e += 256) {
    const int y = e / SB, x = e % SB;
    const int r = br + y, c = bc + x;
    if (r >= rows || c >= cols_pad) continue;
    const int i = r0 + r, j = c0 + c;
    uint16_t v = 0;
    if (c < cols && i < n && j < n) v = referenced(i, j, uplo) ? src[(int64_t)i * lds + j] : mir[y][x];
    dst[(int64_t)r * ldd + c] = v;
  }
}

// Inverse of each diagonal block T_bb (rows and columns [b*NB, b*NB + nb), nb = NB except
// for a shorter last block) of the n x n triangular T, padded to NB x NB with the
// identity.  Workgroup b, thread c computes column c of inv(T_bb) by column-oriented
// substitution in fp32 with the whole column in registers: for each k in order
// (ascending for a lower block, descending for an upper one), x_k = b_k / T_kk, then
// b_r -= T_rk * x_k for the rows r still to come.  The updates of one step are
// independent, so the loop is bound by FMA issue, not by latency; T is kept transposed in
// LDS so that column k is one broadcast row.  The result, zeros outside the triangle, is
// stored in fp32 at dst + b*NB*NB, [NB][NB]; blocks past n are the identity.
template <bool UPPER>
__global__ __launch_bounds__(kTrsmNB) void invert_diag_kernel(const uint16_t* __restrict__ src, int64_t lds, int n,
                                                              int unit, float* __restrict__ dst) {
  constexpr int NB = kTrsmNB;
  constexpr int LD = NB + 4;  // row stride of Tt: float4-aligned, 4-way bank spread on the transposing writes
  __shared__ __attribute__((aligned(16))) float Tt[NB * LD];  // Tt[k * LD + r] = T[r][k]
  const int b = blockIdx.x, o = b * NB;
  const int nb = n - o < NB ? n - o : NB;
  const int c = threadIdx.x;
  for (int e = c; e < NB * NB; e += NB) {  // thread c reads column c of row e / NB
    const int i = e / NB, j = e % NB;
    float v = 0.f;
    if (i == j && (unit || i >= nb)) v = 1.f;
    else if (i < nb && j < nb && (UPPER ? i <= j : i >= j)) v = bf16f(src[(int64_t)(o + i) * lds + o + j]);
    Tt[j * LD + i] = v;
  }
  __syncthreads();
  float x[NB];
#pragma unroll
  for (int r = 0; r < NB; ++r) x[r] = r == c ? 1.f : 0.f;
  // The updates of step s (k = s, or NB-1-s for an upper block) touch rows in 32-row
  // groups; item (s, g) needs the 32 values T[32g .. 32g+31][k].  T never changes, so the
  // values of the next item that has rows to update are read from LDS one item ahead (two
  // register buffers) and the read latency hides behind the current item's FMAs.  Every
  // index is a compile-time constant, so x stays in registers.
  constexpr int G = 32, NG = NB / G;
  float4 buf[2][G / 4];
  auto load = [&](auto item, float4* dstb) {
    constexpr int s = decltype(item)::value / NG, g = decltype(item)::value % NG;
    constexpr int k = UPPER ? NB - 1 - s : s;
    const float4* col = (const float4*)(Tt + k * LD + g * G);
#pragma unroll
    for (int q = 0; q < G / 4; ++q) dstb[q] = col[q];
  };
  constexpr int first = next_item<UPPER, NB, G>(-1);
  load(std::integral_constant<int, first>{}, buf[0]);
  cfor<NB>([&](auto sc) {
    constexpr int s = decltype(sc)::value;
    constexpr int k = UPPER ? NB - 1 - s : s;
    x[k] = x[k] / Tt[k * LD + k];  // x_k, before the updates of its step
    cfor<NG>([&](auto gc) {
      constexpr int g = decltype(gc)::value, it = s * NG + g;
      if constexpr (item_has_work<UPPER, NB, G>(it)) {
        constexpr int nxt = next_item<UPPER, NB, G>(it);
        constexpr int slot = item_slot<UPPER, NB, G>(it);
        if constexpr (nxt >= 0) load(std::integral_constant<int, nxt>{}, buf[slot ^ 1]);
        const float* v = (const float*)buf[slot];
        cfor<G>([&](auto jc) {
          constexpr int r = g * G + decltype(jc)::value;
          if constexpr (UPPER ? r < k : r > k) x[r] -= v[decltype(jc)::value] * x[k];
        });
        __builtin_amdgcn_sched_barrier(0);
      }
    });
  });
  float* out = dst + (int64_t)b * NB * NB;
#pragma unroll
  for (int r = 0; r < NB; ++r) out[r * NB + c] = x[r];
}

// Inverse of each 2 x 2 block of the 128-block inverses: the 256 x 256 diagonal block
// b of T, [A 0; C D] (lower) or [A C; 0 D] (upper), has the inverse
//   lower: [inv(A) 0; -inv(D) C inv(A)  inv(D)],   upper: [inv(A)  -inv(A) C inv(D); 0 inv(D)],
// i.e. Q = -P (C R) with (P, R) = (inv(D), inv(A)) or (inv(A), inv(D)).  Workgroup (b, s)
// computes columns [32s, 32s + 32) of Q in fp32 (W = C R[:, cols], then Q = -P W, each
// thread a 4 x 4 register tile) and writes columns 32s .. 32s + 31 of both halves of the
// block, rounded once to bf16, at dst + b*256*256, [256][256].  inv holds the fp32 128-block
// inverses, block 2b = inv(A), 2b + 1 = inv(D).
constexpr int CB = 2 * kTrsmNB;  // the combined block edge
template <bool UPPER>
__global__ __launch_bounds__(256) void combine_inverse_kernel(const uint16_t* __restrict__ src, int64_t lds, int n,
                                                              const float* __restrict__ inv,
                                                              uint16_t* __restrict__ dst) {
  constexpr int NB = kTrsmNB, SW = 32, LD = NB + 4;
  __shared__ __attribute__((aligned(16))) float Xt[NB * LD];  // C^T, then P^T: Xt[k*LD + i] = X[i][k]
  __shared__ __attribute__((aligned(16))) float Rs[NB * SW];  // R[:, cols]
  __shared__ __attribute__((aligned(16))) float Ws[NB * SW];  // W = C R[:, cols]
  const int b = blockIdx.x, s0 = blockIdx.y * SW, t = threadIdx.x;
  const int o = b * CB;
  const float* Ai = inv + (int64_t)(2 * b) * NB * NB;
  const float* Di = Ai + NB * NB;
  const float* P = UPPER ? Ai : Di;
  const float* R = UPPER ? Di : Ai;
  // C: rows o+128.., columns o.. (lower) or rows o.., columns o+128.. (upper) of T
  const int cr = UPPER ? o : o + NB, cc = UPPER ? o + NB : o;
  for (int e = t; e < NB * NB; e += 256) {
    const int i = e / NB, k = e % NB;
    const int gi = cr + i, gk = cc + k;
    Xt[k * LD + i] = gi < n && gk < n ? bf16f(src[(int64_t)gi * lds + gk]) : 0.f;
  }
  for (int e = t; e < NB * SW; e += 256) Rs[e] = R[(e / SW) * NB + s0 + e % SW];
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
  for (int e = t; e < NB * NB; e += 256) {
    const int i = e / NB, k = e % NB;
    Xt[k * LD + i] = P[e];
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
  uint16_t* out = dst + (int64_t)b * CB * CB;
  // Q's quadrant: rows 128.., columns s0.. (lower) or rows 0.., columns 128 + s0.. (upper)
  const int qr = UPPER ? 0 : NB, qc = UPPER ? NB + s0 : s0;
#pragma unroll
  for (int ii = 0; ii < 4; ++ii)
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) out[(qr + i0 + ii) * CB + qc + j0 + jj] = f2bf(q[ii][jj]);
  // the other three quadrants' columns of this slab: inv(A) at (0, 0), inv(D) at (128, 128),
  // zeros in the quadrant opposite Q
  for (int e = t; e < NB * SW; e += 256) {
    const int i = e / SW, j = s0 + e % SW;
    out[i * CB + j] = f2bf(Ai[i * NB + j]);
    out[(NB + i) * CB + NB + j] = f2bf(Di[i * NB + j]);
    out[(UPPER ? NB + i : i) * CB + (UPPER ? j : NB + j)] = 0;
  }
}

// dst[r][c] = src[r][c] for an rows x cols bf16 block (both row-major with their own
// leading dimensions).
__global__ __launch_bounds__(256) void copy2d_kernel(const uint16_t* __restrict__ src, int64_t lds,
                                                     uint16_t* __restrict__ dst, int64_t ldd, int rows, int cols) {
  const int64_t total = (int64_t)rows * cols;
  for (int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x; e < total; e += (int64_t)gridDim.x * 256) {
    const int r = (int)(e / cols), c = (int)(e % cols);
    dst[(int64_t)r * ldd + c] = src[(int64_t)r * lds + c];
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
  hipLaunchKernelGGL(expand_tri_kernel, dim3(blocks_for((int64_t)rows * (cols_pad / 8))), dim3(256), 0, s,
                     (const uint16_t*)src, lds, (uint16_t*)dst, ldd, r0, c0, rows, cols, cols_pad, uplo, unit);
  return hipGetLastError();
}

hipError_t launch_expand_sym(const void* src, int64_t lds, void* dst, int64_t ldd, int r0, int c0, int rows, int cols,
                             int cols_pad, int n, int uplo, hipStream_t s) {
  dim3 grid((unsigned)((cols_pad + SB - 1) / SB), (unsigned)((rows + SB - 1) / SB));
  hipLaunchKernelGGL(expand_sym_kernel, grid, dim3(256), 0, s, (const uint16_t*)src, lds, (uint16_t*)dst, ldd, r0, c0,
                     rows, cols, cols_pad, n, uplo);
  return hipGetLastError();
}

hipError_t launch_invert_diag(const void* src, int64_t lds, int n, int uplo, int unit, float* inv128, void* dst,
                              hipStream_t s) {
  const int blocks = (n + kTrsmLeaf - 1) / kTrsmLeaf;  // 256-blocks; two 128-blocks each
  if (uplo == 0)
    hipLaunchKernelGGL(invert_diag_kernel<false>, dim3((unsigned)(2 * blocks)), dim3(kTrsmNB), 0, s,
                       (const uint16_t*)src, lds, n, unit, inv128);
  else
    hipLaunchKernelGGL(invert_diag_kernel<true>, dim3((unsigned)(2 * blocks)), dim3(kTrsmNB), 0, s,
                       (const uint16_t*)src, lds, n, unit, inv128);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const dim3 grid((unsigned)blocks, kTrsmNB / 32);
  if (uplo == 0)
    hipLaunchKernelGGL(combine_inverse_kernel<false>, grid, dim3(256), 0, s, (const uint16_t*)src, lds, n,
                       (const float*)inv128, (uint16_t*)dst);
  else
    hipLaunchKernelGGL(combine_inverse_kernel<true>, grid, dim3(256), 0, s, (const uint16_t*)src, lds, n,
                       (const float*)inv128, (uint16_t*)dst);
  return hipGetLastError();
}

hipError_t launch_copy2d(const void* src, int64_t lds, void* dst, int64_t ldd, int rows, int cols, hipStream_t s) {
  int64_t b = ((int64_t)rows * cols + 255) / 256;
  if (b > 8192) b = 8192;
  if (b < 1) b = 1;
  hipLaunchKernelGGL(copy2d_kernel, dim3((unsigned)b), dim3(256), 0, s, (const uint16_t*)src, lds, (uint16_t*)dst, ldd,
                     rows, cols);
  return hipGetLastError();
}

}  // namespace dbgemm
