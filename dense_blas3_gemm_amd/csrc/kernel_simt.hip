// Generic GEMM kernels for gfx950: shapes, strides or alignments the MFMA kernels do
// not take, and the beta-only update.  Same operation and conventions as the MFMA
// path (row-major, op(X) = X or X^T, fp32 accumulation, bf16 RNE or fp32 C).
#include "e4m3_codec.h"
#include "gemm_internal.h"

namespace dbgemm {
namespace {

// bf16 and OCP E4M3 ("FN": bias 7, exponent field 0 = subnormals m * 2^-9,
// S.1111.111 = NaN, no infinities) decoded to fp32.
__device__ inline float bf16_to_f32(uint16_t b) { return __builtin_bit_cast(float, (uint32_t)b << 16); }

__device__ inline float e4m3_to_f32(uint8_t b) {
  const uint32_t sign = (uint32_t)(b >> 7) << 31;
  const uint32_t e = (b >> 3) & 0xF, m = b & 0x7;
  if (e == 0xF && m == 0x7) return __builtin_bit_cast(float, sign | 0x7FC00000u);
  if (e == 0) return __builtin_bit_cast(float, sign | __builtin_bit_cast(uint32_t, (float)m * 0x1p-9f));
  return __builtin_bit_cast(float, sign | ((e + 120u) << 23) | (m << 20));
}

__device__ inline float load_in(const void* p, int64_t idx, int fp8) {
  return fp8 ? e4m3_to_f32(((const uint8_t*)p)[idx]) : bf16_to_f32(((const uint16_t*)p)[idx]);
}

// UE8M0 byte -> 2^(e-127) in fp32 (255 is NaN, 0 is the subnormal 2^-127).
__device__ inline float ue8m0_to_f32(uint8_t e) {
  return e == 255 ? __builtin_nanf("") : __builtin_bit_cast(float, e == 0 ? 0x00400000u : (uint32_t)e << 23);
}

__device__ inline float load_c(const void* p, int64_t idx, int kind) {
  if (kind == C_F32) return ((const float*)p)[idx];
  if (kind == C_E4M3) return e4m3_to_f32(((const uint8_t*)p)[idx]);
  return bf16_to_f32(((const uint16_t*)p)[idx]);
}

__device__ inline void store_c(void* p, int64_t idx, int kind, float v) {
  if (kind == C_F32)
    ((float*)p)[idx] = v;
  else if (kind == C_E4M3)
    ((uint8_t*)p)[idx] = (uint8_t)e4m3_from_f32(v);
  else
    ((uint16_t*)p)[idx] = __builtin_bit_cast(uint16_t, static_cast<__bf16>(v));
}

constexpr int TS = 64;  // tile edge
constexpr int TK = 16;  // K step

// 256 threads = 16 x 16, each computing a 4 x 4 block of a 64 x 64 tile.
__global__ __launch_bounds__(256) void gemm_simt_kernel(GemmArgs a) {
  __shared__ float As[TK][TS + 1];
  __shared__ float Bs[TK][TS + 1];
  const int tn = blockIdx.x, tm = blockIdx.y;
  const int m0 = tm * TS, n0 = tn * TS;
  // a triangle of C: tiles that do not meet it have nothing to write
  if (a.tri == TRI_LOWER && m0 + TS - 1 < n0) return;
  if (a.tri == TRI_UPPER && m0 > n0 + TS - 1) return;
  const int tx = threadIdx.x % 16, ty = threadIdx.x / 16;
  float acc[4][4] = {};
  // K band (zeros of an expanded triangular operand outside it are skipped)
  int klo = 0, khi = a.K;
  if (a.kband == KBAND_A_LOWER) khi = min(a.K, a.band_off + m0 + TS);
  if (a.kband == KBAND_A_UPPER) klo = min(a.K, a.band_off + m0);
  if (a.kband == KBAND_B_LOWER) klo = min(a.K, a.band_off + n0);
  if (a.kband == KBAND_B_UPPER) khi = min(a.K, a.band_off + n0 + TS);
  // one pass over K, or two for a dual call (the second on A2, B2)
  for (int pass = 0; pass < (a.dual ? 2 : 1); ++pass) {
  const void* pa = pass ? a.A2 : a.A;
  const void* pb = pass ? a.B2 : a.B;
  const int64_t lda = pass ? a.lda2 : a.lda, ldb = pass ? a.ldb2 : a.ldb;
  for (int k0 = klo; k0 < khi; k0 += TK) {
    for (int e = threadIdx.x; e < TK * TS; e += 256) {
      const int kk = e / TS, x = e % TS;
      const int k = k0 + kk, m = m0 + x, n = n0 + x;
      float av = 0.f, bv = 0.f;
      if (k < khi && m < a.M) {
        av = load_in(pa, a.transA ? (int64_t)k * lda + m : (int64_t)m * lda + k, a.in_fp8);
        if (a.mx) av *= ue8m0_to_f32(a.sa[(int64_t)m * a.ldsa + k / 32]);
      }
      if (k < khi && n < a.N) {
        bv = load_in(pb, a.transB ? (int64_t)n * ldb + k : (int64_t)k * ldb + n, a.in_fp8);
        if (a.mx) bv *= ue8m0_to_f32(a.sb[(int64_t)n * a.ldsb + k / 32]);
      }
      As[kk][x] = av;
      Bs[kk][x] = bv;
    }
    __syncthreads();
#pragma unroll
    for (int kk = 0; kk < TK; ++kk) {
      float ar[4], br[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) ar[i] = As[kk][ty * 4 + i];
#pragma unroll
      for (int j = 0; j < 4; ++j) br[j] = Bs[kk][tx * 4 + j];
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] += ar[i] * br[j];
    }
    __syncthreads();
  }
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int m = m0 + ty * 4 + i;
    if (m >= a.M) continue;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int n = n0 + tx * 4 + j;
      if (n >= a.N) continue;
      if ((a.tri == TRI_LOWER && n > m) || (a.tri == TRI_UPPER && n < m)) continue;
      const int64_t idx = (int64_t)m * a.ldc + n;
      float v = a.alpha * acc[i][j];
      if (a.beta != 0.f) v += a.beta * load_c(a.C, idx, a.c_kind);
      store_c(a.C, idx, a.c_kind, v);
    }
  }
}

// C <- beta * C over M x N (beta == 0 writes zeros without reading C).
__global__ __launch_bounds__(256) void scale_kernel(GemmArgs a) {
  const int64_t total = (int64_t)a.M * a.N;
  for (int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x; e < total; e += (int64_t)gridDim.x * 256) {
    const int m = (int)(e / a.N), n = (int)(e % a.N);
    if ((a.tri == TRI_LOWER && n > m) || (a.tri == TRI_UPPER && n < m)) continue;
    const int64_t idx = (int64_t)m * a.ldc + n;
    const float v = a.beta != 0.f ? a.beta * load_c(a.C, idx, a.c_kind) : 0.f;
    store_c(a.C, idx, a.c_kind, v);
  }
}

}  // namespace

hipError_t launch_simt(const GemmArgs& a, hipStream_t s) {
  dim3 grid((a.N + TS - 1) / TS, (a.M + TS - 1) / TS);
  hipLaunchKernelGGL(gemm_simt_kernel, grid, dim3(256), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_scale(const GemmArgs& a, hipStream_t s) {
  const int64_t total = (int64_t)a.M * a.N;
  int64_t blocks = (total + 255) / 256;
  if (blocks > 4096) blocks = 4096;
  if (blocks < 1) blocks = 1;
  hipLaunchKernelGGL(scale_kernel, dim3((unsigned)blocks), dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace dbgemm
