// bf16 -> block-scaled E4M3 ("MXFP8") along rows: the weight/activation quantisation in
// front of the MXFP8 GEMMs of the fused profile protocol (section "SM103 MXFP8 QKV
// weight-quantization diagnostics": read bf16, amax of each 32-element group, a UE8M0
// scale, E4M3 conversion, write).  The scale rule is the OCP microscaling one: exponent
// floor(log2(amax)) - 8 (8 = the largest E4M3 exponent), clamped to the UE8M0 range and
// stored as that + 127 (an all-zero group stores 0); each element is x / 2^(e-127)
// rounded to the nearest E4M3 value, ties to the even code, saturating at +-448.
// The conversion is integer/RNE arithmetic, exact.
#include "gemm_internal.h"
#include "e4m3_codec.h"

namespace dbgemm {
namespace {

__device__ inline float bf16f(uint16_t b) { return __builtin_bit_cast(float, (uint32_t)b << 16); }

// UE8M0 scale byte of a group with largest magnitude amax (0 for an all-zero group).
__device__ inline int mx_scale(float amax) {
  if (!(amax > 0.0f)) return 0;
  int ex;  // floor(log2(amax)); amax is a bf16 value, normal or subnormal in fp32
  const uint32_t ab = __builtin_bit_cast(uint32_t, amax);
  if ((ab >> 23) != 0u)
    ex = (int)(ab >> 23) - 127;
  else
    ex = -126 - (__builtin_clz(ab) - 8 - 1) - 1;  // subnormal: 2^-149 * mantissa
  const int e = ex - 8 + 127;
  return e < 0 ? 0 : (e > 254 ? 254 : e);
}

// Four lanes per 32-element group, 8 elements (16 bytes of bf16) each: a wave reads 1 KiB of
// a row and writes 512 bytes of codes, both contiguous.  The group's amax is reduced over its
// four neighbouring lanes, and its first lane writes the scale byte.
__global__ __launch_bounds__(256) void quantize_mx_kernel(int64_t rows, int64_t cols, const uint16_t* src,
                                                          int64_t ld_src, uint8_t* dst, int64_t ld_dst,
                                                          uint8_t* scales, int64_t ld_scales) {
  typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
  typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
  const int64_t nb = (cols + 31) / 32;
  const int64_t per_row = 4 * nb;  // 8-element chunks per row, whole groups
  // x: chunks of a row (a multiple of 4 per block: a group's lanes enter and leave together);
  // y: rows, grid-strided, two per iteration
  const int64_t k = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (k >= per_row) return;
  const int64_t b = k / 4;
  const int64_t c0 = b * 32 + (k % 4) * 8;
  const int n = cols - c0 >= 8 ? 8 : (cols > c0 ? (int)(cols - c0) : 0);
  auto load = [&](int64_t r, float* v) {
    const uint16_t* s = src + r * ld_src + c0;
    if (n == 8 && ((uintptr_t)s & 15u) == 0) {
      const u32x4 w = *(const u32x4*)s;
#pragma unroll
      for (int h = 0; h < 4; ++h) {
        v[2 * h] = __builtin_bit_cast(float, w[h] << 16);
        v[2 * h + 1] = __builtin_bit_cast(float, w[h] & 0xFFFF0000u);
      }
    } else {
#pragma unroll
      for (int j = 0; j < 8; ++j) v[j] = j < n ? bf16f(s[j]) : 0.0f;
    }
  };
  auto finish = [&](int64_t r, const float* v) {
    float amax = 0.0f;
#pragma unroll
    for (int j = 0; j < 8; ++j) amax = __builtin_fmaxf(amax, __builtin_fabsf(v[j]));  // NaN does not set it
    amax = __builtin_fmaxf(amax, __shfl_xor(amax, 1));
    amax = __builtin_fmaxf(amax, __shfl_xor(amax, 2));
    const int e = mx_scale(amax);
    if (k % 4 == 0) scales[r * ld_scales + b] = (uint8_t)e;
    // x / 2^(e-127) = x * 2^(127-e): exact (the results stay below 512 in magnitude)
    const float inv = e == 254 ? 0x1p-127f : __builtin_bit_cast(float, (uint32_t)(254 - e) << 23);
    uint8_t* d = dst + r * ld_dst + c0;
    if (n == 8 && ((uintptr_t)d & 7u) == 0) {
      // the conversion instruction after saturating to +-448: the same codes as e4m3_from_f32
      *(u32x2*)d = (u32x2){e4m3x4_from_f32(v[0] * inv, v[1] * inv, v[2] * inv, v[3] * inv),
                           e4m3x4_from_f32(v[4] * inv, v[5] * inv, v[6] * inv, v[7] * inv)};
    } else {
#pragma unroll
      for (int j = 0; j < 8; ++j)
        if (j < n) d[j] = (uint8_t)e4m3_from_f32(v[j] * inv);
    }
  };
  // two rows per iteration, both loads issued before either is used
  for (int64_t r = blockIdx.y; r < rows; r += 2 * (int64_t)gridDim.y) {
    const int64_t r2 = r + gridDim.y;
    float v[8], v2[8];
    load(r, v);
    if (r2 < rows) load(r2, v2);
    finish(r, v);
    if (r2 < rows) finish(r2, v2);
  }
}

}  // namespace

hipError_t launch_quantize_mx(int64_t rows, int64_t cols, const void* src, int64_t ld_src, void* dst,
                              int64_t ld_dst, uint8_t* scales, int64_t ld_scales, hipStream_t s) {
  const int64_t per_row = 4 * ((cols + 31) / 32);
  const int64_t bx = (per_row + 255) / 256;
  if (bx > 65535) return hipErrorInvalidConfiguration;  // rows past kQuantizeMaxCols (the host checks)
  const int64_t half = (rows + 1) / 2;  // two rows per workgroup and iteration
  const int64_t by = half < 65535 ? half : 65535;
  hipLaunchKernelGGL(quantize_mx_kernel, dim3((unsigned)bx, (unsigned)(by > 0 ? by : 1)), dim3(256), 0, s, rows, cols,
                     (const uint16_t*)src, ld_src, (uint8_t*)dst, ld_dst, scales, ld_scales);
  return hipGetLastError();
}

}  // namespace dbgemm
