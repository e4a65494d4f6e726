// bf16 -> block-scaled E4M3 ("MXFP8") along rows: the weight/activation quantisation in
// front of the MXFP8 GEMMs of the fused profile protocol (section "SM103 MXFP8 QKV
// weight-quantization diagnostics": read bf16, amax of each 32-element group, a UE8M0
// scale, E4M3 conversion, write).  The scale rule is the OCP microscaling one: exponent
// floor(log2(amax)) - 8 (8 = the largest E4M3 exponent), clamped to the UE8M0 range and
// stored as that + 127 (an all-zero group stores 0); each element is x / 2^(e-127)
// rounded to the nearest E4M3 value, ties to the even code, saturating at +-448.
// One thread per 32-element group; the conversion is integer/RNE arithmetic, exact.
#include "gemm_internal.h"
#include "e4m3_codec.h"

namespace dbgemm {
namespace {

__device__ inline float bf16f(uint16_t b) { return __builtin_bit_cast(float, (uint32_t)b << 16); }

__global__ __launch_bounds__(256) void quantize_mx_kernel(int64_t rows, int64_t cols, const uint16_t* src,
                                                          int64_t ld_src, uint8_t* dst, int64_t ld_dst,
                                                          uint8_t* scales, int64_t ld_scales) {
  const int64_t nb = (cols + 31) / 32;
  const int64_t total = rows * nb;
  for (int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; t < total;
       t += (int64_t)gridDim.x * blockDim.x) {
    const int64_t r = t / nb, b = t % nb, c0 = b * 32;
    const int n = (int)(cols - c0 < 32 ? cols - c0 : 32);
    const uint16_t* s = src + r * ld_src + c0;
    float v[32];
    float amax = 0.0f;
    if (n == 32 && ((uintptr_t)s & 15u) == 0) {  // a whole aligned group: four 16-byte loads
      typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const u32x4 w = *(const u32x4*)(s + 8 * q);
#pragma unroll
        for (int h = 0; h < 4; ++h) {
          v[8 * q + 2 * h] = __builtin_bit_cast(float, w[h] << 16);
          v[8 * q + 2 * h + 1] = __builtin_bit_cast(float, w[h] & 0xFFFF0000u);
        }
      }
    } else {
#pragma unroll
      for (int j = 0; j < 32; ++j) v[j] = j < n ? bf16f(s[j]) : 0.0f;
    }
#pragma unroll
    for (int j = 0; j < 32; ++j) amax = __builtin_fmaxf(amax, __builtin_fabsf(v[j]));  // NaN does not set it
    int e = 0;
    if (amax > 0.0f) {
      int ex;  // floor(log2(amax)); amax is a bf16 value, normal or subnormal in fp32
      const uint32_t ab = __builtin_bit_cast(uint32_t, amax);
      if ((ab >> 23) != 0u)
        ex = (int)(ab >> 23) - 127;
      else
        ex = -126 - (__builtin_clz(ab) - 8 - 1) - 1;  // subnormal: 2^-149 * mantissa
      e = ex - 8 + 127;
      e = e < 0 ? 0 : (e > 254 ? 254 : e);
    }
    scales[r * ld_scales + b] = (uint8_t)e;
    // x / 2^(e-127) = x * 2^(127-e): exact (the results stay below 512 in magnitude)
    const float inv = e == 254 ? 0x1p-127f : __builtin_bit_cast(float, (uint32_t)(254 - e) << 23);
    uint8_t* d = dst + r * ld_dst + c0;
    if (n == 32 && ((uintptr_t)d & 15u) == 0) {  // two 16-byte stores of packed codes
      typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
#pragma unroll
      for (int q = 0; q < 2; ++q) {
        u32x4 w;
#pragma unroll
        for (int h = 0; h < 4; ++h) {
          const int j = 16 * q + 4 * h;
          w[h] = e4m3_from_f32(v[j] * inv) | (e4m3_from_f32(v[j + 1] * inv) << 8) | (e4m3_from_f32(v[j + 2] * inv) << 16) |
                 (e4m3_from_f32(v[j + 3] * inv) << 24);
        }
        *(u32x4*)(d + 16 * q) = w;
      }
    } else {
#pragma unroll
      for (int j = 0; j < 32; ++j)
        if (j < n) d[j] = (uint8_t)e4m3_from_f32(v[j] * inv);
    }
  }
}

}  // namespace

hipError_t launch_quantize_mx(int64_t rows, int64_t cols, const void* src, int64_t ld_src, void* dst,
                              int64_t ld_dst, uint8_t* scales, int64_t ld_scales, hipStream_t s) {
  const int64_t groups = rows * ((cols + 31) / 32);
  int64_t blocks = (groups + 255) / 256;
  if (blocks > 8192) blocks = 8192;
  if (blocks < 1) blocks = 1;
  hipLaunchKernelGGL(quantize_mx_kernel, dim3((unsigned)blocks), dim3(256), 0, s, rows, cols,
                     (const uint16_t*)src, ld_src, (uint8_t*)dst, ld_dst, scales, ld_scales);
  return hipGetLastError();
}

}  // namespace dbgemm
