// Hardware microbenchmarks behind the kernels' bounds: the MFMA issue rate and the shader
// clock under full load, and the direct-to-LDS copy rate per CU with a GEMM's panel pattern.
// Each isolates one stage of the GEMM pipeline ("cp.async / ldmatrix ablation -- initial
// plan", section 2.3: a stage timed alone), so that the pipeline's measured time can be
// set against what each stage costs by itself.
#include "gemm_internal.h"
#include "mfma_common.h"

namespace dbgemm {
namespace {

// MFMA issue: every wave runs `iters` clusters of 32 16x16x32 (MT 16) or 16 32x32x16 (MT 32)
// bf16 MFMAs on register operands, four independent accumulators (no chain stalls).  With
// PP the two groups of four waves take turns, one cluster each between workgroup
// barriers, as the ping-pong GEMM does; otherwise all eight waves issue at once.
// cycles[b] = s_memtime (shader clock cycles) after the workgroup's last cluster minus
// before its first, taken by wave 0 of workgroup b.
template <int MT, bool PP>
__global__ __launch_bounds__(512) void probe_mfma_kernel(unsigned long long* cycles, int iters) {
  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  bf16x8 a, b;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    a[e] = (__bf16)(0.25f * (float)((lane * 7 + e * 13) % 29) - 3.0f);
    b[e] = (__bf16)(0.125f * (float)((lane * 5 + e * 3) % 31) - 2.0f);
  }
  const int grp = wave >> 2;
  float sum;
  __syncthreads();
  const unsigned long long t0 = __builtin_amdgcn_s_memtime();
  if constexpr (MT == 16) {
    f32x4 acc[4] = {};
    for (int t = 0; t < iters; ++t) {
#pragma unroll
      for (int ph = 0; ph < (PP ? 2 : 1); ++ph) {
        if (!PP || ph == grp) {
#pragma unroll
          for (int i = 0; i < 32; ++i) acc[i & 3] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, acc[i & 3], 0, 0, 0);
        }
        if constexpr (PP) __syncthreads();
      }
    }
    sum = acc[0][0] + acc[1][1] + acc[2][2] + acc[3][3];
  } else {
    f32x16 acc[4] = {};
    for (int t = 0; t < iters; ++t) {
#pragma unroll
      for (int ph = 0; ph < (PP ? 2 : 1); ++ph) {
        if (!PP || ph == grp) {
#pragma unroll
          for (int i = 0; i < 16; ++i) acc[i & 3] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc[i & 3], 0, 0, 0);
        }
        if constexpr (PP) __syncthreads();
      }
    }
    sum = acc[0][0] + acc[1][5] + acc[2][10] + acc[3][15];
  }
  // the workgroup's time: the last wave's end (waves sharing a SIMD need not keep pace)
  __syncthreads();
  const unsigned long long t1 = __builtin_amdgcn_s_memtime();
  // the sums keep every MFMA (the operands make this value impossible)
  if (threadIdx.x == 0) cycles[blockIdx.x] = sum == 1.0e30f ? 0ull : t1 - t0;
}

// Direct-to-LDS copy rate: workgroup b copies `iters` tiles of 256 rows x RB bytes from
// rows [256 (b % panels), +256) of a [rows][pitch]-byte buffer, tile t from byte column
// (t * RB) % pitch, into two LDS slots in turn; each wave waits for its copies of the
// previous tile while those of the current one are in flight (the ring kernels' depth).
// 8 waves; each copy instruction moves 1 KiB (64 lanes x 16 bytes).
template <int RB>
__global__ __launch_bounds__(512) void probe_copy_kernel(unsigned long long* cycles, const char* src, int64_t rows,
                                                         int64_t pitch, int iters) {
  constexpr int CPR = RB / 16;           // 16-byte chunks per row
  constexpr int IPW = 256 * RB / 1024 / 8;  // copies per wave per tile
  __shared__ __attribute__((aligned(1024))) char lds[2 * 256 * RB];
  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int panels = (int)(rows / 256);
  const int64_t base = (int64_t)(blockIdx.x % panels) * 256 * pitch;
  const __amdgpu_buffer_rsrc_t r = make_rsrc(src + base, (uint32_t)(256 * pitch));
  uint32_t off[IPW];
#pragma unroll
  for (int i = 0; i < IPW; ++i) {
    const int p = (wave * IPW + i) * 64 + lane;
    off[i] = (uint32_t)((p / CPR) * pitch) + (uint32_t)(p % CPR) * 16u;
  }
  const uint32_t lds0 = (uint32_t)(uintptr_t)(lds_char*)lds;
  __syncthreads();
  const unsigned long long t0 = __builtin_amdgcn_s_memtime();
  for (int t = 0; t < iters; ++t) {
    const uint32_t col = (uint32_t)(((int64_t)t * RB) % pitch);
    const uint32_t l0 = lds0 + (uint32_t)(t & 1) * (256u * RB) + (uint32_t)(wave * IPW) * 1024u;
#pragma unroll
    for (int i = 0; i < IPW; ++i) {
      uint32_t saved;
      asm volatile(
          "s_mov_b32 %0, m0\n\ts_mov_b32 m0, %1\n\ts_nop 0\n\tbuffer_load_dwordx4 %2, %3, 0 offen lds\n\t"
          "s_mov_b32 m0, %0"
          : "=&s"(saved)
          : "s"(l0 + (uint32_t)i * 1024u), "v"(off[i] + col), "s"(r)
          : "memory");
    }
    asm volatile("s_waitcnt vmcnt(%0)" ::"n"(IPW) : "memory");
  }
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  const unsigned long long t1 = __builtin_amdgcn_s_memtime();
  __syncthreads();
  if (threadIdx.x == 0) cycles[blockIdx.x] = t1 - t0;
}

}  // namespace

hipError_t launch_hw_probe(int kind, int param, int iters, int workgroups, const void* src, int64_t src_bytes,
                           unsigned long long* cycles, hipStream_t s) {
  const dim3 g(workgroups), b(512);
  switch (kind) {
    case 0:
      if (param) hipLaunchKernelGGL((probe_mfma_kernel<16, true>), g, b, 0, s, cycles, iters);
      else hipLaunchKernelGGL((probe_mfma_kernel<16, false>), g, b, 0, s, cycles, iters);
      break;
    case 1:
      if (param) hipLaunchKernelGGL((probe_mfma_kernel<32, true>), g, b, 0, s, cycles, iters);
      else hipLaunchKernelGGL((probe_mfma_kernel<32, false>), g, b, 0, s, cycles, iters);
      break;
    default: {
      const int64_t rows = src_bytes / kHwProbePitch;
      const char* p = (const char*)src;
      if (param == 64) hipLaunchKernelGGL((probe_copy_kernel<64>), g, b, 0, s, cycles, p, rows, kHwProbePitch, iters);
      else if (param == 128) hipLaunchKernelGGL((probe_copy_kernel<128>), g, b, 0, s, cycles, p, rows, kHwProbePitch, iters);
      else hipLaunchKernelGGL((probe_copy_kernel<256>), g, b, 0, s, cycles, p, rows, kHwProbePitch, iters);
      break;
    }
  }
  return hipGetLastError();
}

}  // namespace dbgemm
