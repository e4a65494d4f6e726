// LDS read microbenchmark: the LDS -> register rung of the ablation plan measured on
// its own ("cp.async / ldmatrix ablation -- initial plan", section 2.3, second pitfall:
// a load-only loop, no MFMA, so the read instruction's cost is not hidden behind the
// matrix cores).  Each lane reads from 8 host-given LDS byte offsets per iteration with
// one read kind; the same offsets serve every wave of every workgroup.
#include "gemm_internal.h"

namespace dbgemm {
namespace {

constexpr int kProbeLds = 65536;

typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef int i32x2 __attribute__((ext_vector_type(2)));

template <int KIND>
__global__ __launch_bounds__(256) void lds_probe_kernel(LdsProbeOffsets offs, int iters) {
  __shared__ __attribute__((aligned(1024))) char lds[kProbeLds];
  for (int i = threadIdx.x; i < kProbeLds / 4; i += blockDim.x) ((int*)lds)[i] = i;
  __syncthreads();
  const uint32_t base = (uint32_t)(uintptr_t)lds;
  uint32_t a[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) a[j] = base + offs.off[j][threadIdx.x & 63];
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      // the results are not used: asm volatile keeps every read
      if constexpr (KIND == 0) {
        i32x4 v;
        asm volatile("ds_read_b128 %0, %1" : "=v"(v) : "v"(a[j]) : "memory");
      } else if constexpr (KIND == 1) {
        i32x2 v;
        asm volatile("ds_read_b64_tr_b16 %0, %1" : "=v"(v) : "v"(a[j]) : "memory");
      } else if constexpr (KIND == 2) {
        int v;
        asm volatile("ds_read_u16 %0, %1" : "=v"(v) : "v"(a[j]) : "memory");
      } else if constexpr (KIND == 3) {
        i32x2 v;
        asm volatile("ds_read_b64 %0, %1" : "=v"(v) : "v"(a[j]) : "memory");
      } else {
        i32x2 v;
        asm volatile("ds_read_b64_tr_b8 %0, %1" : "=v"(v) : "v"(a[j]) : "memory");
      }
    }
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
  }
}

}  // namespace

int lds_probe_width(int kind) { return kind == 0 ? 16 : kind == 2 ? 2 : kind == 1 || kind == 3 || kind == 4 ? 8 : 0; }

hipError_t launch_lds_probe(int kind, const LdsProbeOffsets& offs, int iters, int workgroups, hipStream_t s) {
  switch (kind) {
    case 0: hipLaunchKernelGGL(lds_probe_kernel<0>, dim3(workgroups), dim3(256), 0, s, offs, iters); break;
    case 1: hipLaunchKernelGGL(lds_probe_kernel<1>, dim3(workgroups), dim3(256), 0, s, offs, iters); break;
    case 2: hipLaunchKernelGGL(lds_probe_kernel<2>, dim3(workgroups), dim3(256), 0, s, offs, iters); break;
    case 3: hipLaunchKernelGGL(lds_probe_kernel<3>, dim3(workgroups), dim3(256), 0, s, offs, iters); break;
    default: hipLaunchKernelGGL(lds_probe_kernel<4>, dim3(workgroups), dim3(256), 0, s, offs, iters); break;
  }
  return hipGetLastError();
}

}  // namespace dbgemm
