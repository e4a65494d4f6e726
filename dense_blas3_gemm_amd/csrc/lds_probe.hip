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

// The value of one dword of a read's result (keeps the results used).
__device__ __forceinline__ int first_dword(int v) { return v; }
__device__ __forceinline__ int first_dword(i32x2 v) { return v[0]; }
__device__ __forceinline__ int first_dword(i32x4 v) { return v[0]; }

// The 8 reads of one iteration in one statement that also waits for them, so that no read is
// in flight when the statement ends (the compiler takes an asm statement's outputs as written
// when it ends).  SUFFIX follows the address operand (the second offset of a paired read).
#define DBGEMM_LDS8(INSN, SUFFIX, T)                                                                  \
  {                                                                                                 \
    T v0, v1, v2, v3, v4, v5, v6, v7;                                                               \
    asm volatile(INSN " %0, %8" SUFFIX "\n\t" INSN " %1, %9" SUFFIX "\n\t" INSN " %2, %10" SUFFIX       \
                 "\n\t" INSN " %3, %11" SUFFIX "\n\t" INSN " %4, %12" SUFFIX "\n\t" INSN " %5, %13" SUFFIX  \
                 "\n\t" INSN " %6, %14" SUFFIX "\n\t" INSN " %7, %15" SUFFIX "\n\ts_waitcnt lgkmcnt(0)"      \
                 : "=&v"(v0), "=&v"(v1), "=&v"(v2), "=&v"(v3), "=&v"(v4), "=&v"(v5), "=&v"(v6), "=&v"(v7)   \
                 : "v"(a[0]), "v"(a[1]), "v"(a[2]), "v"(a[3]), "v"(a[4]), "v"(a[5]), "v"(a[6]), "v"(a[7])   \
                 : "memory");                                                                       \
    sink ^= first_dword(v0) ^ first_dword(v1) ^ first_dword(v2) ^ first_dword(v3) ^ first_dword(v4) ^     \
            first_dword(v5) ^ first_dword(v6) ^ first_dword(v7);                                      \
  }

template <int KIND>
__global__ __launch_bounds__(256) void lds_probe_kernel(LdsProbeOffsets offs, int iters, int* sink_out) {
  __shared__ __attribute__((aligned(1024))) char lds[kProbeLds];
  for (int i = threadIdx.x; i < kProbeLds / 4; i += blockDim.x) ((int*)lds)[i] = i;
  __syncthreads();
  const uint32_t base = (uint32_t)(uintptr_t)lds;
  uint32_t a[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) a[j] = base + offs.off[j][threadIdx.x & 63];
  int sink = 0;
  for (int it = 0; it < iters; ++it) {
    if constexpr (KIND == 0) DBGEMM_LDS8("ds_read_b128", "", i32x4)
    else if constexpr (KIND == 1) DBGEMM_LDS8("ds_read_b64_tr_b16", "", i32x2)
    else if constexpr (KIND == 2) DBGEMM_LDS8("ds_read_u16", "", int)
    else if constexpr (KIND == 3) DBGEMM_LDS8("ds_read_b64", "", i32x2)
    else if constexpr (KIND == 4) DBGEMM_LDS8("ds_read_b64_tr_b8", "", i32x2)
    else DBGEMM_LDS8("ds_read2st64_b64", " offset1:4", i32x4)  // 8 bytes at the offset and at + 2048
  }
  // the results feed a value that is stored only if it matches a pattern the fill never
  // produces, so the reads are kept and the store never happens
  if (sink == 0x7fffffff && sink_out) sink_out[0] = sink;
}
#undef DBGEMM_LDS8

}  // namespace

int lds_probe_width(int kind) { return kind == 0 ? 16 : kind == 2 ? 2 : kind >= 1 && kind <= 5 ? 8 : 0; }
int lds_probe_span(int kind) { return kind == 5 ? 2048 + 8 : lds_probe_width(kind); }

hipError_t launch_lds_probe(int kind, const LdsProbeOffsets& offs, int iters, int workgroups, hipStream_t s) {
  switch (kind) {
    case 0: hipLaunchKernelGGL(lds_probe_kernel<0>, dim3(workgroups), dim3(256), 0, s, offs, iters, nullptr); break;
    case 1: hipLaunchKernelGGL(lds_probe_kernel<1>, dim3(workgroups), dim3(256), 0, s, offs, iters, nullptr); break;
    case 2: hipLaunchKernelGGL(lds_probe_kernel<2>, dim3(workgroups), dim3(256), 0, s, offs, iters, nullptr); break;
    case 3: hipLaunchKernelGGL(lds_probe_kernel<3>, dim3(workgroups), dim3(256), 0, s, offs, iters, nullptr); break;
    case 4: hipLaunchKernelGGL(lds_probe_kernel<4>, dim3(workgroups), dim3(256), 0, s, offs, iters, nullptr); break;
    default: hipLaunchKernelGGL(lds_probe_kernel<5>, dim3(workgroups), dim3(256), 0, s, offs, iters, nullptr); break;
  }
  return hipGetLastError();
}

}  // namespace dbgemm
