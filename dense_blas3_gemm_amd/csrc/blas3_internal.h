// Internal interfaces of the BLAS3 family (blas3.cpp, blas3_kernels.hip) and the GEMM
// entry it builds on (api.cpp).
#pragma once

#include "gemm.h"
#include "gemm_internal.h"

namespace dbgemm {

// Rows and columns of the diagonal blocks a triangular solve inverts (one workgroup of
// kTrsmNB threads per block).
constexpr int kTrsmNB = 128;

// What the BLAS3 code needs of a live handle.
struct HandleView {
  int device;
  int cu_count;
  hipStream_t stream;
  void* ws;         // the handle's device workspace, or null
  size_t ws_bytes;
};
bool handle_view(gemm_handle_t h, HandleView* v);  // false for a NULL or destroyed handle

// The parts of a GEMM call beyond gemm_run's arguments (see GemmArgs): a triangle of C,
// a K band, a second product; `policy` forces a table entry (-1: shape-driven choice).
struct GemmExtras {
  int tri = TRI_NONE;
  int kband = KBAND_NONE;
  int band_off = 0;
  int dual = 0;
  const void* A2 = nullptr;
  const void* B2 = nullptr;
  int64_t lda2 = 0, ldb2 = 0;
  int policy = -1;
};

// Enqueues C <- alpha*op(A)*op(B) [+ alpha*op(A2)*op(B2)] + beta*C on the handle's stream;
// the arguments are already checked and the handle's device is current.  With any extra
// set, only the direct-to-LDS bf16 kernels (unsplit) or the generic kernel run.
hipError_t gemm_enqueue(const HandleView& hv, int transA, int transB, int64_t M, int64_t N, int64_t K, float alpha,
                        const void* A, int64_t lda, const void* B, int64_t ldb, float beta, void* C, int64_t ldc,
                        int dtype, const GemmExtras& x);
// Whether the MFMA kernels take these operands (alignment, strides, spans).
bool gemm_fast_ok(int transA, int transB, int64_t M, int64_t N, int64_t K, const void* A, int64_t lda, const void* B,
                  int64_t ldb, const void* C, int64_t ldc, int dtype);

// Operand preparation kernels (blas3_kernels.hip); bf16 throughout.
hipError_t launch_expand_tri(const void* src, int64_t lds, void* dst, int64_t ldd, int r0, int c0, int rows, int cols,
                             int cols_pad, int uplo, int unit, hipStream_t s);
hipError_t launch_expand_sym(const void* src, int64_t lds, void* dst, int64_t ldd, int r0, int c0, int rows, int cols,
                             int cols_pad, int n, int uplo, hipStream_t s);
hipError_t launch_invert_diag(const void* src, int64_t lds, int n, int uplo, int unit, void* dst, hipStream_t s);
hipError_t launch_copy2d(const void* src, int64_t lds, void* dst, int64_t ldd, int rows, int cols, hipStream_t s);

}  // namespace dbgemm
