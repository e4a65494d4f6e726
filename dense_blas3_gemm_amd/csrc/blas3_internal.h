// Internal interfaces of the BLAS3 family (blas3.cpp, blas3_kernels.hip) and the GEMM
// entry it builds on (api.cpp).
#pragma once

#include "gemm.h"
#include "gemm_internal.h"

namespace dbgemm {

// A triangular solve inverts its 128 x 128 diagonal blocks (one workgroup of kTrsmNB
// threads each, fp32), combines pairs of them into the inverses of the 256 x 256 diagonal
// blocks (bf16), and solves kTrsmLeaf rows (columns) at a time with them.
constexpr int kTrsmNB = 128;
constexpr int kTrsmLeaf = 2 * kTrsmNB;

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
  // a batch of equal products (GemmArgs::batch_y ..; the direct-to-LDS kernels only)
  int batch_y = 1, batch_z = 1;
  int64_t bsA[2] = {0, 0}, bsB[2] = {0, 0}, bsC[2] = {0, 0};
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
// dst[r][c] = T^T[r0 + r][c0 + c] for r < rows, c < cols (zeros up to cols_pad): the
// transposed triangular operand, expanded.
hipError_t launch_expand_tri_trans(const void* src, int64_t lds, void* dst, int64_t ldd, int r0, int c0, int rows,
                                   int cols, int cols_pad, int n, int uplo, int unit, hipStream_t s);
hipError_t launch_expand_sym(const void* src, int64_t lds, void* dst, int64_t ldd, int r0, int c0, int rows, int cols,
                             int cols_pad, int n, int uplo, hipStream_t s);
// inv128: 2 * ceil(n / 256) fp32 [128][128] blocks (scratch); dst: ceil(n / lf) bf16
// [lf][lf] blocks (lf a multiple of 256).  With lf = 256, or past T's whole lf-blocks, the
// inverses of T's 256 x 256 diagonal blocks (identity past n) on their diagonals, zeros in
// their 256-blocks outside the triangle; in T's whole lf-blocks (lf > 256), the inverses of
// the 128 x 128 diagonal blocks on the diagonals and zeros in the 128-blocks outside the
// triangle, for the products that double them up to lf x lf.
hipError_t launch_invert_diag(const void* src, int64_t lds, int n, int uplo, int unit, float* inv128, void* dst,
                              int lf, hipStream_t s);
// dst [cols][ldd] = src [rows][lds] transposed (bf16); dst rows zero-padded to a multiple of
// 8 columns (ldd >= round_up(rows, 8)).
hipError_t launch_transpose(const void* src, int64_t lds, void* dst, int64_t ldd, int rows, int cols, hipStream_t s);
// dst [rows][ldd] = src [rows][lds] for cols columns, zeros in columns cols .. cols_pad - 1.
hipError_t launch_copy2d(const void* src, int64_t lds, void* dst, int64_t ldd, int rows, int cols, hipStream_t s,
                         int cols_pad = 0);

}  // namespace dbgemm
