// Host side of the single-GPU BLAS3 family (declared and documented in include/gemm.h):
// argument checks, then the GEMM launches, and the operand preparation each operation
// is built from ("BLASMp development notes", section 2: every operator of the library
// runs its local compute on a GEMM).
//
//   SYRK   one GEMM (A and A, the second read transposed) over a triangle of tiles;
//   SYR2K  one GEMM over a triangle of tiles whose K loop runs over both products (the second
//          half of the K tiles reads the other operand pair), on copies of the operands
//          when they are not both K-contiguous with one stride;
//   SYMM   the symmetric matrix expanded into the workspace (row panels), then GEMMs;
//   TRMM   the triangle expanded with zeros into the workspace (panels), then GEMMs whose
//          tiles skip the K tiles that meet only zeros;
//   TRSM   the 256 x 256 diagonal blocks inverted in two launches (fp32 128-block
//          inverses, then their 2 x 2 combination), then a recursive split: solve one half,
//          update the other half with a GEMM (alpha*B - T21*X1), solve it; a leaf block is the
//          product of its inverted diagonal block with its rows (columns) of B.
#include <climits>
#include <cmath>

#include "blas3_internal.h"

using namespace dbgemm;

namespace {

bool bf16_dtype(int d) { return d == GEMM_BF16_BF16 || d == GEMM_BF16_F32; }
int c_bytes(int d) { return d == GEMM_BF16_F32 ? 4 : 2; }
int64_t at_least_1(int64_t v) { return v > 1 ? v : 1; }
int64_t pad8(int64_t v) { return (v + 7) / 8 * 8; }
bool valid_flag(int f) { return f == 0 || f == 1; }
bool size_ok(int64_t v) { return v >= 0 && v <= INT_MAX; }
// Rows the generic kernel's grid can cover (65535 workgroups of 64 rows).  The operations
// below launch several kernels; checking this bound before the first launch keeps an
// unsupported size from failing half way through, with part of the output written.
constexpr int64_t kMaxRows = (int64_t)65535 * 64;
bool rows_ok(int64_t a, int64_t b) { return a <= kMaxRows && b <= kMaxRows; }

const void* off(const void* p, int64_t row, int64_t col, int64_t ld, int es) {
  return (const char*)p + (row * ld + col) * es;
}
void* off(void* p, int64_t row, int64_t col, int64_t ld, int es) { return (char*)p + (row * ld + col) * es; }

// Makes the handle's device current for the lifetime of the object.
struct DeviceGuard {
  int prev = -1;
  bool ok = false, switched = false;
  explicit DeviceGuard(int dev) {
    if (hipGetDevice(&prev) != hipSuccess) return;
    if (prev != dev) {
      if (hipSetDevice(dev) != hipSuccess) return;
      switched = true;
    }
    ok = true;
  }
  ~DeviceGuard() {
    if (switched) (void)hipSetDevice(prev);
  }
};

gemm_status_t status_of(hipError_t e) {
  if (e == hipSuccess) return GEMM_STATUS_SUCCESS;
  return e == hipErrorInvalidConfiguration ? GEMM_STATUS_NOT_SUPPORTED : GEMM_STATUS_LAUNCH_FAILED;
}

// Rows of an n-wide (padded) bf16 panel that fit the workspace, in whole 256-row tiles;
// 0 when not even one tile row fits.
int64_t panel_rows(const HandleView& hv, int64_t n) {
  if (!hv.ws) return 0;
  const int64_t per_row = pad8(n) * 2;
  int64_t p = (int64_t)(hv.ws_bytes / (size_t)per_row) / 256 * 256;
  return p;
}

// Whether a symmetric update with A (and B) stored [K][N] should first copy its `count`
// operands transposed into the workspace: from 2^20 elements per operand (where the copy,
// HBM-bound, costs much less than running the product with both operands M/N-contiguous),
// when the copies fit and the product would then take the fast kernels.
bool transpose_pays(const HandleView& hv, int64_t N, int64_t K, int count) {
  const int64_t ldt = pad8(K);
  if (!hv.ws || N * K < ((int64_t)1 << 20)) return false;
  if ((size_t)count * (size_t)N * ldt * 2 > hv.ws_bytes) return false;
  return gemm_fast_ok(0, 1, N, N, K, hv.ws, ldt, hv.ws, ldt, hv.ws, N, GEMM_BF16_BF16);
}

// The policies a TRSM leaf runs with when it updates its block of B in place: one 256-row
// (left) or 256-column (right) tile spans the whole leaf, so each workgroup reads the part
// of B it overwrites, all of it before its epilogue, and no other workgroup reads it.
int leaf_policy(int side) {
  static const int left = policy_find("bf16_dma_m256n128k64_w4x2_mt16_s3");
  static const int right = policy_find("bf16_dma_m128n256k64_w2x4_mt16_s3");
  return side == GEMM_SIDE_LEFT ? left : right;
}

// The policy of the batched products that double the diagonal inverses.
int doubling_policy() {
  static const int p = policy_find("bf16_dma_m64n64k64_w2x2_mt16_s4");
  return p;
}

struct Trsm {
  HandleView hv;
  int side, transA;
  bool opT_lower;
  int64_t M, N;
  const void* A;
  int64_t lda;
  void* B;
  int64_t ldb;
  // Inverses of T's lf x lf diagonal blocks, [ceil(n / lf)][lf][lf] (lf = 256, 512 or
  // 1024).  With lf > 256 the whole lf-blocks (n / lf of them) start from the 128-block
  // inverses on their diagonals and are completed by doubling (doubled()), and a leaf of lf
  // rows (columns) is one product with the lf-block inverse; the rest of T (a trailing part
  // shorter than lf) holds 256-block inverses and is solved with 256-leaves.
  uint16_t* inv;
  int64_t lf = kTrsmLeaf;
  uint16_t* scratch;  // one block row (column) of B, for leaves that cannot run in place
  // Out of place: every leaf writes its rows (columns) of X to X [M][ldx] in the workspace,
  // the updates read X from there, and one copy moves X into B at the end.  The leaves then
  // take any tile shape (more workgroups than the one-tile-per-leaf in-place form).
  uint16_t* X = nullptr;
  int64_t ldx = 0;
  hipError_t err = hipSuccess;

  void keep(hipError_t e) {
    if (err == hipSuccess && e != hipSuccess) err = e;
  }
  // op(T)[r0 .. , c0 .. ] as a GEMM operand: the stored block and the transpose flag
  const void* opT_block(int64_t r0, int64_t c0) const {
    return transA ? off(A, c0, r0, lda, 2) : off(A, r0, c0, lda, 2);
  }

  // where the solved rows (columns) of X live: X in the workspace, or B itself
  const void* xsrc(int64_t row, int64_t col) const { return X ? off(X, row, col, ldx, 2) : off(B, row, col, ldb, 2); }
  int64_t xld() const { return X ? ldx : ldb; }

  // the inverse of the diagonal block that starts at o (a multiple of 256), leading dimension lf
  const uint16_t* inv_at(int64_t o) const { return inv + (o / lf) * lf * lf + (o % lf) * (lf + 1); }
  bool whole_lf(int64_t o, int64_t nb) const { return lf > kTrsmLeaf && nb == lf && o % lf == 0; }

  // Completes the inverses of the whole lf-blocks: the inverse of a diagonal block
  // [P 0; C R] (lower T) of edge 2h is [inv(P) 0; -inv(R) C inv(P)  inv(R)], and of
  // [P C; 0 R] (upper) [inv(P)  -inv(P) C inv(R); 0 inv(R)].  For h = 128, 256, .. lf/2, two
  // batched products over every 2h-block of every whole lf-block: W = C inv(P) (lower) or
  // C inv(R) (upper) into the workspace, then the off-diagonal block -inv(R) W or
  // -inv(P) W, each rounded to bf16.  The inverses are triangular: each product's K band
  // skips the K tiles that meet only their zeros.
  void doubled(int uplo, int64_t n, uint16_t* W) {
    const int64_t whole = n / lf;
    if (lf == kTrsmLeaf || whole == 0) return;
    const bool lower = uplo == GEMM_LOWER;
    GemmExtras x;
    x.policy = doubling_policy();
    x.batch_z = (int)whole;
    for (int64_t h = kTrsmNB; 2 * h <= lf; h *= 2) {
      const int64_t per = lf / (2 * h);  // 2h-blocks per lf-block
      x.batch_y = (int)per;
      const void* Cb = lower ? off(A, h, 0, lda, 2) : off(A, 0, h, lda, 2);
      const uint16_t* iP = inv;
      const uint16_t* iR = inv + h * (lf + 1);
      uint16_t* Q = lower ? inv + h * lf : inv + h;
      const int64_t sT[2] = {2 * h * (lda + 1), lf * (lda + 1)};
      const int64_t sI[2] = {2 * h * (lf + 1), lf * lf};
      const int64_t sW[2] = {h * h, per * h * h};
      for (int i = 0; i < 2; ++i) {
        x.bsA[i] = sT[i];
        x.bsB[i] = sI[i];
        x.bsC[i] = sW[i];
      }
      x.kband = lower ? KBAND_B_LOWER : KBAND_B_UPPER;
      keep(gemm_enqueue(hv, 0, 0, h, h, h, 1.f, Cb, lda, lower ? iP : iR, lf, 0.f, W, h, GEMM_BF16_BF16, x));
      for (int i = 0; i < 2; ++i) {
        x.bsA[i] = sI[i];
        x.bsB[i] = sW[i];
        x.bsC[i] = sI[i];
      }
      x.kband = lower ? KBAND_A_LOWER : KBAND_A_UPPER;
      keep(gemm_enqueue(hv, 0, 0, h, h, h, -1.f, lower ? iR : iP, lf, W, h, 0.f, Q, lf, GEMM_BF16_BF16, x));
    }
  }

  void leaf(int64_t o, int64_t nb, float alpha) {
    const uint16_t* ib = inv_at(o);
    const int64_t L = lf;
    GemmExtras x;
    // op(inv) is triangular like op(T): the K band skips the tiles of its zeros
    if (side == GEMM_SIDE_LEFT)
      x.kband = opT_lower ? KBAND_A_LOWER : KBAND_A_UPPER;
    else
      x.kband = opT_lower ? KBAND_B_LOWER : KBAND_B_UPPER;
    if (X) {  // out of place: any policy
      if (side == GEMM_SIDE_LEFT)
        keep(gemm_enqueue(hv, transA, 0, nb, N, nb, alpha, ib, L, off(B, o, 0, ldb, 2), ldb, 0.f, off(X, o, 0, ldx, 2),
                          ldx, GEMM_BF16_BF16, x));
      else
        keep(gemm_enqueue(hv, 0, transA, M, nb, nb, alpha, off(B, 0, o, ldb, 2), ldb, ib, L, 0.f, off(X, 0, o, ldx, 2),
                          ldx, GEMM_BF16_BF16, x));
      return;
    }
    const int pol = leaf_policy(side);
    if (side == GEMM_SIDE_LEFT) {  // X rows [o, o+nb) = alpha * op(inv) * B rows
      void* Bb = off(B, o, 0, ldb, 2);
      if (gemm_fast_ok(transA, 0, nb, N, nb, ib, L, Bb, ldb, Bb, ldb, GEMM_BF16_BF16) && pol >= 0) {
        x.policy = pol;
        keep(gemm_enqueue(hv, transA, 0, nb, N, nb, alpha, ib, L, Bb, ldb, 0.f, Bb, ldb, GEMM_BF16_BF16, x));
      } else {
        const int64_t lds = pad8(N);
        keep(gemm_enqueue(hv, transA, 0, nb, N, nb, alpha, ib, L, Bb, ldb, 0.f, scratch, lds, GEMM_BF16_BF16, x));
        keep(launch_copy2d(scratch, lds, Bb, ldb, (int)nb, (int)N, hv.stream));
      }
    } else {  // X columns [o, o+nb) = alpha * B columns * op(inv)
      void* Bb = off(B, 0, o, ldb, 2);
      if (gemm_fast_ok(0, transA, M, nb, nb, Bb, ldb, ib, L, Bb, ldb, GEMM_BF16_BF16) && pol >= 0) {
        x.policy = pol;
        keep(gemm_enqueue(hv, 0, transA, M, nb, nb, alpha, Bb, ldb, ib, L, 0.f, Bb, ldb, GEMM_BF16_BF16, x));
      } else {
        keep(gemm_enqueue(hv, 0, transA, M, nb, nb, alpha, Bb, ldb, ib, L, 0.f, scratch, kTrsmLeaf, GEMM_BF16_BF16,
                          x));
        keep(launch_copy2d(scratch, kTrsmLeaf, Bb, ldb, (int)M, (int)nb, hv.stream));
      }
    }
  }

  // Rows [r0, r0+m) of op(T) X = alpha * B (left side).
  void left(int64_t r0, int64_t m, float alpha) {
    if (m <= kTrsmLeaf || whole_lf(r0, m)) return leaf(r0, m, alpha);
    const int64_t g = m > lf ? lf : kTrsmLeaf;  // whole lf-blocks while they fit
    const int64_t m1 = ((m + 1) / 2 + g - 1) / g * g;
    const GemmExtras x;
    if (opT_lower) {
      left(r0, m1, alpha);
      keep(gemm_enqueue(hv, transA, 0, m - m1, N, m1, -1.f, opT_block(r0 + m1, r0), lda, xsrc(r0, 0), xld(), alpha,
                        off(B, r0 + m1, 0, ldb, 2), ldb, GEMM_BF16_BF16, x));
      left(r0 + m1, m - m1, 1.f);
    } else {
      left(r0 + m1, m - m1, alpha);
      keep(gemm_enqueue(hv, transA, 0, m1, N, m - m1, -1.f, opT_block(r0, r0 + m1), lda, xsrc(r0 + m1, 0), xld(),
                        alpha, off(B, r0, 0, ldb, 2), ldb, GEMM_BF16_BF16, x));
      left(r0, m1, 1.f);
    }
  }

  // Columns [c0, c0+n) of X op(T) = alpha * B (right side).
  void right(int64_t c0, int64_t n, float alpha) {
    if (n <= kTrsmLeaf || whole_lf(c0, n)) return leaf(c0, n, alpha);
    const int64_t g = n > lf ? lf : kTrsmLeaf;
    const int64_t n1 = ((n + 1) / 2 + g - 1) / g * g;
    const GemmExtras x;
    if (!opT_lower) {  // X1 first: X2 op(T)22 = alpha*B2 - X1 op(T)12
      right(c0, n1, alpha);
      keep(gemm_enqueue(hv, 0, transA, M, n - n1, n1, -1.f, xsrc(0, c0), xld(), opT_block(c0, c0 + n1), lda, alpha,
                        off(B, 0, c0 + n1, ldb, 2), ldb, GEMM_BF16_BF16, x));
      right(c0 + n1, n - n1, 1.f);
    } else {  // X2 first: X1 op(T)11 = alpha*B1 - X2 op(T)21
      right(c0 + n1, n - n1, alpha);
      keep(gemm_enqueue(hv, 0, transA, M, n1, n - n1, -1.f, xsrc(0, c0 + n1), xld(), opT_block(c0 + n1, c0), lda,
                        alpha, off(B, 0, c0, ldb, 2), ldb, GEMM_BF16_BF16, x));
      right(c0, n1, 1.f);
    }
  }
};

}  // namespace

extern "C" {

gemm_status_t gemm_syrk(gemm_handle_t h, int uplo, int trans, int64_t N, int64_t K, float alpha, const void* A,
                        int64_t lda, float beta, void* C, int64_t ldc, int dtype) {
  HandleView hv;
  if (!handle_view(h, &hv)) return GEMM_STATUS_NOT_INITIALIZED;
  if (!valid_flag(uplo) || !valid_flag(trans) || !bf16_dtype(dtype)) return GEMM_STATUS_INVALID_VALUE;
  if (!size_ok(N) || !size_ok(K)) return GEMM_STATUS_INVALID_VALUE;
  if (lda < at_least_1(trans ? N : K) || ldc < at_least_1(N)) return GEMM_STATUS_INVALID_VALUE;
  if (!std::isfinite(alpha) || !std::isfinite(beta) || !rows_ok(N, N)) return GEMM_STATUS_NOT_SUPPORTED;
  if (N == 0) return GEMM_STATUS_SUCCESS;
  if (!C || (K > 0 && alpha != 0.f && !A)) return GEMM_STATUS_INVALID_VALUE;
  DeviceGuard g(hv.device);
  if (!g.ok) return GEMM_STATUS_INTERNAL;
  GemmExtras x;
  x.tri = uplo == GEMM_LOWER ? TRI_LOWER : TRI_UPPER;
  if (trans && K > 0 && alpha != 0.f && transpose_pays(hv, N, K, 1)) {
    // A [K][N] is copied once as A^T [N][K] into the workspace, so the product runs with both
    // operands K-contiguous (the 192-wide tile, plain LDS reads)
    const int64_t ldt = pad8(K);
    hipError_t e = launch_transpose(A, lda, hv.ws, ldt, (int)K, (int)N, hv.stream);
    if (e == hipSuccess) e = gemm_enqueue(hv, 0, 1, N, N, K, alpha, hv.ws, ldt, hv.ws, ldt, beta, C, ldc, dtype, x);
    return status_of(e);
  }
  return status_of(gemm_enqueue(hv, trans, 1 - trans, N, N, K, alpha, A, lda, A, lda, beta, C, ldc, dtype, x));
}

gemm_status_t gemm_syr2k(gemm_handle_t h, int uplo, int trans, int64_t N, int64_t K, float alpha, const void* A,
                         int64_t lda, const void* B, int64_t ldb, float beta, void* C, int64_t ldc, int dtype) {
  HandleView hv;
  if (!handle_view(h, &hv)) return GEMM_STATUS_NOT_INITIALIZED;
  if (!valid_flag(uplo) || !valid_flag(trans) || !bf16_dtype(dtype)) return GEMM_STATUS_INVALID_VALUE;
  if (!size_ok(N) || !size_ok(K)) return GEMM_STATUS_INVALID_VALUE;
  const int64_t row = at_least_1(trans ? N : K);
  if (lda < row || ldb < row || ldc < at_least_1(N)) return GEMM_STATUS_INVALID_VALUE;
  if (!std::isfinite(alpha) || !std::isfinite(beta) || !rows_ok(N, N)) return GEMM_STATUS_NOT_SUPPORTED;
  if (N == 0) return GEMM_STATUS_SUCCESS;
  if (!C || (K > 0 && alpha != 0.f && (!A || !B))) return GEMM_STATUS_INVALID_VALUE;
  DeviceGuard g(hv.device);
  if (!g.ok) return GEMM_STATUS_INTERNAL;
  GemmExtras x;
  x.tri = uplo == GEMM_LOWER ? TRI_LOWER : TRI_UPPER;
  x.dual = 1;  // op(A) op(B)^T, then op(B) op(A)^T, in one K loop and one fp32 sum
  if (K > 0 && alpha != 0.f) {
    // A [N][K], B [N][K] with one stride: straight onto the direct-to-LDS kernels
    if (!trans && lda == ldb && gemm_fast_ok(0, 1, N, N, K, A, lda, B, ldb, C, ldc, dtype)) {
      x.A2 = B;
      x.lda2 = ldb;
      x.B2 = A;
      x.ldb2 = lda;
      return status_of(gemm_enqueue(hv, 0, 1, N, N, K, alpha, A, lda, B, ldb, beta, C, ldc, dtype, x));
    }
    // Otherwise, from 2^16 elements and when both fit the workspace: op(A) and op(B) copied
    // K-contiguous with a common stride (transposed when trans is set), then the same product.
    const int64_t Kp = pad8(K);
    if (N * K >= ((int64_t)1 << 16) && hv.ws && (size_t)2 * N * Kp * 2 <= hv.ws_bytes) {
      uint16_t* At = (uint16_t*)hv.ws;
      uint16_t* Bt = At + N * Kp;
      auto pack = [&](const void* X, int64_t ldx_, uint16_t* dst) {
        return trans ? launch_transpose(X, ldx_, dst, Kp, (int)K, (int)N, hv.stream)
                     : launch_copy2d(X, ldx_, dst, Kp, (int)N, (int)K, hv.stream, (int)Kp);
      };
      hipError_t e = pack(A, lda, At);
      if (e == hipSuccess) e = pack(B, ldb, Bt);
      x.A2 = Bt;
      x.lda2 = Kp;
      x.B2 = At;
      x.ldb2 = Kp;
      if (e == hipSuccess) e = gemm_enqueue(hv, 0, 1, N, N, K, alpha, At, Kp, Bt, Kp, beta, C, ldc, dtype, x);
      return status_of(e);
    }
  }
  // small, or no room to copy: both products in one K loop of the generic kernel
  x.A2 = B;
  x.lda2 = ldb;
  x.B2 = A;
  x.ldb2 = lda;
  return status_of(gemm_enqueue(hv, trans, 1 - trans, N, N, K, alpha, A, lda, B, ldb, beta, C, ldc, dtype, x));
}

gemm_status_t gemm_symm(gemm_handle_t h, int side, int uplo, int64_t M, int64_t N, float alpha, const void* A,
                        int64_t lda, const void* B, int64_t ldb, float beta, void* C, int64_t ldc, int dtype) {
  HandleView hv;
  if (!handle_view(h, &hv)) return GEMM_STATUS_NOT_INITIALIZED;
  if (!valid_flag(side) || !valid_flag(uplo) || !bf16_dtype(dtype)) return GEMM_STATUS_INVALID_VALUE;
  if (!size_ok(M) || !size_ok(N)) return GEMM_STATUS_INVALID_VALUE;
  const int64_t n = side == GEMM_SIDE_LEFT ? M : N;
  if (lda < at_least_1(n) || ldb < at_least_1(N) || ldc < at_least_1(N)) return GEMM_STATUS_INVALID_VALUE;
  if (!std::isfinite(alpha) || !std::isfinite(beta) || !rows_ok(M, N)) return GEMM_STATUS_NOT_SUPPORTED;
  if (M == 0 || N == 0) return GEMM_STATUS_SUCCESS;
  if (!C || (alpha != 0.f && (!A || !B))) return GEMM_STATUS_INVALID_VALUE;
  DeviceGuard g(hv.device);
  if (!g.ok) return GEMM_STATUS_INTERNAL;
  const int es = c_bytes(dtype);
  const GemmExtras x;
  if (alpha == 0.f)  // C <- beta*C
    return status_of(gemm_enqueue(hv, 0, 0, M, N, 0, 0.f, nullptr, 1, nullptr, 1, beta, C, ldc, dtype, x));
  const int64_t P = panel_rows(hv, n);
  if (P <= 0) return GEMM_STATUS_NOT_SUPPORTED;
  const int64_t npad = pad8(n);
  hipError_t err = hipSuccess;
  // Left: C rows [p0, p0+rows) = alpha * S[p0 .., :] B + beta * C.  Right: C columns
  // [p0, p0+rows) = alpha * B S[:, p0 ..] + beta * C, with S[:, p0 ..] = S[p0 .., :]^T.
  const int64_t outer = side == GEMM_SIDE_LEFT ? M : N;
  for (int64_t p0 = 0; p0 < outer && err == hipSuccess; p0 += P) {
    const int64_t rows = outer - p0 < P ? outer - p0 : P;
    err = launch_expand_sym(A, lda, hv.ws, npad, (int)p0, 0, (int)rows, (int)n, (int)npad, (int)n, uplo, hv.stream);
    if (err != hipSuccess) break;
    if (side == GEMM_SIDE_LEFT)
      err = gemm_enqueue(hv, 0, 0, rows, N, n, alpha, hv.ws, npad, B, ldb, beta, off(C, p0, 0, ldc, es), ldc, dtype,
                         x);
    else
      err = gemm_enqueue(hv, 0, 1, M, rows, n, alpha, B, ldb, hv.ws, npad, beta, off(C, 0, p0, ldc, es), ldc, dtype,
                         x);
  }
  return status_of(err);
}

gemm_status_t gemm_trmm(gemm_handle_t h, int side, int uplo, int transA, int diag, int64_t M, int64_t N, float alpha,
                        const void* A, int64_t lda, const void* B, int64_t ldb, void* C, int64_t ldc, int dtype) {
  HandleView hv;
  if (!handle_view(h, &hv)) return GEMM_STATUS_NOT_INITIALIZED;
  if (!valid_flag(side) || !valid_flag(uplo) || !valid_flag(transA) || !valid_flag(diag) || !bf16_dtype(dtype))
    return GEMM_STATUS_INVALID_VALUE;
  if (!size_ok(M) || !size_ok(N)) return GEMM_STATUS_INVALID_VALUE;
  const int64_t n = side == GEMM_SIDE_LEFT ? M : N;
  if (lda < at_least_1(n) || ldb < at_least_1(N) || ldc < at_least_1(N)) return GEMM_STATUS_INVALID_VALUE;
  if (!std::isfinite(alpha) || !rows_ok(M, N)) return GEMM_STATUS_NOT_SUPPORTED;
  if (M == 0 || N == 0) return GEMM_STATUS_SUCCESS;
  if (!C || (alpha != 0.f && (!A || !B))) return GEMM_STATUS_INVALID_VALUE;
  DeviceGuard g(hv.device);
  if (!g.ok) return GEMM_STATUS_INTERNAL;
  const int es = c_bytes(dtype);
  if (alpha == 0.f)  // C <- 0
    return status_of(gemm_enqueue(hv, 0, 0, M, N, 0, 0.f, nullptr, 1, nullptr, 1, 0.f, C, ldc, dtype, GemmExtras{}));
  const int64_t P = panel_rows(hv, n);
  if (P <= 0) return GEMM_STATUS_NOT_SUPPORTED;
  const bool opT_lower = (uplo == GEMM_LOWER) != (transA != 0);
  hipError_t err = hipSuccess;
  const int64_t outer = side == GEMM_SIDE_LEFT ? M : N;
  for (int64_t p0 = 0; p0 < outer && err == hipSuccess; p0 += P) {
    const int64_t w = outer - p0 < P ? outer - p0 : P;  // rows (left) / columns (right) of C
    GemmExtras x;
    x.band_off = (int)p0;
    // The panel of op(T) this part of C needs -- rows [p0, p0+w) of op(T) (left) or its
    // columns (right) -- expanded as op(T) itself (transposed from T when transA is set), so
    // that the product is always NN (the fastest layout of the kernels).
    int64_t ldw;
    if (side == GEMM_SIDE_LEFT) {  // op(T) rows [p0, p0+w) x all n columns
      ldw = pad8(n);
      err = transA ? launch_expand_tri_trans(A, lda, hv.ws, ldw, (int)p0, 0, (int)w, (int)n, (int)ldw, (int)n, uplo,
                                             diag, hv.stream)
                   : launch_expand_tri(A, lda, hv.ws, ldw, (int)p0, 0, (int)w, (int)n, (int)ldw, uplo, diag, hv.stream);
    } else {  // op(T) all n rows x columns [p0, p0+w)
      ldw = pad8(w);
      err = transA ? launch_expand_tri_trans(A, lda, hv.ws, ldw, 0, (int)p0, (int)n, (int)w, (int)ldw, (int)n, uplo,
                                             diag, hv.stream)
                   : launch_expand_tri(A, lda, hv.ws, ldw, 0, (int)p0, (int)n, (int)w, (int)ldw, uplo, diag, hv.stream);
    }
    if (err != hipSuccess) break;
    if (side == GEMM_SIDE_LEFT) {  // C rows = alpha * op(T)[p0.., :] B
      x.kband = opT_lower ? KBAND_A_LOWER : KBAND_A_UPPER;
      err = gemm_enqueue(hv, 0, 0, w, N, M, alpha, hv.ws, ldw, B, ldb, 0.f, off(C, p0, 0, ldc, es), ldc, dtype, x);
    } else {  // C columns = alpha * B op(T)[:, p0..]
      x.kband = opT_lower ? KBAND_B_LOWER : KBAND_B_UPPER;
      err = gemm_enqueue(hv, 0, 0, M, w, N, alpha, B, ldb, hv.ws, ldw, 0.f, off(C, 0, p0, ldc, es), ldc, dtype, x);
    }
  }
  return status_of(err);
}

gemm_status_t gemm_trsm(gemm_handle_t h, int side, int uplo, int transA, int diag, int64_t M, int64_t N, float alpha,
                        const void* A, int64_t lda, void* B, int64_t ldb, int dtype) {
  HandleView hv;
  if (!handle_view(h, &hv)) return GEMM_STATUS_NOT_INITIALIZED;
  if (!valid_flag(side) || !valid_flag(uplo) || !valid_flag(transA) || !valid_flag(diag) || dtype != GEMM_BF16_BF16)
    return GEMM_STATUS_INVALID_VALUE;
  if (!size_ok(M) || !size_ok(N)) return GEMM_STATUS_INVALID_VALUE;
  const int64_t n = side == GEMM_SIDE_LEFT ? M : N;
  if (lda < at_least_1(n) || ldb < at_least_1(N)) return GEMM_STATUS_INVALID_VALUE;
  if (!std::isfinite(alpha) || !rows_ok(M, N)) return GEMM_STATUS_NOT_SUPPORTED;
  if (M == 0 || N == 0) return GEMM_STATUS_SUCCESS;
  if (!B || (alpha != 0.f && !A)) return GEMM_STATUS_INVALID_VALUE;
  DeviceGuard g(hv.device);
  if (!g.ok) return GEMM_STATUS_INTERNAL;
  if (alpha == 0.f)  // X = 0
    return status_of(gemm_enqueue(hv, 0, 0, M, N, 0, 0.f, nullptr, 1, nullptr, 1, 0.f, B, ldb, dtype, GemmExtras{}));
  // workspace: the diagonal inverses (bf16), the fp32 128-block inverses they are made
  // from, the doubling products' W, and X (out of place) or one leaf's rows (columns) of B
  // for leaves that cannot run in place
  auto up256 = [](size_t v) { return (v + 255) / 256 * 256; };
  const int64_t blocks = (n + kTrsmLeaf - 1) / kTrsmLeaf;
  auto inv_bytes_of = [&](int64_t e) { return up256((size_t)((n + e - 1) / e) * e * e * 2); };
  auto w_bytes_of = [&](int64_t e) { return e > kTrsmLeaf ? up256((size_t)(n / e) * e * e / 2) : (size_t)0; };
  const size_t inv128_bytes = up256((size_t)2 * blocks * kTrsmNB * kTrsmNB * 4);
  const size_t scratch_bytes = side == GEMM_SIDE_LEFT ? (size_t)kTrsmLeaf * pad8(N) * 2 : (size_t)M * kTrsmLeaf * 2;
  if (!hv.ws || inv_bytes_of(kTrsmLeaf) + inv128_bytes + scratch_bytes > hv.ws_bytes) return GEMM_STATUS_NOT_SUPPORTED;
  // Out of place for large right-hand sides (from 2^20 elements of B), when X fits beside
  // the inverses: its one copy back is cheaper than leaves limited to one tile per leaf.
  // Out of place, the leaves are lf-blocks: the largest of 1024 and 512 that T holds twice,
  // when T's rows can be read as 16-byte vectors (the batched doubling products) and
  // everything fits; else 256.
  const int64_t ldx = pad8(N);
  const size_t x_bytes = (size_t)M * ldx * 2;
  const bool out_of_place = M * N >= ((int64_t)1 << 20);
  int64_t lf = kTrsmLeaf;
  if (out_of_place && (uintptr_t)A % 16 == 0 && lda % 8 == 0 && doubling_policy() >= 0) {
    for (int64_t e = 4 * kTrsmLeaf; e > kTrsmLeaf; e /= 2)
      if (n >= 2 * e && inv_bytes_of(e) + inv128_bytes + w_bytes_of(e) + x_bytes <= hv.ws_bytes) {
        lf = e;
        break;
      }
  }
  const size_t inv_bytes = inv_bytes_of(lf), w_bytes = w_bytes_of(lf);
  Trsm t;
  t.hv = hv;
  t.side = side;
  t.transA = transA;
  t.opT_lower = (uplo == GEMM_LOWER) != (transA != 0);
  t.M = M;
  t.N = N;
  t.A = A;
  t.lda = lda;
  t.B = B;
  t.ldb = ldb;
  t.inv = (uint16_t*)hv.ws;
  t.lf = lf;
  float* inv128 = (float*)((char*)hv.ws + inv_bytes);
  uint16_t* W = (uint16_t*)((char*)hv.ws + inv_bytes + inv128_bytes);
  t.scratch = (uint16_t*)((char*)hv.ws + inv_bytes + inv128_bytes + w_bytes);
  if (out_of_place && inv_bytes + inv128_bytes + w_bytes + x_bytes <= hv.ws_bytes) {
    t.X = t.scratch;
    t.ldx = ldx;
  }
  t.keep(launch_invert_diag(A, lda, (int)n, uplo, diag, inv128, t.inv, (int)lf, hv.stream));
  if (t.err == hipSuccess) t.doubled(uplo, n, W);
  if (t.err == hipSuccess) {
    if (side == GEMM_SIDE_LEFT)
      t.left(0, M, alpha);
    else
      t.right(0, N, alpha);
  }
  if (t.err == hipSuccess && t.X) t.keep(launch_copy2d(t.X, ldx, B, ldb, (int)M, (int)N, hv.stream));
  return status_of(t.err);
}

}  // extern "C"
