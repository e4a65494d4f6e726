/*
 * Oracle for the dense GEMM path -- TEST INFRASTRUCTURE ONLY.
 *
 * Only the tests, the smoke check and the CPU-baseline leg of the benchmark load
 * this file's library.  The GPU library never links or calls it, and it shares
 * no code with the GPU library: the storage-format decoders below are written
 * here from the formats' definitions.
 *
 * What it computes is the textbook BLAS level-3 GEMM that all three pages rest
 * on: "BLASMp development notes" (section 1: a BLAS3 framework whose local
 * compute is a GEMM), the "cp.async / ldmatrix ablation" plan (section 2: the
 * bf16 hgemm baseline) and the fused communication/compute profile protocol
 * (sections "v10 backward operators", where the weight-gradient GEMM reads dY
 * transposed and accumulates with beta = 1, and "v12 FP8 boundary", where E4M3
 * operands are multiplied with fp32 accumulation).  None of the pages writes the
 * formula out; the plain reading, which every one of those passages supports, is
 *
 *     R[i][j] = alpha * sum_{k<K} opA(i,k) * opB(k,j) + beta * Cold[i][j]
 *
 * with opA(i,k) = A[i][k] (transA = 0) or A[k][i] (transA = 1) and
 *      opB(k,j) = B[k][j] (transB = 0) or B[j][k] (transB = 1),
 * every matrix row-major with its leading dimension as the row stride.
 *
 * It is evaluated in binary64 by a plain loop: for each output row i, for each k
 * in increasing order, add opA(i,k)*opB(k,j) into an fp64 accumulator of every
 * column j.  Each R[i][j] is therefore summed strictly in k order.  Products of
 * two bf16 or two E4M3 values are exact in binary64.  The same loop also returns
 * S[i][j] = sum_k |opA(i,k)*opB(k,j)|, the scale of the rounding-error allowance.
 *
 * BLAS special cases (the pages are silent; the usual BLAS convention): when
 * beta == 0 the old C is never read, so a NaN there cannot reach R; K == 0 gives
 * R = beta*Cold.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

enum { ORACLE_IN_BF16 = 0, ORACLE_IN_E4M3 = 1 };
enum { ORACLE_C_F32 = 0, ORACLE_C_BF16 = 1, ORACLE_C_E4M3 = 2 };

/* bf16 storage: the upper 16 bits of an IEEE-754 binary32. */
double oracle_bf16_value(uint16_t bits) {
  uint32_t u = (uint32_t)bits << 16;
  float f;
  memcpy(&f, &u, sizeof f);
  return (double)f;
}

double oracle_f32_value(uint32_t bits) {
  float f;
  memcpy(&f, &bits, sizeof f);
  return (double)f;
}

/*
 * OCP 8-bit floating point, E4M3 ("FN") variant: sign, 4 exponent bits with bias
 * 7, 3 mantissa bits.  Exponent field 0 holds zero and the subnormals m * 2^-9;
 * S.1111.111 is NaN; there are no infinities, so S.1111.110 = +-448 is the
 * largest finite magnitude.
 */
double oracle_e4m3_value(uint8_t bits) {
  const int sign = bits >> 7;
  const int e = (bits >> 3) & 0xF;
  const int m = bits & 0x7;
  double v;
  if (e == 0xF && m == 0x7) return NAN;
  if (e == 0)
    v = ldexp((double)m, -9);
  else
    v = ldexp(1.0 + (double)m / 8.0, e - 7);
  return sign ? -v : v;
}

/* Round a binary64 value to the nearest bf16 (ties to even); returns its bits. */
uint16_t oracle_round_bf16(double x) {
  if (isnan(x)) return 0x7FC0;
  const double bf16_max = ldexp(255.0, 120); /* (2 - 2^-7) * 2^127 */
  double ax = fabs(x);
  double r;
  if (ax == 0.0) {
    r = 0.0;
  } else {
    int e;
    frexp(ax, &e); /* ax = f * 2^e with f in [0.5, 1) */
    /* 8 significant bits: quantum 2^(e-8), but never finer than the subnormal
       quantum 2^-133 of the binary32 exponent range. */
    int qexp = e - 8;
    if (qexp < -133) qexp = -133;
    r = ldexp(nearbyint(ldexp(ax, -qexp)), qexp); /* default mode: ties to even */
    /* Values at or past the rounding midpoint above the largest finite bf16 overflow. */
    if (r > bf16_max) r = INFINITY;
  }
  float f = (float)copysign(r, x); /* exact: r has at most 8 significant bits */
  uint32_t u;
  memcpy(&u, &f, sizeof u);
  return (uint16_t)(u >> 16);
}

/* Round a binary64 value to the nearest binary32 (ties to even); returns its bits. */
uint32_t oracle_round_f32(double x) {
  float f = (float)x;
  uint32_t u;
  memcpy(&u, &f, sizeof u);
  return u;
}

static double e4m3_table[256];
static int e4m3_ready = 0;

static void init_tables(void) {
  if (e4m3_ready) return;
  for (int c = 0; c < 256; ++c) e4m3_table[c] = oracle_e4m3_value((uint8_t)c);
  e4m3_ready = 1;
}

static inline double in_value(const void* p, int64_t idx, int fmt) {
  if (fmt == ORACLE_IN_BF16) return oracle_bf16_value(((const uint16_t*)p)[idx]);
  return e4m3_table[((const uint8_t*)p)[idx]];
}

/* The old value of C for the beta term, decoded from C's storage format. */
static inline double c_value(const void* p, int64_t idx, int fmt) {
  if (fmt == ORACLE_C_BF16) return oracle_bf16_value(((const uint16_t*)p)[idx]);
  if (fmt == ORACLE_C_E4M3) return oracle_e4m3_value(((const uint8_t*)p)[idx]);
  return oracle_f32_value(((const uint32_t*)p)[idx]);
}

/*
 * R (and S when not NULL) receive nrows x N values, one row per entry of `rows`
 * (all M rows in order when rows == NULL).  Returns 0, or -1 for bad arguments.
 */
int oracle_gemm(int transA, int transB, int64_t M, int64_t N, int64_t K, double alpha,
                const void* A, int64_t lda, const void* B, int64_t ldb, double beta,
                const void* C, int64_t ldc, int in_fmt, int c_fmt, const int64_t* rows,
                int64_t nrows, double* R, double* S, int nthreads) {
  if (M < 0 || N < 0 || K < 0) return -1;
  if (in_fmt != ORACLE_IN_BF16 && in_fmt != ORACLE_IN_E4M3) return -1;
  if (c_fmt != ORACLE_C_F32 && c_fmt != ORACLE_C_BF16 && c_fmt != ORACLE_C_E4M3) return -1;
  if (rows == NULL) nrows = M;
  if (nrows == 0 || N == 0) return 0;
  init_tables();
  if (nthreads <= 0) nthreads = 1;

  int bad = 0;
#pragma omp parallel for schedule(dynamic, 1) num_threads(nthreads)
  for (int64_t r = 0; r < nrows; ++r) {
    const int64_t i = rows ? rows[r] : r;
    if (i < 0 || i >= M) {
      bad = 1;
      continue;
    }
    double* acc = R + r * N;
    double* sab = S ? S + r * N : NULL;
    for (int64_t j = 0; j < N; ++j) acc[j] = 0.0;
    if (sab)
      for (int64_t j = 0; j < N; ++j) sab[j] = 0.0;
    for (int64_t k = 0; k < K; ++k) {
      const double a = in_value(A, transA ? k * lda + i : i * lda + k, in_fmt);
      if (sab) {
        for (int64_t j = 0; j < N; ++j) {
          const double p = a * in_value(B, transB ? j * ldb + k : k * ldb + j, in_fmt);
          acc[j] += p;
          sab[j] += fabs(p);
        }
      } else {
        for (int64_t j = 0; j < N; ++j)
          acc[j] += a * in_value(B, transB ? j * ldb + k : k * ldb + j, in_fmt);
      }
    }
    for (int64_t j = 0; j < N; ++j) {
      double v = alpha * acc[j];
      if (beta != 0.0) v += beta * c_value(C, i * ldc + j, c_fmt);
      acc[j] = v;
    }
  }
  return bad ? -1 : 0;
}

/*
 * Block-scaled E4M3 GEMM ("MXFP8").  The fused profile protocol's MXFP8 paths (section
 * "SM103 MXFP8 QKV weight-quantization diagnostics": E4M3 elements, one UE8M0 scale
 * per group of 32 along K, obtained from the group's amax) multiply such operands.
 * A UE8M0 byte e stands for 2^(e-127); e = 255 is NaN.  The plain reading of a
 * block-scaled product, with both operands K-contiguous (A stored [M][lda], B stored
 * [N][ldb], one scale byte per row and 32-element K block in SA [M][ldsa] and
 * SB [N][ldsb]):
 *
 *   R[i][j] = alpha * sum_k (A(i,k) * 2^(SA[i][k/32]-127)) * (B(j,k) * 2^(SB[j][k/32]-127))
 *             + beta * Cold[i][j]
 *
 * summed in binary64 in k order like oracle_gemm; every scaled value and every
 * product is exact in binary64.  S receives sum_k |product|.
 */
static inline double mx_scale(uint8_t e) { return e == 255 ? NAN : ldexp(1.0, (int)e - 127); }

int oracle_gemm_mx(int64_t M, int64_t N, int64_t K, double alpha, const uint8_t* A, int64_t lda,
                   const uint8_t* SA, int64_t ldsa, const uint8_t* B, int64_t ldb,
                   const uint8_t* SB, int64_t ldsb, double beta, const void* C, int64_t ldc,
                   int c_fmt, const int64_t* rows, int64_t nrows, double* R, double* S,
                   int nthreads) {
  if (M < 0 || N < 0 || K < 0) return -1;
  if (c_fmt != ORACLE_C_F32 && c_fmt != ORACLE_C_BF16 && c_fmt != ORACLE_C_E4M3) return -1;
  if (rows == NULL) nrows = M;
  if (nrows == 0 || N == 0) return 0;
  init_tables();
  if (nthreads <= 0) nthreads = 1;
  int bad = 0;
#pragma omp parallel for schedule(dynamic, 1) num_threads(nthreads)
  for (int64_t r = 0; r < nrows; ++r) {
    const int64_t i = rows ? rows[r] : r;
    if (i < 0 || i >= M) {
      bad = 1;
      continue;
    }
    double* acc = R + r * N;
    double* sab = S ? S + r * N : NULL;
    for (int64_t j = 0; j < N; ++j) {
      double sum = 0.0, sabs = 0.0;
      for (int64_t k = 0; k < K; ++k) {
        const double a = e4m3_table[A[i * lda + k]] * mx_scale(SA[i * ldsa + k / 32]);
        const double b = e4m3_table[B[j * ldb + k]] * mx_scale(SB[j * ldsb + k / 32]);
        sum += a * b;
        sabs += fabs(a * b);
      }
      double v = alpha * sum;
      if (beta != 0.0) v += beta * c_value(C, i * ldc + j, c_fmt);
      acc[j] = v;
      if (sab) sab[j] = sabs;
    }
  }
  return bad ? -1 : 0;
}

/* Bulk helpers for the Python wrapper. */
void oracle_decode(int fmt, const void* bits, int64_t n, double* out) {
  init_tables();
  for (int64_t i = 0; i < n; ++i) {
    switch (fmt) {
      case 0: out[i] = oracle_bf16_value(((const uint16_t*)bits)[i]); break;
      case 1: out[i] = e4m3_table[((const uint8_t*)bits)[i]]; break;
      default: out[i] = oracle_f32_value(((const uint32_t*)bits)[i]); break;
    }
  }
}

void oracle_round_bf16_array(const double* x, int64_t n, uint16_t* out) {
  for (int64_t i = 0; i < n; ++i) out[i] = oracle_round_bf16(x[i]);
}

void oracle_round_f32_array(const double* x, int64_t n, uint32_t* out) {
  for (int64_t i = 0; i < n; ++i) out[i] = oracle_round_f32(x[i]);
}
