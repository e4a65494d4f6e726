/*
 * gemm.h -- C-ABI of the MI355X (gfx950) dense GEMM library.
 *
 * Operation.  Every entry point that computes evaluates the BLAS level-3 GEMM
 *
 *     C <- alpha * op(A) * op(B) + beta * C,      op(X) = X or X^T,
 *
 * the local compute that the pages are built on: the GEMM under the distributed
 * BLAS3 operators of "BLASMp development notes" (section 1), the bf16 hgemm of the
 * "cp.async / ldmatrix ablation" plan (section 2, fixed baseline M = N = K = 4096),
 * and the projection-backward and FP8 GEMMs of the fused communication/compute
 * profile protocol (sections "formal launch and timing rules": weight gradient with
 * beta = 1 accumulating into bf16, plain mode beta = 0; "v10 backward operators":
 * dW = dY^T X read in place; "v12 FP8 boundary": E4M3 operands, fp32 accumulation,
 * no scales inside the operator).
 *
 * Layout.  Row-major only; the leading dimension is the row stride in elements.
 *   op(A) is M x K: A is stored [M][lda >= K] (transA = 0) or [K][lda >= M] (transA = 1).
 *   op(B) is K x N: B is stored [K][ldb >= N] (transB = 0) or [N][ldb >= K] (transB = 1).
 *   C is stored [M][ldc >= N].
 * A column-major caller uses C^T = op(B)^T op(A)^T.  A transposed operand is read in
 * place; the library never makes a transposed copy.
 *
 * Types.  Inputs are bf16 or OCP E4M3 ("FN": bias 7, no infinities, max 448);
 * products are accumulated in fp32; C is bf16 (round to nearest even) or fp32.
 * E4M3 runs with unit scale: any scaling is the caller's (alpha may carry it).
 *
 * Memory and ownership.  A, B and C are device pointers owned by the caller.  The
 * handle owns its host-side state, one 256 MiB device workspace for split-K, stream-K
 * and the BLAS3 calls, and 64 KiB of stream-K flags (allocated by gemm_create, freed by
 * gemm_destroy).  gemm_run never allocates,
 * never synchronises and returns once the kernel is enqueued on the handle's stream;
 * faults during execution surface at the caller's next synchronisation.  A handle
 * must be used from one host thread at a time, and its calls must not overlap on
 * the device: calls on one stream are ordered, but two streams must not run calls
 * of the same handle concurrently (they would share the workspace).
 *
 * Split-K.  When the output tiles alone would leave CUs idle (small M x N, long K),
 * the policy may split each tile's K range over 2 to 16 workgroups.  Each writes its
 * fp32 partial to the workspace and a second kernel on the same stream adds the
 * partials in split order and applies alpha and beta, so results are deterministic
 * (bitwise the same run to run) but rounded differently from the unsplit sum.
 *
 * Stream-K (by policy name only: "<ping-pong policy>+streamk", see gemm_set_policy).  The
 * whole rounds of tiles over the CUs run one tile per workgroup, and the K loops of the
 * remaining tiles are laid end to end and shared evenly by one further workgroup per CU
 * (or the number the name gives).  The shape-driven choice does not use it: on 160 or 400
 * tiles of 256 x 256 it measured slower than the plain grid (its workgroups sit at
 * scattered K offsets, which costs the L2 reuse of workgroups stepping through K
 * together).  A workgroup whose share starts inside a tile leaves
 * its fp32 partial in the workspace; the workgroup holding the tile's first K steps adds
 * those partials in K order and runs the epilogue.  Results are deterministic for a given
 * shape and device, and rounded differently from the unsplit sum.  The hand-off waits
 * need every workgroup of the call resident on the device in turn; with the device
 * shared by other work for seconds a wait gives up and the tile is written as NaN.
 *
 * Errors.  Arguments are checked before anything is launched; on any error status
 * nothing is launched and nothing is written.
 *
 * Special cases (BLAS convention):  M == 0 or N == 0: nothing to do, SUCCESS.
 * K == 0 or alpha == 0: C <- beta * C.  beta == 0: C is written without being
 * read, so NaN or Inf already in C does not propagate.
 *
 * Fast path.  The MFMA kernels need 16-byte aligned A, B and C, leading dimensions
 * whose byte size is a multiple of 16, and the contiguous extent of each operand
 * (K for a K-contiguous operand, M or N otherwise) a multiple of 8 elements (bf16)
 * or 16 (E4M3).  Anything else runs on a generic kernel: slower, never an error.
 */
#ifndef DENSE_BLAS3_GEMM_AMD_GEMM_H
#define DENSE_BLAS3_GEMM_AMD_GEMM_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct gemm_handle_s* gemm_handle_t;

typedef enum { GEMM_OP_N = 0, GEMM_OP_T = 1 } gemm_op_t;

/* input dtype -> C dtype; accumulation is always fp32 */
typedef enum {
  GEMM_BF16_F32 = 0,    /* bf16 A, B; fp32 C */
  GEMM_BF16_BF16 = 1,   /* bf16 A, B; bf16 C */
  GEMM_E4M3_BF16 = 2,   /* E4M3 A, B; bf16 C */
  GEMM_E4M3_F32 = 3,    /* E4M3 A, B; fp32 C */
  GEMM_MXE4M3_BF16 = 4, /* block-scaled E4M3 A, B (gemm_run_mx only); bf16 C */
  GEMM_MXE4M3_F32 = 5,  /* block-scaled E4M3 A, B (gemm_run_mx only); fp32 C */
  GEMM_E4M3_E4M3 = 6,   /* E4M3 A, B; E4M3 C (see below) */
  GEMM_MXE4M3_E4M3 = 7  /* block-scaled E4M3 A, B (gemm_run_mx only); E4M3 C */
} gemm_dtype_t;
/* E4M3 C (the fp8 data path of the fused-protocol page, "v12 FP8 boundary": inputs and
 * outputs are already E4M3, the scales are the caller's): C <- E4M3(alpha * acc + beta *
 * C_old), with C_old decoded from its E4M3 codes.  The caller folds its output scale into
 * alpha.  Rounding is to the nearest E4M3 value, ties to the even code; magnitudes at or
 * above 448 (and values that round past it) saturate to +-448; NaN stays NaN. */

typedef enum {
  GEMM_STATUS_SUCCESS = 0,
  GEMM_STATUS_INVALID_VALUE = 1,   /* bad size, leading dimension, pointer, op or dtype */
  GEMM_STATUS_NOT_SUPPORTED = 2,   /* well-formed but unsupported (non-finite alpha/beta, policy) */
  GEMM_STATUS_NOT_INITIALIZED = 3, /* NULL or destroyed handle; no usable HIP device */
  GEMM_STATUS_LAUNCH_FAILED = 4,   /* the HIP runtime refused the launch */
  GEMM_STATUS_INTERNAL = 5
} gemm_status_t;

/* Creates a handle bound to HIP device `device`; reads its CU count, builds the
 * tile-policy table and allocates the workspace and the stream-K flags on that device,
 * zeroing the flags and waiting for that (if an allocation fails the handle still works,
 * without split-K and stream-K).  The handle starts on the default stream (NULL).  On
 * error *h is set to NULL. */
gemm_status_t gemm_create(gemm_handle_t* h, int device);

/* Releases the handle and its workspace (hipFree waits for the device's work in
 * flight, so enqueued calls finish first).  NULL is accepted. */
gemm_status_t gemm_destroy(gemm_handle_t h);

/* Binds the hipStream_t (passed as void*) that later gemm_run calls enqueue on.
 * NULL selects the default stream.  The caller keeps ownership of the stream. */
gemm_status_t gemm_set_stream(gemm_handle_t h, void* stream);

/* C <- alpha*op(A)*op(B) + beta*C on the handle's device and stream.  transA and
 * transB take gemm_op_t values, dtype a gemm_dtype_t value.  Device pointers; A and B
 * may be NULL only when the product is empty (M, N or K is 0), C only when M or N
 * is 0. */
gemm_status_t gemm_run(gemm_handle_t h, int transA, int transB, int64_t M, int64_t N,
                       int64_t K, float alpha, const void* A, int64_t lda, const void* B,
                       int64_t ldb, float beta, void* C, int64_t ldc, int dtype);

/* The same call as gemm_run, for callers that cannot allocate device memory: code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc.  It needs no
 * handle and calls no allocating routine.  The split-K and stream-K partials and the
 * stream-K flags, which gemm_run keeps in its handle's workspace, go to a device array
 * instead: GEMM_STATIC_SCRATCH_BYTES of partials, then 64 KiB of flags.
 *
 * The array: the library's code object holds one copy per device it runs on, placed by
 * the loader and held until the process ends.  Every call on a device shares that copy,
 * so calls that overlap on one device (two streams, two host threads) race and must not
 * be made.  The first call on a device looks up the array's device address; make that
 * call outside graph capture.
 *
 * Arguments:
 * - device: the HIP device, made current for the call and restored after it.
 * - stream: a hipStream_t of that device (passed as void*; NULL for the default stream).
 * - policy: NULL or "auto" for the shape-driven choice, which is gemm_run's on a handle
 *   of that device.  Or a policy name as gemm_set_policy takes it.
 * - The remaining arguments, the dtypes and the special cases are gemm_run's.
 *
 * Errors: as gemm_run, plus these.
 * - INVALID_VALUE: a bad device index (or one of 64 or more), or an unknown policy name.
 * - NOT_SUPPORTED: a forced split or stream-K grid whose partials would exceed
 *   GEMM_STATIC_SCRATCH_BYTES.  The shape-driven choice never needs more. */
#define GEMM_STATIC_SCRATCH_BYTES ((size_t)64 << 20)
gemm_status_t gemm_run_noalloc(int device, void* stream, const char* policy, int transA, int transB,
                               int64_t M, int64_t N, int64_t K, float alpha, const void* A,
                               int64_t lda, const void* B, int64_t ldb, float beta, void* C,
                               int64_t ldc, int dtype);

/* Block-scaled E4M3 ("MXFP8") GEMM: the MXFP8 operands of the fused profile protocol
 * (section "SM103 MXFP8 QKV weight-quantization diagnostics": E4M3 elements with one
 * UE8M0 scale per 32 elements along K).  Computes
 *
 *   C <- alpha * sum_k (A[m][k] * 2^(sa[m][k/32]-127)) * (B[n][k] * 2^(sb[n][k/32]-127)) + beta*C
 *
 * Layout (both operands K-contiguous, the layout whose 32-element blocks are
 * contiguous): A is E4M3 [M][lda >= K]; B is E4M3 [N][ldb >= K] (op(B) = B^T);
 * scale_a is one byte per row and block, [M][ld_scale_a >= ceil(K/32)]; scale_b
 * [N][ld_scale_b >= ceil(K/32)]; C as in gemm_run.  A scale byte e stands for 2^(e-127)
 * (255 is NaN).  dtype is GEMM_MXE4M3_BF16, GEMM_MXE4M3_F32 or GEMM_MXE4M3_E4M3 (C's
 * type).  By default every scaled element is widened exactly to bf16 and accumulated in
 * fp32 (scaled values below the bf16 range lose precision).  The policy
 * "mxe4m3native_dma_m256n256k128_w2x4_mt32_s2" (gemm_set_policy) runs the scaled f8f6f4
 * MFMA instead, which sums each group of products at reduced precision (bits below
 * 2^-13 of the group's largest product are dropped); it needs 4-byte aligned scale
 * arrays with ld_scale_a and ld_scale_b multiples of 4 (else NOT_SUPPORTED) and never
 * uses the scale bytes of blocks past K.  Device pointers; errors and special cases as
 * gemm_run; NOT_SUPPORTED when a scale array spans 2^31 bytes or more. */
gemm_status_t gemm_run_mx(gemm_handle_t h, int64_t M, int64_t N, int64_t K, float alpha,
                          const void* A, int64_t lda, const uint8_t* scale_a, int64_t ld_scale_a,
                          const void* B, int64_t ldb, const uint8_t* scale_b, int64_t ld_scale_b,
                          float beta, void* C, int64_t ldc, int dtype);

/* Quantises a bf16 matrix to block-scaled E4M3 along its rows (the quantisation step
 * before the MXFP8 GEMMs in the same section of the profile protocol: amax of each
 * 32-element group, a UE8M0 scale, E4M3 conversion).  src is bf16 [rows][ld_src >=
 * cols]; dst receives E4M3 [rows][ld_dst >= cols] and scales one byte per row and
 * 32-element group [rows][ld_scales >= ceil(cols/32)] (the last group of a row may be
 * shorter).  Rule (OCP microscaling): e = clamp(floor(log2(amax)) - 8 + 127, 0, 254),
 * 0 for an all-zero group; element = x / 2^(e-127) rounded to the nearest E4M3 value,
 * ties to the even code, saturating at +-448; NaN stays NaN and does not set the scale.
 * Rows of more than 65535 * 2048 elements: NOT_SUPPORTED.  Device pointers, enqueued on
 * the handle's stream; writes nothing on an error. */
gemm_status_t gemm_quantize_mx(gemm_handle_t h, int64_t rows, int64_t cols, const void* src,
                               int64_t ld_src, void* dst, int64_t ld_dst, uint8_t* scales,
                               int64_t ld_scales);

/* Validates gemm_run's arguments on the host only (no handle, no device). */
gemm_status_t gemm_check_args(int transA, int transB, int64_t M, int64_t N, int64_t K,
                              float alpha, const void* A, int64_t lda, const void* B,
                              int64_t ldb, float beta, const void* C, int64_t ldc, int dtype);

/* Writes the name of the policy gemm_run (gemm_run_mx for the block-scaled dtypes,
 * with transA = 0, transB = 1) would use for these arguments into
 * name[len] (NUL-terminated, truncated to fit), with "+sk<S>" appended when the call
 * is split S ways along K, "+streamk" (or "+streamk<G>") when a forced stream-K policy
 * runs stream-K on these arguments.  The pointers are only inspected for alignment.  h may be
 * NULL: then a 256-CU device with a workspace and no forced policy are assumed.
 * Pure host code. */
gemm_status_t gemm_query_policy(gemm_handle_t h, int transA, int transB, int64_t M, int64_t N,
                                int64_t K, const void* A, int64_t lda, const void* B,
                                int64_t ldb, const void* C, int64_t ldc, int dtype, char* name,
                                size_t len);

/* Forces the named policy for later gemm_run calls on this handle (for ablations and
 * invariance checks); NULL or "auto" restores the shape-driven choice.  The name is a
 * table entry, optionally followed by "+sk<S>" (S = 2, 4, 8 or 16; direct-to-LDS
 * policies only) to force split-K, or by "+streamk" (ping-pong policies only) to force
 * stream-K with one stream-K workgroup per CU, "+streamk<G>" with G of them (1..4096,
 * at most the CU count is used); a forced stream-K on a grid of whole rounds runs plain.  A forced policy that cannot serve a call (dtype,
 * alignment, a split that leaves a split fewer than two K tiles or does not fit the
 * workspace) returns NOT_SUPPORTED from gemm_run.  Unknown names return
 * INVALID_VALUE. */
gemm_status_t gemm_set_policy(gemm_handle_t h, const char* name);

/* Diagnostic LDS read microbenchmark (the LDS -> register rung of the ablation plan,
 * "cp.async / ldmatrix ablation -- initial plan", section 2.3: a load-only loop without
 * MFMA).  Enqueues on the handle's stream `workgroups` workgroups of 256 threads; each
 * fills a 64 KiB LDS array, then every lane repeats `iters` times: 8 reads of one kind
 * at LDS byte offsets offsets[j*64 + (lane % 64)], j = 0..7 (a host array of 512
 * values, copied at the call), then a wait for them.  kind: 0 ds_read_b128 (16 bytes),
 * 1 ds_read_b64_tr_b16 (8), 2 ds_read_u16 (2), 3 ds_read_b64 (8), 4 ds_read_b64_tr_b8 (8),
 * 5 ds_read2st64_b64 (8 bytes at the offset and 8 at the offset + 2048: two fragments 16
 * rows of 128 bytes apart in one instruction).  Each offset must be a multiple of the width
 * and leave the read inside the 64 KiB (at most 65536 - width, 65536 - 2056 for kind 5),
 * else INVALID_VALUE (nothing is launched).  Time it with events around the call; it writes
 * no memory. */
gemm_status_t gemm_lds_probe(gemm_handle_t h, int kind, const uint32_t* offsets, int iters,
                             int workgroups);

/* Diagnostic hardware microbenchmarks: one stage of the GEMM pipeline timed alone ("cp.async /
 * ldmatrix ablation -- initial plan", section 2.3: isolate a stage with a microbenchmark), to
 * set a kernel's time against the cost of each stage.  Enqueues on the handle's stream
 * `workgroups` workgroups of 512 threads (8 waves); wave 0 of workgroup b writes to
 * cycles[b] (a device array of `workgroups` values, caller-owned) the s_memtime count
 * (shader clock cycles) from a workgroup barrier before the first iteration to one after
 * the last wave's last iteration.
 *   kind 0: each wave issues `iters` clusters of 32 v_mfma_f32_16x16x32_bf16 on register
 *           operands (4 independent accumulators).  param 0: all 8 waves at once; param 1:
 *           the two groups of 4 waves take turns, one cluster each between workgroup
 *           barriers (the ping-pong kernel's schedule).
 *   kind 1: the same with clusters of 16 v_mfma_f32_32x32x16_bf16.
 *   kind 2: direct-to-LDS copies (buffer_load_dwordx4 ... lds): workgroup b copies `iters`
 *           tiles of 256 rows x param bytes (param 64, 128 or 256) from the 256-row panel
 *           b % (src_bytes / (256*8192)) of src, a device buffer of rows of 8192 bytes
 *           (src_bytes a multiple of 2 MiB, at most 2 GiB, src 16-byte aligned), tile t from
 *           byte column (t * param) % 8192, into two LDS slots in turn, one tile in flight
 *           while the previous one lands.
 * Arguments outside these ranges: INVALID_VALUE, nothing launched.  Time the call with
 * events; cycles / time gives the clock under that load. */
gemm_status_t gemm_hw_probe(gemm_handle_t h, int kind, int param, int iters, int workgroups,
                            const void* src, int64_t src_bytes, unsigned long long* cycles);

/* The policy table: count and names (index 0 .. count-1).  Out-of-range -> NULL. */
int gemm_policy_count(void);
const char* gemm_policy_name(int index);

/* Library and policy-table version string, e.g. "dbgemm 0.1.0 policy-table 1". */
const char* gemm_version(void);

/* Human-readable name of a status code. */
const char* gemm_status_string(int status);

/* ---------------------------------------------------------------------------------
 * The single-GPU BLAS level-3 family on the GEMM core: the operator set of "BLASMp
 * development notes" (section 1: a BLAS3 library; section 2: SYRK built on the GEMM,
 * then TRSM, SYR2K, SYMM and TRMM), on one GPU, without the 2D block-cyclic
 * distribution.  The operations are the textbook BLAS ones, in the row-major
 * convention of gemm_run: element (i, j) is row i, column j, and the leading
 * dimension is the row stride.
 *
 *   uplo  GEMM_LOWER: the lower triangle (i >= j) is referenced (written, for SYRK and
 *         SYR2K); GEMM_UPPER: the upper triangle (i <= j).  The other triangle of a
 *         triangular or symmetric operand is never read (it may hold anything, NaN
 *         included); the other triangle of a SYRK / SYR2K result is never written.
 *   side  GEMM_SIDE_LEFT: the triangular / symmetric matrix multiplies from the left;
 *         GEMM_SIDE_RIGHT: from the right.
 *   diag  GEMM_DIAG_UNIT: the triangular matrix has ones on its diagonal, which is not
 *         read; GEMM_DIAG_NON_UNIT: the diagonal is read.
 *
 * Types: bf16 operands, fp32 accumulation; dtype GEMM_BF16_BF16 (bf16 C) or
 * GEMM_BF16_F32 (fp32 C) where a C is produced, GEMM_BF16_BF16 only for gemm_trsm.
 * Memory: device pointers owned by the caller; the calls use the handle's workspace
 * (SYMM and TRMM expand the triangle into it, TRSM keeps the inverted diagonal blocks
 * there), so, like split-K GEMMs, calls of one handle must not overlap on the device.
 * Nothing is allocated; the calls return once everything is enqueued on the handle's
 * stream.  Errors: arguments are checked before anything is launched (INVALID_VALUE
 * for a bad size, leading dimension, flag, pointer or dtype; NOT_SUPPORTED for
 * non-finite alpha / beta, M or N above 65535 * 64, or an operand larger than the
 * workspace handles, see each call); on an error nothing is written.  Fast path: the MFMA kernels need the GEMM
 * fast-path alignment of gemm.h; anything else runs on the generic kernel.
 * --------------------------------------------------------------------------------- */
typedef enum { GEMM_LOWER = 0, GEMM_UPPER = 1 } gemm_uplo_t;
typedef enum { GEMM_SIDE_LEFT = 0, GEMM_SIDE_RIGHT = 1 } gemm_side_t;
typedef enum { GEMM_DIAG_NON_UNIT = 0, GEMM_DIAG_UNIT = 1 } gemm_diag_t;

/* Symmetric rank-K update of one triangle:
 *   C <- alpha * op(A) op(A)^T + beta * C   on the uplo triangle of the N x N C,
 * op(A) N x K: A is [N][lda >= K] (trans = GEMM_OP_N) or [K][lda >= N] (GEMM_OP_T).
 * The GEMM kernels run over the tiles on one side of the diagonal only, and the
 * epilogue masks the diagonal tiles.  K == 0 or alpha == 0: C <- beta*C on the
 * triangle; beta == 0: C is not read. */
gemm_status_t gemm_syrk(gemm_handle_t h, int uplo, int trans, int64_t N, int64_t K, float alpha,
                        const void* A, int64_t lda, float beta, void* C, int64_t ldc, int dtype);

/* Symmetric rank-2K update of one triangle:
 *   C <- alpha * (op(A) op(B)^T + op(B) op(A)^T) + beta * C   on the uplo triangle,
 * op(A), op(B) N x K stored like syrk's A.  Both products accumulate in one fp32 sum
 * (one rounding of C), in one K loop: on the caller's buffers for trans = GEMM_OP_N with
 * lda == ldb, else (from N*K = 2^16, when they fit) on copies of op(A), op(B) made
 * K-contiguous in the workspace; smaller calls run on the generic kernel. */
gemm_status_t gemm_syr2k(gemm_handle_t h, int uplo, int trans, int64_t N, int64_t K, float alpha,
                         const void* A, int64_t lda, const void* B, int64_t ldb, float beta, void* C,
                         int64_t ldc, int dtype);

/* Symmetric matrix product: C <- alpha * S B + beta * C (side LEFT, S M x M) or
 * alpha * B S + beta * C (side RIGHT, S N x N); B and C are M x N ([M][ldb], [M][ldc]).
 * S is given by the uplo triangle of A ([n][lda >= n], n = M or N).  S is expanded
 * into the workspace in row panels, so NOT_SUPPORTED when 256 rows of it exceed the
 * workspace (n > 131072). */
gemm_status_t gemm_symm(gemm_handle_t h, int side, int uplo, int64_t M, int64_t N, float alpha,
                        const void* A, int64_t lda, const void* B, int64_t ldb, float beta, void* C,
                        int64_t ldc, int dtype);

/* Triangular matrix product, out of place: C <- alpha * op(T) B (side LEFT, T M x M) or
 * alpha * B op(T) (side RIGHT, T N x N); T is the uplo triangle of A ([n][lda >= n])
 * with the diagonal per diag; B and C are M x N and must not overlap.  T is expanded
 * with zeros into the workspace in panels and each output tile skips the K tiles that
 * meet only zeros of op(T).  NOT_SUPPORTED when n > 131072. */
gemm_status_t gemm_trmm(gemm_handle_t h, int side, int uplo, int transA, int diag, int64_t M,
                        int64_t N, float alpha, const void* A, int64_t lda, const void* B,
                        int64_t ldb, void* C, int64_t ldc, int dtype);

/* Triangular solve, in place: B <- X with op(T) X = alpha * B (side LEFT, T M x M) or
 * X op(T) = alpha * B (side RIGHT, T N x N); T as in gemm_trmm, B is bf16 M x N
 * ([M][ldb]); dtype must be GEMM_BF16_BF16.  The method is the blocked recursive one:
 * the 256 x 256 diagonal blocks of T are inverted in fp32 (from the inverses of their
 * 128 x 128 halves; stored as bf16 in the workspace), each 256-row (or column) block of X
 * is a product with its inverted block,
 * and the rest of B is updated with GEMMs (alpha*B - T_21 X_1), each rounded to bf16.
 * T must be non-singular (a zero on a non-unit diagonal gives Inf / NaN).  The result
 * is checked, as the pages' own TRSM checks were, by residual and forward / backward
 * error rather than element by element against an exact solution.  NOT_SUPPORTED when
 * the inverted blocks plus one block row (column) of B exceed the workspace.
 * alpha == 0: B <- 0. */
gemm_status_t gemm_trsm(gemm_handle_t h, int side, int uplo, int transA, int diag, int64_t M,
                        int64_t N, float alpha, const void* A, int64_t lda, void* B, int64_t ldb,
                        int dtype);

#ifdef __cplusplus
}
#endif

#endif /* DENSE_BLAS3_GEMM_AMD_GEMM_H */
