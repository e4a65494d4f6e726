"""GPU parity of the BLAS3 family (gemm_syrk, gemm_syr2k, gemm_symm, gemm_trmm, gemm_trsm)
against the float64 oracle (oracle/blas3.py), through the C-ABI.

Ragged sizes run on the generic kernel, sizes in whole 16-byte chunks on the MFMA kernels;
both are compared element by element.  Unreferenced triangles of the operands hold NaN
(a read of them shows), and the triangle of C that SYRK / SYR2K must not write starts as
NaN or as known values that must come back bit for bit.
"""
import numpy as np
import pytest

import gemm_inputs as gi
import oracle
import tolerance
from gpu_util import to_device, to_host
from oracle import blas3

pytestmark = pytest.mark.gpu

LOWER, UPPER, LEFT, RIGHT = 0, 1, 0, 1
C_FMT = {"bf16": oracle.C_BF16, "f32": oracle.C_F32}


def sync():
    import torch
    torch.cuda.synchronize()


def c_bits(shape, c_dtype, seed, std=1.0):
    return gi.draw("normal", shape, seed, gi.BF16 if c_dtype == "bf16" else gi.F32, std)


def tri_mask(N, uplo):
    i, j = np.arange(N)[:, None], np.arange(N)[None, :]
    return (i >= j) if uplo == LOWER else (i <= j)


def check_c(got_bits, c_dtype, R, S, K, mask=None):
    got = got_bits if mask is None else got_bits[mask]
    Rm = R if mask is None else R[mask]
    Sm = S if mask is None else S[mask]
    res = tolerance.check(got.reshape(1, -1), c_dtype, Rm.reshape(1, -1), Sm.reshape(1, -1), K)
    assert res["ok"], res


# ------------------------------------------------------------------------------ SYRK

SYRK_SHAPES = [(264, 200), (512, 136), (301, 203), (1024, 512)]


@pytest.mark.parametrize("N,K", SYRK_SHAPES)
@pytest.mark.parametrize("uplo", [LOWER, UPPER])
@pytest.mark.parametrize("trans", [0, 1])
@pytest.mark.parametrize("c_dtype", ["bf16", "f32"])
def test_syrk(gpu, N, K, uplo, trans, c_dtype):
    A = gi.bf16_uniform((K, N) if trans else (N, K), 0)
    C0 = c_bits((N, N), c_dtype, 2)
    C = to_device(C0, c_dtype)
    gpu.syrk(to_device(A, "bf16"), C, uplo=uplo, trans=trans, alpha=-1.5, beta=0.5)
    sync()
    got = to_host(C)
    R, S = blas3.syrk(uplo, trans, N, K, -1.5, A, 0.5, C0, C_FMT[c_dtype])
    m = tri_mask(N, uplo)
    check_c(got, c_dtype, R, S, K, m)
    assert np.array_equal(got[~m], C0[~m]), "the other triangle was written"


@pytest.mark.parametrize("N,K", [(256, 64), (520, 72), (77, 33)])
@pytest.mark.parametrize("uplo", [LOWER, UPPER])
def test_syrk_beta0_nan_c_and_exact(gpu, N, K, uplo):
    """Integer inputs: every product and sum is exact in fp32, so the triangle must equal the
    rounded exact result bit for bit; beta = 0 never reads the NaN-filled C, and the other
    triangle keeps its NaN."""
    import torch
    A = gi.ints((N, K), 5, -4, 4, gi.BF16)
    C = torch.full((N, N), float("nan"), dtype=torch.bfloat16, device="cuda:0")
    gpu.syrk(to_device(A, "bf16"), C, uplo=uplo, trans=0, alpha=1.0, beta=0.0)
    sync()
    got = to_host(C)
    R, _ = blas3.syrk(uplo, 0, N, K, 1.0, A, 0.0, None, oracle.C_BF16)
    m = tri_mask(N, uplo)
    assert np.array_equal(got[m], oracle.round_bf16(R[m]))
    assert np.isnan(tolerance.bf16_bits_to_f64(got[~m])).all()


def test_syrk_k0_scales_triangle_only(gpu):
    N = 64
    C0 = c_bits((N, N), "f32", 3)
    C = to_device(C0, "f32")
    A = to_device(gi.bf16_uniform((N, 8), 1), "bf16")
    assert gpu.syrk_raw(LOWER, 0, N, 0, 1.0, A.data_ptr(), 8, 2.0, C.data_ptr(), N, 0) == 0
    sync()
    got = tolerance.f32_bits_to_f64(to_host(C))
    old = tolerance.f32_bits_to_f64(C0)
    m = tri_mask(N, LOWER)
    assert np.array_equal(got[m], 2.0 * old[m]) and np.array_equal(got[~m], old[~m])


def test_syrk_4096_sampled_rows(gpu):
    """The measured SYRK workload (N = K = 4096, lower, bf16 C): rows sampled over every tile
    row against the GEMM oracle restricted to them, the rest of the triangle checked for
    finiteness and the upper triangle for being untouched."""
    import torch
    N = K = 4096
    A = gi.bf16_uniform((N, K), 0)
    C = torch.full((N, N), float("nan"), dtype=torch.bfloat16, device="cuda:0")
    gpu.syrk(to_device(A, "bf16"), C, uplo=LOWER, trans=0)
    sync()
    got = to_host(C)
    rows = sorted(set([0, 1, 255, 256, 2047, 2048, 4095] + list(range(37, N, 331))))
    R, S = oracle.gemm(0, 1, N, N, K, 1.0, A, K, A, K, 0.0, None, N, oracle.IN_BF16, oracle.C_BF16, rows=rows)
    for t, r in enumerate(rows):
        res = tolerance.check(got[r, : r + 1].reshape(1, -1), "bf16", R[t, : r + 1].reshape(1, -1),
                              S[t, : r + 1].reshape(1, -1), K)
        assert res["ok"], (r, res)
    v = tolerance.bf16_bits_to_f64(got)
    m = tri_mask(N, LOWER)
    assert np.isfinite(v[m]).all() and np.isnan(v[~m]).all()


# ------------------------------------------------------------------------------ SYR2K

@pytest.mark.parametrize("N,K", [(264, 200), (301, 203), (512, 264)])
@pytest.mark.parametrize("uplo", [LOWER, UPPER])
@pytest.mark.parametrize("trans", [0, 1])
@pytest.mark.parametrize("c_dtype", ["bf16", "f32"])
def test_syr2k(gpu, N, K, uplo, trans, c_dtype):
    shape = (K, N) if trans else (N, K)
    A, B = gi.bf16_uniform(shape, 0), gi.bf16_uniform(shape, 1)
    C0 = c_bits((N, N), c_dtype, 2)
    C = to_device(C0, c_dtype)
    gpu.syr2k(to_device(A, "bf16"), to_device(B, "bf16"), C, uplo=uplo, trans=trans, alpha=0.75, beta=-1.0)
    sync()
    got = to_host(C)
    R, S = blas3.syr2k(uplo, trans, N, K, 0.75, A, B, -1.0, C0, C_FMT[c_dtype])
    m = tri_mask(N, uplo)
    check_c(got, c_dtype, R, S, 2 * K, m)
    assert np.array_equal(got[~m], C0[~m])


def test_syr2k_different_leading_dimensions(gpu):
    """lda != ldb: the generic kernel (two K passes with their own strides)."""
    import torch
    N, K = 136, 72
    A = gi.bf16_uniform((N, K), 3)
    Bw = gi.bf16_uniform((N, K + 24), 4)
    C = torch.zeros((N, N), dtype=torch.float32, device="cuda:0")
    Bd = to_device(Bw, "bf16")[:, :K]
    gpu.syr2k(to_device(A, "bf16"), Bd, C, uplo=UPPER, trans=0, alpha=1.0, beta=0.0)
    sync()
    R, S = blas3.syr2k(UPPER, 0, N, K, 1.0, A, np.ascontiguousarray(Bw[:, :K]), 0.0, None, oracle.C_F32)
    m = tri_mask(N, UPPER)
    check_c(to_host(C), "f32", R, S, 2 * K, m)


@pytest.mark.parametrize("K,extra_a,extra_b", [(203, 0, 0), (264, 8, 24), (203, 5, 13)])
def test_syr2k_padded_copies(gpu, K, extra_a, extra_b):
    """N * K >= 2^16 with K not a multiple of 8 or lda != ldb: the operands are copied into the
    workspace with zero-padded K-contiguous rows of one common stride, then the dual-product
    kernel runs.  The unused columns of the caller's wider buffers hold NaN, so reading past K
    in them would show."""
    import torch
    N = 512
    A = gi.bf16_uniform((N, K), 21)
    B = gi.bf16_uniform((N, K), 22)
    nan = np.uint16(0x7FC0)
    Aw = np.full((N, K + extra_a), nan, dtype=np.uint16)
    Bw = np.full((N, K + extra_b), nan, dtype=np.uint16)
    Aw[:, :K], Bw[:, :K] = A, B
    C0 = c_bits((N, N), "f32", 23)
    C = to_device(C0, "f32")
    Ad = to_device(Aw, "bf16")[:, :K]
    Bd = to_device(Bw, "bf16")[:, :K]
    gpu.syr2k(Ad, Bd, C, uplo=LOWER, trans=0, alpha=0.5, beta=1.0)
    sync()
    got = to_host(C)
    R, S = blas3.syr2k(LOWER, 0, N, K, 0.5, A, B, 1.0, C0, oracle.C_F32)
    m = tri_mask(N, LOWER)
    check_c(got, "f32", R, S, 2 * K, m)
    assert np.array_equal(got[~m], C0[~m])


def test_syr2k_exact_integers(gpu):
    import torch
    N, K = 384, 128
    A, B = gi.ints((N, K), 6, -4, 4, gi.BF16), gi.ints((N, K), 7, -4, 4, gi.BF16)
    C = torch.full((N, N), float("nan"), dtype=torch.float32, device="cuda:0")
    gpu.syr2k(to_device(A, "bf16"), to_device(B, "bf16"), C, uplo=LOWER, trans=0, alpha=1.0, beta=0.0)
    sync()
    R, _ = blas3.syr2k(LOWER, 0, N, K, 1.0, A, B, 0.0, None, oracle.C_F32)
    m = tri_mask(N, LOWER)
    assert np.array_equal(tolerance.f32_bits_to_f64(to_host(C))[m], R[m])


# ------------------------------------------------------------------------------ SYMM

@pytest.mark.parametrize("M,N", [(264, 136), (301, 203), (512, 384)])
@pytest.mark.parametrize("side", [LEFT, RIGHT])
@pytest.mark.parametrize("uplo", [LOWER, UPPER])
@pytest.mark.parametrize("c_dtype", ["bf16", "f32"])
def test_symm(gpu, M, N, side, uplo, c_dtype):
    n = M if side == LEFT else N
    A = gi.bf16_symmetric_stored(n, uplo, 0)
    B = gi.bf16_uniform((M, N), 1)
    C0 = c_bits((M, N), c_dtype, 2)
    C = to_device(C0, c_dtype)
    gpu.symm(to_device(A, "bf16"), to_device(B, "bf16"), C, side=side, uplo=uplo, alpha=1.25, beta=-0.5)
    sync()
    R, S = blas3.symm(side, uplo, M, N, 1.25, A, B, -0.5, C0, C_FMT[c_dtype])
    check_c(to_host(C), c_dtype, R, S, n)


# ------------------------------------------------------------------------------ TRMM

@pytest.mark.parametrize("M,N", [(264, 200), (301, 203)])
@pytest.mark.parametrize("side", [LEFT, RIGHT])
@pytest.mark.parametrize("uplo", [LOWER, UPPER])
@pytest.mark.parametrize("transA", [0, 1])
@pytest.mark.parametrize("unit", [0, 1])
def test_trmm(gpu, M, N, side, uplo, transA, unit):
    import torch
    n = M if side == LEFT else N
    A = gi.bf16_triangular(n, uplo, 0, unit=bool(unit))
    B = gi.bf16_uniform((M, N), 1)
    C = torch.full((M, N), float("nan"), dtype=torch.bfloat16, device="cuda:0")
    gpu.trmm(to_device(A, "bf16"), to_device(B, "bf16"), C, side=side, uplo=uplo, transA=transA, diag=unit,
             alpha=-2.0)
    sync()
    R, S = blas3.trmm(side, uplo, transA, unit, M, N, -2.0, A, B)
    check_c(to_host(C), "bf16", R, S, n)


@pytest.mark.parametrize("side", [LEFT, RIGHT])
@pytest.mark.parametrize("uplo", [LOWER, UPPER])
@pytest.mark.parametrize("transA", [0, 1])
def test_trmm_larger_fp32(gpu, side, uplo, transA):
    import torch
    M, N = 1024, 768
    n = M if side == LEFT else N
    A = gi.bf16_triangular(n, uplo, 2)
    B = gi.bf16_uniform((M, N), 3)
    C = torch.full((M, N), float("nan"), dtype=torch.float32, device="cuda:0")
    gpu.trmm(to_device(A, "bf16"), to_device(B, "bf16"), C, side=side, uplo=uplo, transA=transA)
    sync()
    R, S = blas3.trmm(side, uplo, transA, 0, M, N, 1.0, A, B)
    check_c(to_host(C), "f32", R, S, n)


# ------------------------------------------------------------------------------ TRSM

def _int_system(n, M, N, side, uplo, transA, unit, seed):
    A = gi.int_triangular(n, uplo, seed, unit=bool(unit))
    Xt = gi.ints((M, N), seed + 1, -2, 2, gi.BF16)
    # B = op(T) X (or X op(T)) from the oracle's product: exact integers here
    Bv, _ = blas3.trmm(side, uplo, transA, unit, M, N, 1.0, A, Xt)
    assert np.abs(Bv).max() < 256
    return A, Xt, gi.f32_to_bf16_bits(Bv.astype(np.float32))


def _report(res):
    """Prints the achieved backward error beside the floor of one bf16 rounding of the exact
    solution, so a run with -s shows how far the solve is from its bound."""
    import os
    print("trsm %s eta=%.3e eta_round=%.3e ratio=%.2f bound=%.3e forward=%.3e kappa=%.1f" % (
        os.environ.get("PYTEST_CURRENT_TEST", "").split(" ")[0], res["eta"], res["eta_round"],
        res["eta"] / max(res["eta_round"], 1e-300), res["eta_bound"], res["forward"], res["kappa"]))


@pytest.mark.parametrize("M,N", [(512, 264), (300, 136), (136, 300)])
@pytest.mark.parametrize("side", [LEFT, RIGHT])
@pytest.mark.parametrize("uplo", [LOWER, UPPER])
@pytest.mark.parametrize("transA", [0, 1])
@pytest.mark.parametrize("unit", [1, 0])
def test_trsm_exact_integer_system(gpu, M, N, side, uplo, transA, unit):
    """op(T) X = B with T integer, its strictly triangular part squaring to zero, and X
    integer: every block inverse, leaf product and update is exact in bf16 and fp32, so the
    solution must come back bit for bit (this pins indexing, sides, transposes, the
    recursion's splits and the partial last block)."""
    n = M if side == LEFT else N
    A, Xt, Bb = _int_system(n, M, N, side, uplo, transA, unit, 10)
    Bd = to_device(Bb, "bf16")
    gpu.trsm(to_device(A, "bf16"), Bd, side=side, uplo=uplo, transA=transA, diag=unit, alpha=1.0)
    sync()
    assert np.array_equal(to_host(Bd), Xt)


@pytest.mark.parametrize("M,N", [(512, 264), (301, 203), (264, 520)])
@pytest.mark.parametrize("side", [LEFT, RIGHT])
@pytest.mark.parametrize("uplo", [LOWER, UPPER])
@pytest.mark.parametrize("transA", [0, 1])
@pytest.mark.parametrize("unit", [0, 1])
def test_trsm_real(gpu, M, N, side, uplo, transA, unit):
    n = M if side == LEFT else N
    A = gi.bf16_triangular(n, uplo, 20, unit=bool(unit))
    B = gi.bf16_uniform((M, N), 21)
    Bd = to_device(B, "bf16")
    alpha = 0.5
    gpu.trsm(to_device(A, "bf16"), Bd, side=side, uplo=uplo, transA=transA, diag=unit, alpha=alpha)
    sync()
    X = tolerance.bf16_bits_to_f64(to_host(Bd))
    X_ref = blas3.trsm(side, uplo, transA, unit, M, N, alpha, A, B)
    T = blas3.triangular(A, n, uplo, unit)
    opT = T.T if transA else T
    res = tolerance.trsm_check(X, X_ref, opT, alpha * tolerance.bf16_bits_to_f64(B), side, n)
    _report(res)
    assert res["ok"], res


def test_trsm_alpha0_zeroes_b(gpu):
    import torch
    B = torch.full((64, 48), float("nan"), dtype=torch.bfloat16, device="cuda:0")
    A = to_device(gi.bf16_triangular(64, LOWER, 1), "bf16")
    gpu.trsm(A, B, alpha=0.0)
    sync()
    assert (B.float() == 0).all().item()


def test_trsm_4096_sampled_columns(gpu):
    """The measured TRSM workload (M = N = 4096, left, lower, no transpose, non-unit): the
    columns of X are independent systems, so sampled columns are checked against the oracle
    solved for those columns only."""
    M = N = 4096
    A = gi.bf16_triangular(M, LOWER, 30)
    B = gi.bf16_uniform((M, N), 31)
    Bd = to_device(B, "bf16")
    gpu.trsm(to_device(A, "bf16"), Bd, side=LEFT, uplo=LOWER)
    sync()
    X = tolerance.bf16_bits_to_f64(to_host(Bd))
    cols = [0, 1, 127, 128, 2047, 4095] + list(range(300, N, 517))
    Bs = np.ascontiguousarray(B[:, cols])
    X_ref = blas3.trsm(LEFT, LOWER, 0, 0, M, len(cols), 1.0, A, Bs)
    T = blas3.triangular(A, M, LOWER, 0)
    res = tolerance.trsm_check(X[:, cols], X_ref, T, tolerance.bf16_bits_to_f64(Bs), LEFT, M)
    _report(res)
    assert res["ok"], res
    assert np.isfinite(X).all()


@pytest.mark.parametrize("M,N,K", [(4096, 4096, 256), (600, 328, 200), (192, 192, 64)])
def test_gemm_192_tile_nt(gpu, M, N, K):
    """The 192 x 192 tile (chosen for the symmetric updates) as a plain GEMM by name: A [M][K],
    B [N][K], ragged edges, every element against the oracle; other layouts are refused."""
    import dataclasses
    from gpu_util import compare, run_gpu
    p = gi.Gemm("nt192", M, N, K, transA=0, transB=1, c_dtype="f32", alpha=0.5, beta=0.0)
    data = p.make()
    C = run_gpu(gpu, p, data, policy="bf16_dma_m192n192k64_w2x4_mt16_s2_nt")
    res = compare(p, data, C)
    assert res["ok"], res
    q = dataclasses.replace(p, transB=0)
    dq = q.make()
    A, B = to_device(dq["A"], "bf16"), to_device(dq["B"], "bf16")
    import torch
    Cq = torch.zeros((M, N), dtype=torch.float32, device="cuda:0")
    gpu.set_policy("bf16_dma_m192n192k64_w2x4_mt16_s2_nt")
    try:
        st = gpu.run_raw(0, 0, M, N, K, 1.0, A.data_ptr(), K, B.data_ptr(), N, 0.0, Cq.data_ptr(), N, 0)
    finally:
        gpu.set_policy(None)
    assert st == 2  # NOT_SUPPORTED


@pytest.mark.parametrize("side", [LEFT, RIGHT])
@pytest.mark.parametrize("uplo", [LOWER, UPPER])
@pytest.mark.parametrize("transA", [0, 1])
def test_trsm_exact_integer_out_of_place(gpu, side, uplo, transA):
    """From 2^20 elements of B the solve keeps X in the workspace and copies it back at the
    end (the leaves then run on any tile shape): the exact integer system at 1024 x 1024
    pins that form bit for bit, as the smaller cases pin the in-place one."""
    M = N = 1024
    n = M if side == LEFT else N
    A, Xt, Bb = _int_system(n, M, N, side, uplo, transA, 0, 40)
    Bd = to_device(Bb, "bf16")
    gpu.trsm(to_device(A, "bf16"), Bd, side=side, uplo=uplo, transA=transA, diag=0, alpha=1.0)
    sync()
    assert np.array_equal(to_host(Bd), Xt)


def _padded_t(A, n):
    """T on the device with its rows padded to a multiple of 8 elements (16-byte aligned rows,
    which the doubled leaves need), NaN in the padding."""
    ld = (n + 7) // 8 * 8 + 8
    full = np.full((n, ld), gi.BF16_NAN, dtype=np.uint16)
    full[:, :n] = A
    return to_device(full, "bf16")[:, :n]


@pytest.mark.parametrize("n,m", [(1500, 700), (2300, 456), (2047, 520), (2048, 512)])
@pytest.mark.parametrize("side", [LEFT, RIGHT])
@pytest.mark.parametrize("uplo", [LOWER, UPPER])
@pytest.mark.parametrize("transA", [0, 1])
def test_trsm_exact_integer_doubled_leaves(gpu, n, m, side, uplo, transA):
    """From 2^20 elements of B, with T's rows 16-byte aligned, the leaves are whole 512- or
    1024-blocks of T whose inverses are doubled up from the 128-block ones by batched
    products: n = 1500 (two 512-blocks and a 476-row tail of 256-leaves), 2300 (two
    1024-blocks and a 252 tail), 2047 (three 512-blocks and a 511 tail), 2048 (two
    1024-blocks), bit for bit on exact integer systems."""
    M, N = (n, m) if side == LEFT else (m, n)
    A, Xt, Bb = _int_system(n, M, N, side, uplo, transA, 1, 50)
    Bd = to_device(Bb, "bf16")
    gpu.trsm(_padded_t(A, n), Bd, side=side, uplo=uplo, transA=transA, diag=1, alpha=1.0)
    sync()
    assert np.array_equal(to_host(Bd), Xt)


@pytest.mark.parametrize("side", [LEFT, RIGHT])
def test_trsm_exact_integer_unaligned_t(gpu, side):
    """T with rows that are not 16-byte aligned (n = 1500, lda = n): 256-leaves only."""
    n, m = 1500, 700
    M, N = (n, m) if side == LEFT else (m, n)
    A, Xt, Bb = _int_system(n, M, N, side, LOWER, 0, 1, 51)
    Bd = to_device(Bb, "bf16")
    gpu.trsm(to_device(A, "bf16"), Bd, side=side, uplo=LOWER, transA=0, diag=1, alpha=1.0)
    sync()
    assert np.array_equal(to_host(Bd), Xt)


@pytest.mark.parametrize("n,m", [(1500, 700), (2300, 456)])
@pytest.mark.parametrize("side", [LEFT, RIGHT])
@pytest.mark.parametrize("uplo", [LOWER, UPPER])
def test_trsm_real_doubled_leaves(gpu, n, m, side, uplo):
    """The doubled 512- and 1024-block inverses on real-valued systems, residual and forward
    error within the bound."""
    M, N = (n, m) if side == LEFT else (m, n)
    A = gi.bf16_triangular(n, uplo, 60)
    B = gi.bf16_uniform((M, N), 61)
    Bd = to_device(B, "bf16")
    gpu.trsm(_padded_t(A, n), Bd, side=side, uplo=uplo, transA=0, diag=0, alpha=0.75)
    sync()
    X = tolerance.bf16_bits_to_f64(to_host(Bd))
    X_ref = blas3.trsm(side, uplo, 0, 0, M, N, 0.75, A, B)
    T = blas3.triangular(A, n, uplo, 0)
    res = tolerance.trsm_check(X, X_ref, T, 0.75 * tolerance.bf16_bits_to_f64(B), side, n)
    _report(res)
    assert res["ok"], res


# ------------------------------------------------------------------ panels and strides

@pytest.mark.parametrize("side", [LEFT, RIGHT])
def test_symm_two_panels(gpu, side):
    """n = 12288: the expanded symmetric matrix (12288 x 12288 bf16, 288 MiB) exceeds the 256 MiB
    workspace, so it is expanded and multiplied in two row panels (10752 + 1536 rows; the
    second panel's mirrored elements come from rows of the first)."""
    n, other = 12288, 40
    M, N = (n, other) if side == LEFT else (other, n)
    A = gi.bf16_symmetric_stored(n, UPPER, 5)
    B = gi.bf16_uniform((M, N), 6)
    C0 = c_bits((M, N), "f32", 7)
    C = to_device(C0, "f32")
    gpu.symm(to_device(A, "bf16"), to_device(B, "bf16"), C, side=side, uplo=UPPER, alpha=0.5, beta=2.0)
    sync()
    R, S = blas3.symm(side, UPPER, M, N, 0.5, A, B, 2.0, C0, oracle.C_F32)
    check_c(to_host(C), "f32", R, S, n)


@pytest.mark.parametrize("side", [LEFT, RIGHT])
@pytest.mark.parametrize("transA", [0, 1])
def test_trmm_two_panels(gpu, side, transA):
    """n = 6144 in two panels, each with its own K-band offset."""
    import torch
    n, other = 6144, 48
    M, N = (n, other) if side == LEFT else (other, n)
    A = gi.bf16_triangular(n, LOWER, 8)
    B = gi.bf16_uniform((M, N), 9)
    C = torch.full((M, N), float("nan"), dtype=torch.float32, device="cuda:0")
    gpu.trmm(to_device(A, "bf16"), to_device(B, "bf16"), C, side=side, uplo=LOWER, transA=transA, alpha=1.0)
    sync()
    R, S = blas3.trmm(side, LOWER, transA, 0, M, N, 1.0, A, B)
    check_c(to_host(C), "f32", R, S, n)


def _strided(bits, extra):
    """A device view of `bits` inside a wider buffer (leading dimension + extra), the padding
    NaN so that a read past the row shows."""
    import torch
    rows, cols = bits.shape
    wide = np.full((rows, cols + extra), 0x7FC0, dtype=np.uint16)
    wide[:, :cols] = bits
    return to_device(wide, "bf16")[:, :cols]


def test_blas3_strided_operands(gpu):
    """Every operand with a leading dimension larger than its row (views of wider buffers
    with NaN padding): SYRK, SYR2K (lda == ldb), SYMM, TRMM and TRSM against the oracle."""
    import torch
    N, K = 136, 72
    A = gi.bf16_uniform((N, K), 1)
    B = gi.bf16_uniform((N, K), 2)
    C = torch.zeros((N, N + 16), dtype=torch.float32, device="cuda:0")[:, :N]
    gpu.syrk(_strided(A, 8), C, uplo=LOWER, trans=0)
    sync()
    R, S = blas3.syrk(LOWER, 0, N, K, 1.0, A, 0.0, None, oracle.C_F32)
    m = tri_mask(N, LOWER)
    check_c(to_host(C), "f32", R, S, K, m)
    C.zero_()
    gpu.syr2k(_strided(A, 8), _strided(B, 8), C, uplo=UPPER, trans=0)
    sync()
    R, S = blas3.syr2k(UPPER, 0, N, K, 1.0, A, B, 0.0, None, oracle.C_F32)
    check_c(to_host(C), "f32", R, S, 2 * K, tri_mask(N, UPPER))
    M2, N2 = 136, 200
    Sm = gi.bf16_symmetric_stored(M2, LOWER, 3)
    B2 = gi.bf16_uniform((M2, N2), 4)
    C2 = torch.zeros((M2, N2 + 8), dtype=torch.float32, device="cuda:0")[:, :N2]
    gpu.symm(_strided(Sm, 16), _strided(B2, 8), C2, side=LEFT, uplo=LOWER)
    sync()
    R, S = blas3.symm(LEFT, LOWER, M2, N2, 1.0, Sm, B2, 0.0, None, oracle.C_F32)
    check_c(to_host(C2), "f32", R, S, M2)
    T = gi.bf16_triangular(M2, UPPER, 5)
    C2.zero_()
    gpu.trmm(_strided(T, 24), _strided(B2, 8), C2, side=LEFT, uplo=UPPER, transA=1)
    sync()
    R, S = blas3.trmm(LEFT, UPPER, 1, 0, M2, N2, 1.0, T, B2)
    check_c(to_host(C2), "f32", R, S, M2)
    Bd = _strided(B2, 8)
    gpu.trsm(_strided(T, 24), Bd, side=LEFT, uplo=UPPER, transA=1, alpha=1.0)
    sync()
    X = tolerance.bf16_bits_to_f64(to_host(Bd))
    X_ref = blas3.trsm(LEFT, UPPER, 1, 0, M2, N2, 1.0, T, B2)
    opT = blas3.triangular(T, M2, UPPER, 0).T
    res = tolerance.trsm_check(X, X_ref, opT, tolerance.bf16_bits_to_f64(B2), LEFT, M2)
    _report(res)
    assert res["ok"], res


@pytest.mark.parametrize("N,K", [(1536, 768), (1100, 1024)])
@pytest.mark.parametrize("uplo", [LOWER, UPPER])
@pytest.mark.parametrize("c_dtype", ["bf16", "f32"])
def test_syrk_transposed_copy(gpu, N, K, uplo, c_dtype):
    """A stored [K][N] with N*K >= 2^20: A is first copied transposed into the workspace and
    the triangle runs with both operands K-contiguous."""
    A = gi.bf16_uniform((K, N), 11)
    C0 = c_bits((N, N), c_dtype, 12)
    C = to_device(C0, c_dtype)
    gpu.syrk(to_device(A, "bf16"), C, uplo=uplo, trans=1, alpha=0.5, beta=1.0)
    sync()
    got = to_host(C)
    R, S = blas3.syrk(uplo, 1, N, K, 0.5, A, 1.0, C0, C_FMT[c_dtype])
    m = tri_mask(N, uplo)
    check_c(got, c_dtype, R, S, K, m)
    assert np.array_equal(got[~m], C0[~m])


@pytest.mark.parametrize("uplo", [LOWER, UPPER])
def test_syr2k_transposed_copy(gpu, uplo):
    N, K = 1024, 1024
    A, B = gi.bf16_uniform((K, N), 13), gi.bf16_uniform((K, N), 14)
    C0 = c_bits((N, N), "f32", 15)
    C = to_device(C0, "f32")
    gpu.syr2k(to_device(A, "bf16"), to_device(B, "bf16"), C, uplo=uplo, trans=1, alpha=1.0, beta=-1.0)
    sync()
    got = to_host(C)
    R, S = blas3.syr2k(uplo, 1, N, K, 1.0, A, B, -1.0, C0, oracle.C_F32)
    m = tri_mask(N, uplo)
    check_c(got, "f32", R, S, 2 * K, m)
    assert np.array_equal(got[~m], C0[~m])


# ------------------------------------------------------------------ degenerate sizes

@pytest.mark.parametrize("M,N", [(1, 1), (1, 7), (9, 1), (3, 2)])
def test_blas3_tiny(gpu, M, N):
    """One row, one column, 1 x 1: every operation of the family against the oracle."""
    import torch
    A = gi.bf16_uniform((M, M), 1)
    Bm = gi.bf16_uniform((M, N), 2)
    C = torch.zeros((M, M), dtype=torch.float32, device="cuda:0")
    gpu.syrk(to_device(gi.bf16_uniform((M, N), 3), "bf16"), C, uplo=LOWER, trans=0)
    sync()
    R, S = blas3.syrk(LOWER, 0, M, N, 1.0, gi.bf16_uniform((M, N), 3), 0.0, None, oracle.C_F32)
    check_c(to_host(C), "f32", R, S, N, tri_mask(M, LOWER))
    Sm = gi.bf16_symmetric_stored(M, UPPER, 4)
    C2 = torch.zeros((M, N), dtype=torch.float32, device="cuda:0")
    gpu.symm(to_device(Sm, "bf16"), to_device(Bm, "bf16"), C2, side=LEFT, uplo=UPPER)
    sync()
    R, S = blas3.symm(LEFT, UPPER, M, N, 1.0, Sm, Bm, 0.0, None, oracle.C_F32)
    check_c(to_host(C2), "f32", R, S, M)
    T = gi.bf16_triangular(M, LOWER, 5)
    gpu.trmm(to_device(T, "bf16"), to_device(Bm, "bf16"), C2, side=LEFT, uplo=LOWER, transA=1)
    sync()
    R, S = blas3.trmm(LEFT, LOWER, 1, 0, M, N, 1.0, T, Bm)
    check_c(to_host(C2), "f32", R, S, M)
    Bd = to_device(Bm, "bf16")
    gpu.trsm(to_device(T, "bf16"), Bd, side=LEFT, uplo=LOWER, transA=0, alpha=2.0)
    sync()
    X = tolerance.bf16_bits_to_f64(to_host(Bd))
    X_ref = blas3.trsm(LEFT, LOWER, 0, 0, M, N, 2.0, T, Bm)
    res = tolerance.trsm_check(X, X_ref, blas3.triangular(T, M, LOWER, 0), 2.0 * tolerance.bf16_bits_to_f64(Bm),
                               LEFT, M)
    _report(res)
    assert res["ok"], res


def test_blas3_empty_calls_write_nothing(gpu):
    """M, N or K = 0: success, nothing launched or written (C keeps its NaN); K = 0 SYRK
    scales the triangle only (covered above); invalid flags and dtypes are refused."""
    import torch
    C = torch.full((8, 8), float("nan"), dtype=torch.float32, device="cuda:0")
    p = C.data_ptr()
    assert gpu.syrk_raw(LOWER, 0, 0, 4, 1.0, p, 4, 0.0, p, 8, 0) == 0
    assert gpu.syr2k_raw(UPPER, 1, 0, 4, 1.0, p, 1, p, 1, 0.0, p, 8, 0) == 0
    assert gpu.symm_raw(LEFT, LOWER, 0, 8, 1.0, p, 1, p, 8, 0.0, p, 8, 0) == 0
    assert gpu.trmm_raw(RIGHT, UPPER, 0, 0, 8, 0, 1.0, p, 1, p, 1, p, 8, 0) == 0
    assert gpu.trsm_raw(LEFT, LOWER, 0, 0, 0, 8, 1.0, p, 1, p, 8) == 0
    sync()
    assert torch.isnan(C).all().item()
    # bad flags / dtypes: INVALID_VALUE, nothing written
    assert gpu.syrk_raw(2, 0, 8, 8, 1.0, p, 8, 0.0, p, 8, 0) == 1
    assert gpu.symm_raw(LEFT, LOWER, 8, 8, 1.0, p, 8, p, 8, 0.0, p, 8, 2) == 1   # E4M3 not in the family
    assert gpu.trsm_raw(LEFT, LOWER, 0, 0, 8, 8, 1.0, p, 8, p, 8, 0) == 1       # TRSM is bf16 in and out
    assert gpu.trmm_raw(LEFT, LOWER, 0, 3, 8, 8, 1.0, p, 8, p, 8, p, 8, 0) == 1  # diag flag
    assert gpu.trsm_raw(LEFT, LOWER, 0, 0, 8, 8, float("inf"), p, 8, p, 8) == 2  # non-finite alpha
    sync()
    assert torch.isnan(C).all().item()
