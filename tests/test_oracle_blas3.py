"""Pins of the BLAS3-family oracle (oracle/blas3.py) against things other than itself:
the C GEMM oracle (itself pinned in test_oracle.py), closed forms worked by hand, exact
rational brute force, invariants of the operations, scipy's triangular solver as a
library routine, and exact integer systems whose solution is known in advance."""
from fractions import Fraction

import numpy as np
import pytest
import scipy.linalg

import gemm_inputs as gi
import oracle
from oracle import blas3

LOWER, UPPER, LEFT, RIGHT = 0, 1, 0, 1
bf = gi.f32_to_bf16_bits


def dec(bits):
    return oracle.decode(np.ascontiguousarray(bits), "bf16")


def rand_bits(shape, seed):
    return gi.bf16_uniform(shape, seed)


def zero_other(bits, uplo, unit=False):
    """The same operand with zeros (and ones on a unit diagonal) in place of the NaNs."""
    n = bits.shape[0]
    out = bits.copy()
    i, j = np.arange(n)[:, None], np.arange(n)[None, :]
    other = (i < j) if uplo == LOWER else (i > j)
    out[other] = 0
    if unit:
        out[np.arange(n), np.arange(n)] = bf(np.ones(n, np.float32))
    return out


# ------------------------------------------------------------------------------ SYRK

def test_syrk_hand_worked():
    # A = [[1, 2], [3, 4]], A A^T = [[5, 11], [11, 25]]; lower, alpha 1, beta 1,
    # C_old = [[1, 7], [2, 3]] -> [[6, 7], [13, 28]]: (0, 1) is outside and stays 7.
    A = bf(np.array([[1, 2], [3, 4]], np.float32))
    C = bf(np.array([[1, 7], [2, 3]], np.float32))
    R, _ = blas3.syrk(LOWER, 0, 2, 2, 1.0, A, 1.0, C, oracle.C_BF16)
    assert R.tolist() == [[6, 7], [13, 28]]
    # upper, A^T A = [[10, 14], [14, 20]], alpha 2, beta 0 -> [[20, 28], [C_old 2, 40]]
    R, _ = blas3.syrk(UPPER, 1, 2, 2, 2.0, A, 0.0, C, oracle.C_BF16)
    assert R.tolist() == [[20, 28], [2, 40]]


@pytest.mark.parametrize("uplo", [LOWER, UPPER])
@pytest.mark.parametrize("trans", [0, 1])
def test_syrk_matches_gemm_oracle(uplo, trans):
    N, K = 37, 29
    A = rand_bits((K, N) if trans else (N, K), 3)
    C = gi.bf16_normal((N, N), 4)
    R, S = blas3.syrk(uplo, trans, N, K, -1.5, A, 0.5, C, oracle.C_BF16)
    G, GS = oracle.gemm(trans, 1 - trans, N, N, K, -1.5, A, A.shape[1], A, A.shape[1], 0.5, C, N,
                        oracle.IN_BF16, oracle.C_BF16)
    i, j = np.arange(N)[:, None], np.arange(N)[None, :]
    tri = (i >= j) if uplo == LOWER else (i <= j)
    np.testing.assert_allclose(R[tri], G[tri], rtol=1e-13, atol=1e-13)
    np.testing.assert_allclose(S[tri], GS[tri], rtol=1e-13, atol=1e-13)
    assert np.array_equal(R[~tri], dec(C)[~tri])  # the other triangle is C_old, bit for bit


def test_syrk_beta0_never_reads_c():
    N, K = 8, 5
    A = rand_bits((N, K), 1)
    C = np.full((N, N), 0x7FC0, np.uint16)
    R, _ = blas3.syrk(LOWER, 0, N, K, 1.0, A, 0.0, C, oracle.C_BF16)
    i, j = np.arange(N)[:, None], np.arange(N)[None, :]
    assert np.isfinite(R[i >= j]).all() and np.isnan(R[i < j]).all()


def test_syrk_exact_fractions():
    N, K = 4, 3
    A = gi.ints((N, K), 5, -4, 4, gi.BF16)
    C = gi.ints((N, N), 6, -4, 4, gi.BF16)
    a = [[Fraction(float(v)) for v in row] for row in dec(A)]
    c = [[Fraction(float(v)) for v in row] for row in dec(C)]
    al, be = Fraction(3, 2), Fraction(-1, 4)
    R, _ = blas3.syrk(UPPER, 0, N, K, 1.5, A, -0.25, C, oracle.C_BF16)
    for i in range(N):
        for j in range(N):
            want = al * sum(a[i][k] * a[j][k] for k in range(K)) + be * c[i][j] if i <= j else c[i][j]
            assert Fraction(R[i, j]) == want


# ------------------------------------------------------------------------------ SYR2K

@pytest.mark.parametrize("uplo", [LOWER, UPPER])
@pytest.mark.parametrize("trans", [0, 1])
def test_syr2k_matches_two_gemms(uplo, trans):
    N, K = 23, 31
    A = rand_bits((K, N) if trans else (N, K), 7)
    B = rand_bits((K, N) if trans else (N, K), 8)
    C = gi.bf16_normal((N, N), 9)
    R, S = blas3.syr2k(uplo, trans, N, K, 0.75, A, B, 2.0, C, oracle.C_BF16)
    ld = A.shape[1]
    G1, S1 = oracle.gemm(trans, 1 - trans, N, N, K, 0.75, A, ld, B, ld, 0.0, None, N, oracle.IN_BF16,
                         oracle.C_BF16)
    G2, S2 = oracle.gemm(trans, 1 - trans, N, N, K, 0.75, B, ld, A, ld, 2.0, C, N, oracle.IN_BF16,
                         oracle.C_BF16)
    i, j = np.arange(N)[:, None], np.arange(N)[None, :]
    tri = (i >= j) if uplo == LOWER else (i <= j)
    np.testing.assert_allclose(R[tri], (G1 + G2)[tri], rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(S[tri], (S1 + S2)[tri], rtol=1e-12, atol=1e-12)
    assert np.array_equal(R[~tri], dec(C)[~tri])


def test_syr2k_of_a_with_itself_is_twice_syrk():
    N, K = 19, 11
    A = rand_bits((N, K), 10)
    C = gi.bf16_normal((N, N), 11)
    R2, _ = blas3.syr2k(LOWER, 0, N, K, 1.0, A, A, 1.0, C, oracle.C_BF16)
    R1, _ = blas3.syrk(LOWER, 0, N, K, 2.0, A, 1.0, C, oracle.C_BF16)
    np.testing.assert_allclose(R2, R1, rtol=1e-13, atol=1e-13)


def test_syr2k_symmetric_in_a_and_b():
    N, K = 13, 9
    A, B = rand_bits((K, N), 12), rand_bits((K, N), 13)
    Ra, _ = blas3.syr2k(UPPER, 1, N, K, 1.0, A, B, 0.0, None, oracle.C_F32)
    Rb, _ = blas3.syr2k(UPPER, 1, N, K, 1.0, B, A, 0.0, None, oracle.C_F32)
    np.testing.assert_allclose(Ra, Rb, rtol=1e-14, atol=1e-14)


# ------------------------------------------------------------------------------ SYMM

def test_symm_hand_worked():
    # stored lower [[1, *], [2, 3]] -> Sym = [[1, 2], [2, 3]]; B = [[1, 0], [1, 1]]
    # Sym B = [[3, 2], [5, 3]]; B Sym = [[1, 2], [3, 5]]
    A = np.array([[bf(np.float32([1]))[0], 0x7FC0], bf(np.float32([2, 3]))], np.uint16)
    B = bf(np.array([[1, 0], [1, 1]], np.float32))
    R, _ = blas3.symm(LEFT, LOWER, 2, 2, 1.0, A, B, 0.0, None, oracle.C_F32)
    assert R.tolist() == [[3, 2], [5, 3]]
    R, _ = blas3.symm(RIGHT, LOWER, 2, 2, 1.0, A, B, 0.0, None, oracle.C_F32)
    assert R.tolist() == [[1, 2], [3, 5]]


@pytest.mark.parametrize("side", [LEFT, RIGHT])
@pytest.mark.parametrize("uplo", [LOWER, UPPER])
def test_symm_matches_gemm_on_full_symmetric(side, uplo):
    M, N = 21, 17
    n = M if side == LEFT else N
    X = dec(rand_bits((n, n), 14))
    full = bf(((X + X.T) / 2).astype(np.float32))   # a symmetric bf16 matrix (exact halving)
    assert np.array_equal(full, full.T)
    stored = gi.bf16_symmetric_stored(n, uplo, 0)   # NaN template for the other triangle
    i, j = np.arange(n)[:, None], np.arange(n)[None, :]
    keep = (i >= j) if uplo == LOWER else (i <= j)
    stored[keep] = full[keep]
    B = rand_bits((M, N), 15)
    C = gi.bf16_normal((M, N), 16)
    R, S = blas3.symm(side, uplo, M, N, 1.25, stored, B, -1.0, C, oracle.C_BF16)
    if side == LEFT:
        G, GS = oracle.gemm(0, 0, M, N, M, 1.25, full, n, B, N, -1.0, C, N, oracle.IN_BF16, oracle.C_BF16)
    else:
        G, GS = oracle.gemm(0, 0, M, N, N, 1.25, B, N, full, n, -1.0, C, N, oracle.IN_BF16, oracle.C_BF16)
    np.testing.assert_allclose(R, G, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(S, GS, rtol=1e-12, atol=1e-12)


def test_symm_left_right_transpose_identity():
    M, N = 9, 14
    A = gi.bf16_symmetric_stored(M, UPPER, 17)
    B = rand_bits((M, N), 18)
    R_left, _ = blas3.symm(LEFT, UPPER, M, N, 1.0, A, B, 0.0, None, oracle.C_F32)
    Bt = np.ascontiguousarray(B.T)
    R_right, _ = blas3.symm(RIGHT, UPPER, N, M, 1.0, A, Bt, 0.0, None, oracle.C_F32)
    np.testing.assert_allclose(R_left, R_right.T, rtol=1e-14, atol=1e-14)


# ------------------------------------------------------------------------------ TRMM

@pytest.mark.parametrize("side", [LEFT, RIGHT])
@pytest.mark.parametrize("uplo", [LOWER, UPPER])
@pytest.mark.parametrize("transA", [0, 1])
@pytest.mark.parametrize("unit", [False, True])
def test_trmm_matches_gemm_with_zeroed_triangle(side, uplo, transA, unit):
    M, N = 19, 26
    n = M if side == LEFT else N
    A = gi.bf16_triangular(n, uplo, 20, unit=unit)
    Z = zero_other(A, uplo, unit)
    B = rand_bits((M, N), 21)
    R, S = blas3.trmm(side, uplo, transA, int(unit), M, N, -0.5, A, B)
    if side == LEFT:
        G, GS = oracle.gemm(transA, 0, M, N, M, -0.5, Z, n, B, N, 0.0, None, N, oracle.IN_BF16, oracle.C_F32)
    else:
        G, GS = oracle.gemm(0, transA, M, N, N, -0.5, B, N, Z, n, 0.0, None, N, oracle.IN_BF16, oracle.C_F32)
    assert np.isfinite(R).all()
    np.testing.assert_allclose(R, G, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(S, GS, rtol=1e-12, atol=1e-12)


def test_trmm_unit_identity():
    n, N = 6, 4
    A = np.full((n, n), 0x7FC0, np.uint16)
    i, j = np.arange(n)[:, None], np.arange(n)[None, :]
    A[i > j] = 0                            # strictly lower zeros, NaN diagonal and upper
    B = rand_bits((n, N), 22)
    R, _ = blas3.trmm(LEFT, LOWER, 0, 1, n, N, 2.0, A, B)
    assert np.array_equal(R, 2.0 * dec(B))


def test_trmm_hand_worked():
    # upper T = [[2, 1], [*, 3]], op(T) = T^T = [[2, 0], [1, 3]]; B = [[1, 1], [2, 0]]
    # T^T B = [[2, 2], [7, 1]]; right side B T = [[2, 4], [4, 2]]
    A = np.array([bf(np.float32([2, 1])), [0x7FC0, bf(np.float32([3]))[0]]], np.uint16)
    B = bf(np.array([[1, 1], [2, 0]], np.float32))
    R, _ = blas3.trmm(LEFT, UPPER, 1, 0, 2, 2, 1.0, A, B)
    assert R.tolist() == [[2, 2], [7, 1]]
    R, _ = blas3.trmm(RIGHT, UPPER, 0, 0, 2, 2, 1.0, A, B)
    assert R.tolist() == [[2, 4], [4, 2]]


# ------------------------------------------------------------------------------ TRSM

def test_trsm_hand_worked():
    # lower T = [[2, *], [1, 4]], B = [[2, 4], [5, 10]]: row 0 = [1, 2];
    # row 1 = ([5, 10] - 1 * [1, 2]) / 4 = [1, 2]
    A = np.array([[bf(np.float32([2]))[0], 0x7FC0], bf(np.float32([1, 4]))], np.uint16)
    B = bf(np.array([[2, 4], [5, 10]], np.float32))
    X = blas3.trsm(LEFT, LOWER, 0, 0, 2, 2, 1.0, A, B)
    assert X.tolist() == [[1, 2], [1, 2]]
    # right side, X T = B with T lower: x = [x0, x1], x0*2 + x1*1 = b0, x1*4 = b1
    X = blas3.trsm(RIGHT, LOWER, 0, 0, 2, 2, 1.0, A, B)
    assert X.tolist() == [[0.5, 1.0], [2.5 - 10 / 8, 2.5]]


def _int_product(T, X, side):
    """op(T) X (left) or X op(T) (right) in Python integers (brute force)."""
    T = [[int(v) for v in row] for row in T]
    X = [[int(v) for v in row] for row in X]
    if side == LEFT:
        return [[sum(T[i][k] * X[k][j] for k in range(len(X))) for j in range(len(X[0]))] for i in range(len(T))]
    return [[sum(X[i][k] * T[k][j] for k in range(len(T))) for j in range(len(T[0]))] for i in range(len(X))]


@pytest.mark.parametrize("side", [LEFT, RIGHT])
@pytest.mark.parametrize("uplo", [LOWER, UPPER])
@pytest.mark.parametrize("transA", [0, 1])
@pytest.mark.parametrize("unit", [True, False])
def test_trsm_exact_integer_system(side, uplo, transA, unit):
    M, N = 24, 10
    n = M if side == LEFT else N
    A = gi.int_triangular(n, uplo, 30, unit=unit)
    T = dec(zero_other(A, uplo, unit))
    opT = T.T if transA else T
    Xt = dec(gi.ints((M, N), 31, -2, 2, gi.BF16))
    B = np.array(_int_product(opT, Xt, side), dtype=np.float64)
    assert np.abs(B).max() < 256      # exact in bf16
    X = blas3.trsm(side, uplo, transA, int(unit), M, N, 1.0, A, bf(B.astype(np.float32)))
    assert np.array_equal(X, Xt)
    # alpha scales the right-hand side: alpha = 2 with B / 2
    X2 = blas3.trsm(side, uplo, transA, int(unit), M, N, 2.0, A, bf((B / 2).astype(np.float32)))
    assert np.array_equal(X2, Xt)


@pytest.mark.parametrize("side", [LEFT, RIGHT])
@pytest.mark.parametrize("uplo", [LOWER, UPPER])
@pytest.mark.parametrize("transA", [0, 1])
@pytest.mark.parametrize("unit", [False, True])
def test_trsm_matches_scipy(side, uplo, transA, unit):
    M, N = 33, 21
    n = M if side == LEFT else N
    A = gi.bf16_triangular(n, uplo, 40, unit=unit)
    B = rand_bits((M, N), 41)
    X = blas3.trsm(side, uplo, transA, int(unit), M, N, 0.5, A, B)
    T = dec(zero_other(A, uplo, unit))
    b = 0.5 * dec(B)
    if side == LEFT:
        ref = scipy.linalg.solve_triangular(T, b, lower=(uplo == LOWER), trans=transA, unit_diagonal=unit)
    else:  # X op(T) = b  <=>  op(T)^T X^T = b^T
        ref = scipy.linalg.solve_triangular(T, b.T, lower=(uplo == LOWER), trans=1 - transA,
                                            unit_diagonal=unit).T
    np.testing.assert_allclose(X, ref, rtol=1e-12, atol=1e-12)
    # the solved system holds: op(T) X (or X op(T)) gives back alpha * B
    opT = T.T if transA else T
    back = opT @ X if side == LEFT else X @ opT
    np.testing.assert_allclose(back, b, rtol=1e-12, atol=1e-12)


def test_trsm_residual_tiny():
    M, N = 64, 12
    A = gi.bf16_triangular(M, LOWER, 50)
    B = rand_bits((M, N), 51)
    X = blas3.trsm(LEFT, LOWER, 0, 0, M, N, 1.0, A, B)
    T = dec(zero_other(A, LOWER))
    r = np.linalg.norm(T @ X - dec(B)) / (np.linalg.norm(T) * np.linalg.norm(X))
    assert r < 1e-15


def test_generators_poison_unreferenced():
    A = gi.bf16_triangular(5, UPPER, 1, unit=True)
    v = dec(A)
    i, j = np.arange(5)[:, None], np.arange(5)[None, :]
    assert np.isnan(v[i >= j]).all() and np.isfinite(v[i < j]).all()
    S = gi.bf16_symmetric_stored(5, LOWER, 2)
    assert np.isnan(dec(S)[i < j]).all() and np.isfinite(dec(S)[i >= j]).all()
