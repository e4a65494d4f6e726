"""CPU oracle for the single-GPU BLAS level-3 family -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and ``bench.py``'s ``cpu_baseline`` leg may
import this module; the GPU library never calls it and shares no code with it.

"BLASMp development notes" (section 1 and the timeline of section 2: SYRK, TRSM, SYR2K,
SYMM and TRMM on top of a GEMM core) names the operator set; the pages give no formula,
so each function below is the textbook BLAS definition, written out in float64 on
matrices decoded from their storage bits by the oracle's own decoders
(``oracle.decode``).  A float64 matrix product (numpy ``@``) serves as a step where the
definition is a product; the triangular solve is written as plain substitution.

Conventions (row-major, element (i, j) is row i, column j; the leading dimension is the
row stride):
  uplo  0: the lower triangle (i >= j) is referenced / written; 1: the upper (i <= j).
  trans 0: op(X) = X; 1: op(X) = X^T.
  side  0: the triangular / symmetric matrix multiplies from the left; 1: from the right.
  diag  0: the diagonal of the triangular matrix is read; 1: it is taken as all ones and
        never read.

Every function returns float64 results; those that feed the GEMM tolerance also return
S, the matching sum of |products| (the same product on |entries|, without alpha, as the
GEMM oracle's S).
"""
from __future__ import annotations

from typing import Optional, Tuple

import numpy as np

from . import C_BF16, C_E4M3, C_F32, decode

LOWER, UPPER = 0, 1
LEFT, RIGHT = 0, 1
NON_UNIT, UNIT = 0, 1

_FMT = {C_F32: "f32", C_BF16: "bf16", C_E4M3: "e4m3"}


def _mat(bits: np.ndarray, rows: int, cols: int, fmt: str = "bf16") -> np.ndarray:
    """Decodes the leading rows x cols block of a row-major [rows][ld] bit array."""
    bits = np.asarray(bits)
    if rows == 0 or cols == 0:
        return np.zeros((rows, cols), dtype=np.float64)
    return decode(np.ascontiguousarray(bits[:rows, :cols]), fmt)


def _op(X: np.ndarray, trans: int) -> np.ndarray:
    return X.T if trans else X


def _in_triangle(n_rows: int, n_cols: int, uplo: int) -> np.ndarray:
    """Boolean mask of the referenced triangle: i >= j (lower) or i <= j (upper)."""
    i = np.arange(n_rows)[:, None]
    j = np.arange(n_cols)[None, :]
    return (i >= j) if uplo == LOWER else (i <= j)


def _c_old(C: Optional[np.ndarray], rows: int, cols: int, c_fmt: int) -> np.ndarray:
    if C is None:
        return np.zeros((rows, cols), dtype=np.float64)
    return _mat(C, rows, cols, _FMT[c_fmt])


def triangular(A: np.ndarray, n: int, uplo: int, diag: int) -> np.ndarray:
    """The n x n triangular matrix T that the stored A stands for: the uplo triangle of A,
    zeros in the other (whatever A holds there), ones on the diagonal if diag is UNIT."""
    X = _mat(A, n, n)
    T = np.where(_in_triangle(n, n, uplo), X, 0.0)
    if diag == UNIT:
        np.fill_diagonal(T, 1.0)
    return T


def symmetric(A: np.ndarray, n: int, uplo: int) -> np.ndarray:
    """The n x n symmetric matrix the stored A stands for: entry (i, j) of the uplo
    triangle is A[i][j]; entry (j, i) mirrors it; the other triangle of A is never read."""
    X = _mat(A, n, n)
    keep = _in_triangle(n, n, uplo)
    return np.where(keep, X, X.T)


def syrk(uplo: int, trans: int, N: int, K: int, alpha: float, A: np.ndarray, beta: float,
         C: Optional[np.ndarray], c_fmt: int) -> Tuple[np.ndarray, np.ndarray]:
    """Symmetric rank-K update on one triangle:
        R = alpha * op(A) op(A)^T + beta * C_old  where (i, j) is in the uplo triangle,
        R = C_old                                 elsewhere (not written).
    op(A) is N x K: A is [N][K] (trans 0) or [K][N] (trans 1).  beta == 0: C_old is not
    read inside the triangle (a NaN there does not reach R)."""
    a = _op(_mat(A, K, N) if trans else _mat(A, N, K), trans)
    P = a @ a.T
    S = np.abs(a) @ np.abs(a).T
    old = _c_old(C, N, N, c_fmt)
    tri = _in_triangle(N, N, uplo)
    upd = alpha * P + (beta * old if beta != 0.0 else 0.0)
    R = np.where(tri, upd, old)
    return R, np.where(tri, S, 0.0)


def syr2k(uplo: int, trans: int, N: int, K: int, alpha: float, A: np.ndarray, B: np.ndarray,
          beta: float, C: Optional[np.ndarray], c_fmt: int) -> Tuple[np.ndarray, np.ndarray]:
    """Symmetric rank-2K update on one triangle:
        R = alpha * (op(A) op(B)^T + op(B) op(A)^T) + beta * C_old  inside the triangle,
        R = C_old  elsewhere.
    op(A), op(B) are N x K, stored like A of syrk."""
    a = _op(_mat(A, K, N) if trans else _mat(A, N, K), trans)
    b = _op(_mat(B, K, N) if trans else _mat(B, N, K), trans)
    P = a @ b.T + b @ a.T
    S = np.abs(a) @ np.abs(b).T + np.abs(b) @ np.abs(a).T
    old = _c_old(C, N, N, c_fmt)
    tri = _in_triangle(N, N, uplo)
    upd = alpha * P + (beta * old if beta != 0.0 else 0.0)
    return np.where(tri, upd, old), np.where(tri, S, 0.0)


def symm(side: int, uplo: int, M: int, N: int, alpha: float, A: np.ndarray, B: np.ndarray,
         beta: float, C: Optional[np.ndarray], c_fmt: int) -> Tuple[np.ndarray, np.ndarray]:
    """Symmetric matrix product: R = alpha * Sym(A) B + beta * C_old (side LEFT, A is M x M)
    or alpha * B Sym(A) + beta * C_old (side RIGHT, A is N x N); B and C are M x N.  Sym(A)
    is built from A's uplo triangle only."""
    n = M if side == LEFT else N
    Sy = symmetric(A, n, uplo)
    b = _mat(B, M, N)
    if side == LEFT:
        P, S = Sy @ b, np.abs(Sy) @ np.abs(b)
    else:
        P, S = b @ Sy, np.abs(b) @ np.abs(Sy)
    old = _c_old(C, M, N, c_fmt)
    R = alpha * P + (beta * old if beta != 0.0 else 0.0)
    return R, S


def trmm(side: int, uplo: int, transA: int, diag: int, M: int, N: int, alpha: float,
         A: np.ndarray, B: np.ndarray) -> Tuple[np.ndarray, np.ndarray]:
    """Triangular matrix product (out of place): R = alpha * op(T) B (side LEFT, T is
    M x M) or alpha * B op(T) (side RIGHT, T is N x N), T = triangular(A, uplo, diag);
    B is M x N."""
    n = M if side == LEFT else N
    T = _op(triangular(A, n, uplo, diag), transA)
    b = _mat(B, M, N)
    if side == LEFT:
        return alpha * (T @ b), np.abs(T) @ np.abs(b)
    return alpha * (b @ T), np.abs(b) @ np.abs(T)


def _substitute(T: np.ndarray, rhs: np.ndarray, lower: bool) -> np.ndarray:
    """Solves T X = rhs for X by substitution, T square triangular (lower: forward, row 0
    first; upper: backward, the last row first).  Row i of X is (rhs_i - sum over the
    already solved rows j of T_ij X_j) / T_ii, every column at once."""
    n = T.shape[0]
    X = np.zeros_like(rhs)
    order = range(n) if lower else range(n - 1, -1, -1)
    for i in order:
        done = slice(0, i) if lower else slice(i + 1, n)
        acc = rhs[i] - T[i, done] @ X[done]
        X[i] = acc / T[i, i]
    return X


def trsm(side: int, uplo: int, transA: int, diag: int, M: int, N: int, alpha: float,
         A: np.ndarray, B: np.ndarray) -> np.ndarray:
    """Triangular solve: X with op(T) X = alpha * B (side LEFT, T is M x M) or
    X op(T) = alpha * B (side RIGHT, T is N x N); B and X are M x N.  The right-side
    system is solved through its transpose, op(T)^T X^T = alpha * B^T."""
    n = M if side == LEFT else N
    T = _op(triangular(A, n, uplo, diag), transA)
    b = alpha * _mat(B, M, N)
    if side == LEFT:
        lower = (uplo == LOWER) != bool(transA)
        return _substitute(T, b, lower)
    Tt = T.T
    lower = (uplo == LOWER) == bool(transA)  # op(T)^T is lower iff op(T) is upper
    return _substitute(Tt, b.T.copy(), lower).T
