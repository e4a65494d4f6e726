"""CPU tests of the acceptance criteria in tolerance.py: a correct result passes, and
results with planted mistakes fail (the mistakes are planted here, on the CPU)."""
import numpy as np

import gemm_inputs as gi
import oracle
import tolerance
from oracle import blas3

LOWER, LEFT = 0, 0


def _bf16(x):
    return tolerance.bf16_bits_to_f64(oracle.round_bf16(np.asarray(x, dtype=np.float64)))


def _system(n, m, seed):
    A = gi.bf16_triangular(n, LOWER, seed)
    B = gi.bf16_uniform((n, m), seed + 1)
    T = blas3.triangular(A, n, LOWER, 0)
    X_ref = blas3.trsm(LEFT, LOWER, 0, 0, n, m, 1.0, A, B)
    return T, tolerance.bf16_bits_to_f64(B), X_ref


def _blocked_solve(T, B, leaf):
    """The blocked method's roundings, modelled in float64: each leaf's inverted diagonal
    block and its product with B, and each update of B, rounded to bf16 once."""
    n = T.shape[0]
    if n <= leaf:
        return _bf16(_bf16(np.linalg.inv(T)) @ B)
    h = (n // 2 + leaf - 1) // leaf * leaf
    X1 = _blocked_solve(T[:h, :h], B[:h], leaf)
    B2 = _bf16(B[h:] - T[h:, :h] @ X1)
    return np.vstack([X1, _blocked_solve(T[h:, h:], B2, leaf)])


def test_trsm_check_accepts_the_rounded_solution():
    T, B, X_ref = _system(300, 40, 3)
    res = tolerance.trsm_check(_bf16(X_ref), X_ref, T, B, LEFT, 300)
    assert res["ok"], res
    assert abs(res["eta"] - res["eta_round"]) <= 1e-12


def test_trsm_check_accepts_the_blocked_method():
    for n in (256, 512, 1024):
        T, B, X_ref = _system(n, 32, 7)
        res = tolerance.trsm_check(_blocked_solve(T, B, 256), X_ref, T, B, LEFT, n)
        assert res["ok"], (n, res)


def test_trsm_check_rejects_small_errors():
    T, B, X_ref = _system(512, 32, 11)
    rng = np.random.default_rng(0)
    # every element off by 3 bf16 units (relative 3 * 2^-8) in a random direction
    bad = _bf16(X_ref * (1 + 3 * 2.0 ** -8 * rng.choice([-1.0, 1.0], X_ref.shape)))
    assert not tolerance.trsm_check(bad, X_ref, T, B, LEFT, 512)["ok"]
    # the whole solution 1% too large (a scale slip)
    assert not tolerance.trsm_check(_bf16(X_ref * 1.01), X_ref, T, B, LEFT, 512)["ok"]
    # one row of the solution left at its right-hand side (a dropped update or solve)
    bad = _bf16(X_ref)
    bad[300] = B[300]
    assert not tolerance.trsm_check(bad, X_ref, T, B, LEFT, 512)["ok"]
    # a NaN anywhere
    bad = _bf16(X_ref)
    bad[5, 5] = np.nan
    assert not tolerance.trsm_check(bad, X_ref, T, B, LEFT, 512)["ok"]


def test_gemm_check_rejects_planted_mistakes():
    p = gi.Gemm("t", 64, 48, 200, dist="normal")
    data = p.make()
    R, S = oracle.gemm_problem(p, data)
    good = oracle.round_bf16(R)
    assert tolerance.check(good, "bf16", R, S, p.K)["ok"]
    # a dropped K term: the sum over k < K - 1 only
    q = gi.Gemm("t", 64, 48, 199, dist="normal")
    short = {"A": np.ascontiguousarray(data["A"][:, :199]), "B": np.ascontiguousarray(data["B"][:199])}
    R2, _ = oracle.gemm_problem(q, short)
    assert not tolerance.check(oracle.round_bf16(R2), "bf16", R, S, p.K)["ok"]
    # a sign flip of one element, and transposed output indices on a square corner
    bad = good.copy()
    bad[3, 7] ^= 0x8000
    assert not tolerance.check(bad, "bf16", R, S, p.K)["ok"]
    bad = good.copy()
    bad[:32, :32] = good[:32, :32].T
    assert not tolerance.check(bad, "bf16", R, S, p.K)["ok"]
