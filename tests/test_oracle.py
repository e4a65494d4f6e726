"""Pins of the CPU oracle against values fixed outside it (no GPU needed).

Each test pins one way the oracle could be wrong: a format decoder, the rounding
used for exact comparisons, the indexing of the four transpose cases, the length
of the accumulation, the alpha and beta terms, or the row selection.
"""
import math
import os
from fractions import Fraction

import numpy as np
import pytest

import gemm_inputs as gi
import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
TRANS = [(0, 0), (0, 1), (1, 0), (1, 1)]


def _store(op_mat: np.ndarray, trans: int) -> np.ndarray:
    """Storage of a logical operand: op(X) = X (trans 0) or X^T (trans 1)."""
    return np.ascontiguousarray(op_mat.T if trans else op_mat)


def _bf16(x):
    return gi.f32_to_bf16_bits(np.asarray(x, dtype=np.float32))


def _run(tA, tB, opA_bits, opB_bits, alpha=1.0, beta=0.0, C=None, c_fmt=oracle.C_F32,
         in_fmt=oracle.IN_BF16, rows=None):
    M, K = opA_bits.shape
    N = opB_bits.shape[1]
    A = _store(opA_bits, tA)
    B = _store(opB_bits, tB)
    return oracle.gemm(tA, tB, M, N, K, alpha, A, A.shape[1], B, B.shape[1], beta, C, N,
                       in_fmt, c_fmt, rows=rows)


# ---------------------------------------------------------------- format codecs

def _frac(s: str):
    if s == "nan":
        return None
    if s == "-0":
        return Fraction(0)
    return Fraction(s)


def test_e4m3_golden_codes():
    lines = [l.split("#")[0].split() for l in open(os.path.join(GOLDEN, "e4m3_codes.txt"))]
    lines = [l for l in lines if l]
    assert len(lines) >= 20
    for code_s, val_s in lines:
        code = int(code_s, 16)
        got = oracle.load().oracle_e4m3_value(code)
        want = _frac(val_s)
        if want is None:
            assert math.isnan(got), code_s
        else:
            assert Fraction(got) == want, (code_s, got, want)
            if val_s == "-0":
                assert math.copysign(1.0, got) < 0


def test_e4m3_all_codes_closed_form_and_library():
    import torch
    codes = np.arange(256, dtype=np.uint8)
    mine = oracle.decode(codes, "e4m3")
    lib = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    nan_mine = np.isnan(mine)
    assert nan_mine.sum() == 2 and nan_mine[0x7F] and nan_mine[0xFF]
    assert np.array_equal(nan_mine, np.isnan(lib))
    assert np.array_equal(mine[~nan_mine], lib[~nan_mine])
    finite = mine[~nan_mine]
    assert np.nanmax(finite) == 448.0 and np.nanmin(finite) == -448.0
    # 253 distinct finite values (+0 and -0 compare equal)
    assert len(set(finite.tolist())) == 253
    # closed form for every code, written independently of the decoder
    for c in range(256):
        s, e, m = c >> 7, (c >> 3) & 15, c & 7
        if e == 15 and m == 7:
            continue
        v = Fraction(m, 8) * Fraction(2) ** -6 if e == 0 else (1 + Fraction(m, 8)) * Fraction(2) ** (e - 7)
        assert Fraction(mine[c]) == (-v if s else v), hex(c)


def test_bf16_decode_all_codes_against_library():
    import torch
    codes = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    mine = oracle.decode(codes, "bf16")
    lib = torch.from_numpy(codes.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    nan = np.isnan(lib)
    assert np.array_equal(np.isnan(mine), nan)
    assert np.array_equal(mine[~nan], lib[~nan])


def test_bf16_round_golden():
    for line in open(os.path.join(GOLDEN, "bf16_round.txt")):
        line = line.split("#")[0].strip()
        if not line:
            continue
        x_s, bits_s = line.split()
        x = float.fromhex(x_s) if x_s.lstrip("-").startswith("0x") else float(x_s)
        assert oracle.load().oracle_round_bf16(x) == int(bits_s, 16), line


def test_f32_round_golden():
    xs, want = [], []
    for line in open(os.path.join(GOLDEN, "f32_round.txt")):
        line = line.split("#")[0].strip()
        if not line:
            continue
        x_s, bits_s = line.split()
        xs.append(float.fromhex(x_s) if x_s.lstrip("-").startswith("0x") else float(x_s))
        want.append(int(bits_s, 16))
    got = oracle.round_f32(np.array(xs, dtype=np.float64))
    for x, g, w in zip(xs, got.tolist(), want):
        assert g == w, (x.hex(), hex(g), hex(w))


def test_bf16_round_matches_library_on_f32_values():
    import torch
    rng = np.random.default_rng(7)
    x = rng.standard_normal(200000).astype(np.float32) * np.float32(1e3)
    x = np.concatenate([x, rng.random(1000).astype(np.float32) * np.float32(1e-38)])
    mine = oracle.round_bf16(x.astype(np.float64))
    lib = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(mine, lib)


# ---------------------------------------------------------------- worked example

def test_worked_example():
    rows = [l.split("#")[0].split() for l in open(os.path.join(GOLDEN, "worked_gemm.txt"))]
    rows = [[float(v) for v in r] for r in rows if r]
    A, B, C0 = np.array(rows[0:2]), np.array(rows[2:5]), np.array(rows[5:7])
    alpha, beta = rows[7]
    want = np.array(rows[8:10])
    for tA, tB in TRANS:
        R, S = _run(tA, tB, _bf16(A), _bf16(B), alpha=alpha, beta=beta,
                    C=gi.f32_bits(C0), c_fmt=oracle.C_F32)
        assert np.array_equal(R, want), (tA, tB, R)
        assert np.array_equal(S, np.abs(A) @ np.abs(B))


# ---------------------------------------------------------------- closed forms

@pytest.mark.parametrize("tA,tB", TRANS)
def test_identity_gives_op_b(tA, tB):
    M = K = 13
    N = 7
    I = _bf16(np.eye(M))
    Bv = gi.bf16_uniform((K, N), 3)
    R, _ = _run(tA, tB, I, Bv)
    assert np.array_equal(R, oracle.decode(Bv, "bf16"))
    # and on the right: op(A) * I = op(A)
    Av = gi.bf16_uniform((N, K), 4)
    R2, _ = _run(tA, tB, Av, I)
    assert np.array_equal(R2, oracle.decode(Av, "bf16"))


@pytest.mark.parametrize("tA,tB", TRANS)
def test_permutation_permutes_rows(tA, tB):
    rng = np.random.default_rng(11)
    M = K = 17
    N = 9
    perm = rng.permutation(M)
    P = np.zeros((M, K))
    P[np.arange(M), perm] = 1.0
    Bv = gi.bf16_uniform((K, N), 5)
    R, _ = _run(tA, tB, _bf16(P), Bv)
    assert np.array_equal(R, oracle.decode(Bv, "bf16")[perm])


@pytest.mark.parametrize("K", [1, 5, 256, 4096, 5120])
def test_all_ones_gives_k(K):
    M, N = 3, 4
    R, S = _run(0, 0, _bf16(np.ones((M, K))), _bf16(np.ones((K, N))))
    assert np.all(R == K) and np.all(S == K)


def test_alpha_scales_and_beta_accumulates():
    A = gi.ints((6, 5), 1, -4, 4, "bf16")
    B = gi.ints((5, 7), 2, -4, 4, "bf16")
    C0 = gi.ints((6, 7), 3, -4, 4, "bf16")
    Ad, Bd, Cd = (oracle.decode(x, "bf16") for x in (A, B, C0))
    R, _ = _run(0, 0, A, B, alpha=-2.5, beta=1.0, C=C0, c_fmt=oracle.C_BF16)
    assert np.array_equal(R, -2.5 * (Ad @ Bd) + Cd)
    R, _ = _run(0, 0, A, B, alpha=1.0, beta=-0.5, C=C0, c_fmt=oracle.C_BF16)
    assert np.array_equal(R, Ad @ Bd - 0.5 * Cd)
    # alpha = 0 and A = 0 both leave beta * C exactly
    R, _ = _run(0, 0, A, B, alpha=0.0, beta=3.0, C=C0, c_fmt=oracle.C_BF16)
    assert np.array_equal(R, 3.0 * Cd)
    Z = _bf16(np.zeros((6, 5)))
    R, _ = _run(0, 0, Z, B, alpha=1.0, beta=1.0, C=C0, c_fmt=oracle.C_BF16)
    assert np.array_equal(R, Cd)


def test_beta_zero_never_reads_c():
    A = gi.bf16_uniform((4, 8), 1)
    B = gi.bf16_uniform((8, 5), 2)
    nan_c = gi.f32_bits(np.full((4, 5), np.nan, dtype=np.float32))
    R, _ = _run(0, 0, A, B, beta=0.0, C=nan_c)
    assert np.isfinite(R).all()
    R1, _ = _run(0, 0, A, B, beta=1.0, C=nan_c)
    assert np.isnan(R1).all()


def test_k_zero_gives_beta_c():
    C0 = gi.f32_bits(np.arange(6, dtype=np.float32).reshape(2, 3))
    A = np.zeros((2, 0), dtype=np.uint16)
    B = np.zeros((0, 3), dtype=np.uint16)
    R, S = oracle.gemm(0, 0, 2, 3, 0, 1.0, A, 1, B, 3, 2.0, C0, 3, oracle.IN_BF16, oracle.C_F32)
    assert np.array_equal(R, 2.0 * np.arange(6).reshape(2, 3)) and np.all(S == 0)


# ---------------------------------------------------------------- brute force / library

def test_exact_rational_brute_force():
    """Tiny case summed in exact rationals by pure-Python loops."""
    M, N, K = 3, 4, 5
    for tA, tB in TRANS:
        A = gi.bf16_uniform((M, K), 21)
        B = gi.bf16_uniform((K, N), 22)
        C0 = gi.bf16_uniform((M, N), 23)
        Af = [[Fraction(float(v)) for v in row] for row in oracle.decode(A, "bf16")]
        Bf = [[Fraction(float(v)) for v in row] for row in oracle.decode(B, "bf16")]
        Cf = [[Fraction(float(v)) for v in row] for row in oracle.decode(C0, "bf16")]
        alpha, beta = Fraction(3, 4), Fraction(-5, 2)
        R, _ = _run(tA, tB, A, B, alpha=0.75, beta=-2.5, C=C0, c_fmt=oracle.C_BF16)
        for i in range(M):
            for j in range(N):
                s = sum(Af[i][k] * Bf[k][j] for k in range(K))
                want = alpha * s + beta * Cf[i][j]
                assert R[i, j] == float(want), (tA, tB, i, j)


@pytest.mark.parametrize("tA,tB", TRANS)
@pytest.mark.parametrize("in_fmt", ["bf16", "e4m3"])
def test_against_numpy_float64(tA, tB, in_fmt):
    import torch
    M, N, K = 37, 29, 91
    if in_fmt == "bf16":
        A = gi.bf16_normal((M, K), 31)
        B = gi.bf16_normal((K, N), 32)
        dec = lambda x: torch.from_numpy(x.view(np.int16)).view(torch.bfloat16).double().numpy()
        code = oracle.IN_BF16
    else:
        A = gi.e4m3_normal((M, K), 31)
        B = gi.e4m3_normal((K, N), 32)
        dec = lambda x: torch.from_numpy(x).view(torch.float8_e4m3fn).double().numpy()
        code = oracle.IN_E4M3
    R, S = _run(tA, tB, A, B, in_fmt=code)
    ref = dec(A) @ dec(B)
    assert np.allclose(R, ref, rtol=1e-12, atol=1e-12 * np.abs(dec(A)).max() * np.abs(dec(B)).max() * K)
    assert np.allclose(S, np.abs(dec(A)) @ np.abs(dec(B)), rtol=1e-12)
    assert np.all(S >= np.abs(R) - 1e-12 * S)


def test_row_subset_equals_full():
    g = gi.Gemm("t", 50, 40, 30, transA=1, transB=1, beta=1.0, c_dist="normal", c_std=0.5)
    data = g.make()
    R, S = oracle.gemm_problem(g, data)
    rows = [49, 0, 17, 17, 3]
    Rs, Ss = oracle.gemm_problem(g, data, rows=rows)
    assert np.array_equal(Rs, R[rows]) and np.array_equal(Ss, S[rows])
    with pytest.raises(ValueError):
        oracle.gemm_problem(g, data, rows=[50])


def test_threads_do_not_change_results():
    g = gi.Gemm("t", 64, 48, 200, dist="normal")
    data = g.make()
    R1, S1 = oracle.gemm_problem(g, data, threads=1)
    R4, S4 = oracle.gemm_problem(g, data, threads=4)
    assert np.array_equal(R1, R4) and np.array_equal(S1, S4)


# ---------------------------------------------------------------- input recipe

def test_input_recipe_is_deterministic_and_in_range():
    a = gi.bf16_uniform((64, 64), 0)
    assert np.array_equal(a, gi.bf16_uniform((64, 64), 0))
    assert not np.array_equal(a, gi.bf16_uniform((64, 64), 1))
    v = oracle.decode(a, "bf16")
    assert v.min() >= -1.0 and v.max() <= 1.0
    e = oracle.decode(gi.e4m3_normal((256, 256), 0), "e4m3")
    assert np.isfinite(e).all() and np.abs(e).max() <= 448.0
    assert 0.9 < e.std() < 1.1
    i4 = oracle.decode(gi.ints((100, 100), 3, -4, 4, "bf16"), "bf16")
    assert np.array_equal(i4, np.round(i4)) and i4.min() == -4 and i4.max() == 4
    i8 = oracle.decode(gi.ints((100, 100), 3, -8, 8, "e4m3"), "e4m3")
    assert np.array_equal(i8, np.round(i8)) and i8.min() == -8 and i8.max() == 8


def test_tolerance_helper_accepts_rounded_and_rejects_wrong():
    import tolerance
    g = gi.Gemm("t", 40, 30, 300, dist="normal")
    data = g.make()
    R, S = oracle.gemm_problem(g, data)
    good = oracle.round_bf16(R)
    assert tolerance.check(good, "bf16", R, S, g.K)["ok"]
    bad = good.copy()
    bad[3, 4] ^= 0x0040  # flip a mantissa bit
    assert not tolerance.check(bad, "bf16", R, S, g.K)["ok"]
    good32 = oracle.round_f32(R)
    assert tolerance.check(good32, "f32", R, S, g.K)["ok"]
    bad32 = oracle.round_f32(R * (1 + 1e-4))
    assert not tolerance.check(bad32, "f32", R, S, g.K)["ok"]


# ---------------------------------------------------------------- block-scaled E4M3 (MXFP8)

def _golden_mx():
    vals = {}
    for line in open(os.path.join(GOLDEN, "worked_mx.txt")):
        line = line.split("#")[0].strip()
        if line:
            k, *rest = line.split()
            vals[k] = rest
    return vals


def _expand(spec):
    out = []
    for item in spec:
        n, code = item.split("x")
        out += [int(code, 16)] * int(n)
    return np.array(out, dtype=np.uint8)


def test_mx_worked_example():
    v = _golden_mx()
    K = int(v["K"][0])
    A, B = _expand(v["A"])[None, :], _expand(v["B"])[None, :]
    SA = np.array([int(x) for x in v["SA"]], np.uint8)[None, :]
    SB = np.array([int(x) for x in v["SB"]], np.uint8)[None, :]
    R, S = oracle.gemm_mx(1, 1, K, 1.0, A, K, SA, 2, B, K, SB, 2, 0.0, None, 1, oracle.C_F32)
    assert R[0, 0] == float(v["R"][0]) and S[0, 0] == float(v["R"][0])


def _finite_e4m3_codes(rng, shape):
    c = rng.integers(0, 256, size=shape, dtype=np.uint8)
    c[(c & 0x7F) == 0x7F] = 0x38  # no NaN codes
    return c


def test_mx_unit_scales_equal_plain_e4m3():
    """Scale byte 127 is x1: the block-scaled product equals the (pinned) plain E4M3 GEMM
    with B stored [N][K] (transB = 1), bit for bit, R and S."""
    rng = np.random.default_rng(11)
    M, N, K = 9, 7, 100
    A, B = _finite_e4m3_codes(rng, (M, K)), _finite_e4m3_codes(rng, (N, K))
    one = lambda r: np.full((r, 4), 127, np.uint8)
    C = gi.f32_to_bf16_bits(rng.standard_normal((M, N)).astype(np.float32))
    R1, S1 = oracle.gemm_mx(M, N, K, 0.75, A, K, one(M), 4, B, K, one(N), 4, -2.0, C, N, oracle.C_BF16)
    R2, S2 = oracle.gemm(0, 1, M, N, K, 0.75, A, K, B, K, -2.0, C, N, oracle.IN_E4M3, oracle.C_BF16)
    assert np.array_equal(R1, R2) and np.array_equal(S1, S2)


def test_mx_exact_rational_brute_force():
    """Random codes and scales, summed in Fractions: R within the fp64 summation bound."""
    rng = np.random.default_rng(12)
    M, N, K = 3, 4, 70  # three K blocks, the last one partial
    A, B = _finite_e4m3_codes(rng, (M, K)), _finite_e4m3_codes(rng, (N, K))
    SA = rng.integers(110, 145, size=(M, 3), dtype=np.uint8)
    SB = rng.integers(110, 145, size=(N, 3), dtype=np.uint8)
    R, S = oracle.gemm_mx(M, N, K, 1.0, A, K, SA, 3, B, K, SB, 3, 0.0, None, N, oracle.C_F32)
    tab = oracle.decode(np.arange(256, dtype=np.uint8), "e4m3")
    for i in range(M):
        for j in range(N):
            ex = sum(Fraction(tab[A[i, k]]) * Fraction(2) ** (int(SA[i, k // 32]) - 127) *
                     Fraction(tab[B[j, k]]) * Fraction(2) ** (int(SB[j, k // 32]) - 127) for k in range(K))
            assert abs(R[i, j] - float(ex)) <= K * 2.0 ** -53 * S[i, j]


def test_mx_scale_255_is_nan_and_beta_zero_never_reads_c():
    A = np.full((2, 32), 0x38, np.uint8)
    B = np.full((2, 32), 0x38, np.uint8)
    SA = np.array([[127], [255]], np.uint8)
    SB = np.array([[127], [127]], np.uint8)
    Cnan = np.full((2, 2), 0x7FC00000, np.uint32)
    R, _ = oracle.gemm_mx(2, 2, 32, 1.0, A, 32, SA, 1, B, 32, SB, 1, 0.0, Cnan, 2, oracle.C_F32)
    assert np.all(R[0] == 32.0) and np.all(np.isnan(R[1]))


def test_mx_quantize_golden():
    for line in open(os.path.join(GOLDEN, "mx_quantize.txt")):
        line = line.split("#")[0].strip()
        if not line:
            continue
        xs, e, cs = [part.split() for part in line.split("|")]
        x = np.array([[float(v) for v in xs]])
        codes, scales = oracle.quantize_mx(x)
        assert int(scales[0, 0]) == int(e[0]), line
        assert [int(c) for c in codes[0]] == [int(c, 16) for c in cs], line


def test_mx_quantize_grid_round_trip_and_partial_block():
    """Every finite E4M3 value times 2^s, in blocks whose amax is in [256, 448), comes back
    as its own code with scale byte s + 127; a 70-wide row has a 6-element last block."""
    rng = np.random.default_rng(13)
    tab = oracle.decode(np.arange(256, dtype=np.uint8), "e4m3")
    finite = [c for c in range(256) if (c & 0x7F) != 0x7F]
    for s in (-20, 0, 7):
        codes = np.array(rng.choice(finite, size=(4, 70)), dtype=np.uint8)
        codes[:, 0] = 0x7E  # 448 in every block's first slot: amax 448 -> e = 127 + s
        codes[:, 32] = 0x7E
        codes[:, 64] = 0x7E
        x = tab[codes] * 2.0 ** s
        got, scales = oracle.quantize_mx(x)
        assert np.all(scales == 127 + s)
        same = (got == codes) | ((got & 0x7F) == 0) & ((codes & 0x7F) == 0)
        assert same.all()


def test_mx_quantize_matches_library_cast_and_error_bound():
    """For in-range values the element rounding equals torch's float8_e4m3fn cast (round to
    nearest even, a library routine) of x / 2^(e-127); the decoded block then lies within
    half an E4M3 step of x."""
    import torch
    rng = np.random.default_rng(14)
    x = rng.standard_normal((6, 96)) * np.exp(rng.uniform(-6, 6, size=(6, 1)))
    codes, scales = oracle.quantize_mx(x)
    tab = oracle.decode(np.arange(256, dtype=np.uint8), "e4m3")
    for i in range(6):
        for b in range(3):
            sc = 2.0 ** (int(scales[i, b]) - 127)
            q = x[i, 32 * b:32 * b + 32] / sc
            lib = torch.from_numpy(q.astype(np.float64)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
            got = codes[i, 32 * b:32 * b + 32]
            inr = np.abs(q) <= 448.0  # the library cast does not saturate (it gives NaN)
            assert np.array_equal(lib[inr], got[inr])
            assert np.all((got[~inr] & 0x7F) == 0x7E)
            back = tab[got] * sc
            xb = x[i, 32 * b:32 * b + 32]
            err = np.abs(back - xb)
            assert np.all(err[inr] <= np.abs(xb[inr]) * 2.0 ** -4 + sc * 2.0 ** -10)
            # saturated elements (|q| in (448, 512) by the scale rule) come back as 448
            assert np.all(np.abs(back[~inr]) == 448.0 * sc) and np.all(np.abs(xb[~inr]) < 512.0 * sc)


def test_e4m3_round_golden():
    for line in open(os.path.join(GOLDEN, "e4m3_round.txt")):
        line = line.split("#")[0].strip()
        if not line:
            continue
        x_s, code_s = line.split()
        x = float.fromhex(x_s) if x_s.lstrip("-").startswith("0x") else float(x_s)
        assert int(oracle.round_e4m3(np.array([x]))[0]) == int(code_s, 16), line


def test_e4m3_round_grid_and_special_values():
    """Every finite E4M3 value rounds to its own code (both zeros keep their sign); NaN
    gives the NaN code; +-inf and everything at or past 448 saturate."""
    codes = np.array([c for c in range(256) if (c & 0x7F) != 0x7F], dtype=np.uint8)
    vals = oracle.decode(codes, "e4m3")
    assert np.array_equal(oracle.round_e4m3(vals), codes)
    got = oracle.round_e4m3(np.array([np.nan, np.inf, -np.inf, 448.0, 449.0, -1e300]))
    assert list(got) == [0x7F, 0x7E, 0xFE, 0x7E, 0x7E, 0xFE]


def test_e4m3_round_matches_library_cast_in_range():
    """In range (|x| <= 448) the rounding equals torch's float8_e4m3fn cast (round to
    nearest even, a library routine) on fp32-representable values, normal and subnormal."""
    import torch
    rng = np.random.default_rng(21)
    x = np.concatenate([rng.standard_normal(20000) * 60.0, rng.uniform(-2.0 ** -5, 2.0 ** -5, 20000),
                        rng.uniform(-448.0, 448.0, 20000)]).astype(np.float32)
    mine = oracle.round_e4m3(x.astype(np.float64))
    lib = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    inr = np.abs(x) <= 448.0
    assert inr.sum() > 55000
    assert np.array_equal(mine[inr], lib[inr])


def test_e4m3_output_beta_reads_e4m3():
    """With an E4M3 C the beta term reads C's old codes as E4M3 values."""
    A = np.ones((1, 2), dtype=np.uint16) * 0x3F80  # bf16 1.0
    B = np.ones((2, 1), dtype=np.uint16) * 0x3F80
    C = np.array([[0x48]], dtype=np.uint8)  # E4M3 4.0
    R, _ = oracle.gemm(0, 0, 1, 1, 2, 1.0, A, 2, B, 1, 0.5, C, 1, oracle.IN_BF16, oracle.C_E4M3)
    assert R[0, 0] == 2.0 + 0.5 * 4.0
