"""Seeded synthetic inputs for the dense GEMM path.

This module is shared by the tests, the benchmark and the oracle's checks.  It
holds none of the GEMM's arithmetic: it only draws random numbers and turns them
into storage bits of the input formats.  The rounding into those formats is done
by PyTorch's own casts (float32 -> bfloat16 and float32 -> float8_e4m3fn, both
round-to-nearest-even), so neither the oracle nor the GPU library supplies it.

Recipe (one numpy PCG64 generator per tensor, seeded 0, 1, 2, ... in the order
a workload lists its tensors):
  * "uniform":  float32 U[-1, 1)  -> bf16
  * "normal":   float32 N(0, std) -> bf16
  * "e4m3":     float32 N(0, 1), clamped to +-448 -> OCP E4M3 (FN)
  * "int":      integers drawn uniformly from [lo, hi] (exact in bf16 and E4M3)

Workloads come from the pages' shapes: the 4096^3 bf16 ablation baseline and
the K x M/N sweep of the cp.async/ldmatrix ablation plan (sections 2 and 2.3),
the projection-backward pair and the pure-E4M3 forward shape of the fused
communication/compute profile protocol (sections on the v10 backward operators
and the v12 FP8 boundary).
"""
from __future__ import annotations

import dataclasses
from typing import Dict, List, Optional, Tuple

import numpy as np

BF16 = "bf16"
E4M3 = "e4m3"
F32 = "f32"

# dtype codes shared with the C-ABI (input dtype -> C dtype)
DTYPE_CODES = {
    (BF16, F32): 0,
    (BF16, BF16): 1,
    (E4M3, BF16): 2,
    (E4M3, F32): 3,
    (E4M3, E4M3): 6,
}


def _torch():
    import torch  # imported lazily: only the casts are needed
    return torch


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """float32 array -> bf16 storage bits (uint16), PyTorch RNE cast."""
    torch = _torch()
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def f32_to_e4m3_bits(x: np.ndarray) -> np.ndarray:
    """float32 array -> OCP E4M3FN storage bits (uint8), PyTorch RNE cast."""
    torch = _torch()
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    return t.to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def bf16_uniform(shape, seed: int) -> np.ndarray:
    rng = np.random.default_rng(seed)
    x = rng.random(shape, dtype=np.float32) * np.float32(2.0) - np.float32(1.0)
    return f32_to_bf16_bits(x)


def bf16_normal(shape, seed: int, std: float = 1.0) -> np.ndarray:
    rng = np.random.default_rng(seed)
    x = rng.standard_normal(shape, dtype=np.float32)
    if std != 1.0:
        x = x * np.float32(std)
    return f32_to_bf16_bits(x)


def e4m3_normal(shape, seed: int) -> np.ndarray:
    rng = np.random.default_rng(seed)
    x = rng.standard_normal(shape, dtype=np.float32)
    x = np.clip(x, np.float32(-448.0), np.float32(448.0))
    return f32_to_e4m3_bits(x)


def ints(shape, seed: int, lo: int, hi: int, dtype: str) -> np.ndarray:
    rng = np.random.default_rng(seed)
    x = rng.integers(lo, hi + 1, size=shape).astype(np.float32)
    return f32_to_bf16_bits(x) if dtype == BF16 else f32_to_e4m3_bits(x)


def f32_bits(x: np.ndarray) -> np.ndarray:
    return np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)


def draw(kind: str, shape, seed: int, dtype: str, std: float = 1.0) -> np.ndarray:
    """Storage bits for one tensor of the given distribution and dtype."""
    if kind == "uniform":
        assert dtype == BF16
        return bf16_uniform(shape, seed)
    if kind == "normal":
        if dtype == BF16:
            return bf16_normal(shape, seed, std)
        if dtype == F32:
            rng = np.random.default_rng(seed)
            return f32_bits(rng.standard_normal(shape, dtype=np.float32) * np.float32(std))
        raise ValueError(dtype)
    if kind == "e4m3":
        return e4m3_normal(shape, seed)
    if kind == "int4":
        return ints(shape, seed, -4, 4, dtype)
    if kind == "int8":
        return ints(shape, seed, -8, 8, dtype)
    raise ValueError(kind)


@dataclasses.dataclass(frozen=True)
class Gemm:
    """One GEMM call C = alpha*op(A)*op(B) + beta*C on row-major storage."""
    name: str
    M: int
    N: int
    K: int
    transA: int = 0
    transB: int = 0
    in_dtype: str = BF16
    c_dtype: str = BF16
    alpha: float = 1.0
    beta: float = 0.0
    dist: str = "uniform"          # distribution of A and B
    c_dist: Optional[str] = None   # distribution of the initial C (beta != 0)
    c_std: float = 1.0
    seeds: Tuple[int, int, int] = (0, 1, 2)

    @property
    def dtype_code(self) -> int:
        return DTYPE_CODES[(self.in_dtype, self.c_dtype)]

    @property
    def a_shape(self) -> Tuple[int, int]:
        return (self.K, self.M) if self.transA else (self.M, self.K)

    @property
    def b_shape(self) -> Tuple[int, int]:
        return (self.N, self.K) if self.transB else (self.K, self.N)

    @property
    def flops(self) -> float:
        return 2.0 * self.M * self.N * self.K

    @property
    def algorithmic_bytes(self) -> float:
        ib = 2 if self.in_dtype == BF16 else 1
        ob = 2 if self.c_dtype == BF16 else 4
        return ib * (self.M * self.K + self.K * self.N) + ob * self.M * self.N * (1 + (self.beta != 0.0))

    def make(self, seeds: Optional[Tuple[int, int, int]] = None) -> Dict[str, np.ndarray]:
        sa, sb, sc = seeds if seeds is not None else self.seeds
        A = draw(self.dist, self.a_shape, sa, self.in_dtype)
        B = draw(self.dist, self.b_shape, sb, self.in_dtype)
        out = {"A": A, "B": B}
        if self.beta != 0.0 and self.c_dist is not None:
            out["C"] = draw(self.c_dist, (self.M, self.N), sc, self.c_dtype, self.c_std)
        return out


def _sweep() -> List[Gemm]:
    out = []
    for mn in (512, 4096):
        for k in (256, 512, 1024, 4096, 8192):
            out.append(Gemm(f"sweep_mn{mn}_k{k}", mn, mn, k))
    return out


# The five workload families.  The projection-backward pair draws dY, W, X and the
# initial dW with seeds 0, 1, 2, 3; dY is the same buffer in both calls (it is read
# transposed, in place, by the weight-gradient GEMM).
SMALL_256 = Gemm("gemm_256_bf16_f32", 256, 256, 256, c_dtype=F32)
SQUARE_4096 = Gemm("gemm_4096_bf16", 4096, 4096, 4096)
SWEEP = _sweep()
PROJ_DX = Gemm("proj_bwd_dx", 2048, 5120, 5120, dist="normal", seeds=(0, 1, 2))
PROJ_DW = Gemm("proj_bwd_dw", 5120, 5120, 2048, transA=1, transB=0, dist="normal",
               beta=1.0, c_dist="normal", c_std=0.02, seeds=(0, 2, 3))
FP8_FWD = Gemm("fp8_e4m3_16384x5120x5120", 16384, 5120, 5120, in_dtype=E4M3, dist="e4m3")

ALL = [SMALL_256, SQUARE_4096] + SWEEP + [PROJ_DX, PROJ_DW, FP8_FWD]
BY_NAME = {g.name: g for g in ALL}


def proj_backward_inputs(seed_offset: int = 0) -> Dict[str, np.ndarray]:
    """dY[2048,5120], W[5120,5120], X[2048,5120] bf16 N(0,1); dW_init[5120,5120] bf16 N(0,0.02)."""
    s = seed_offset
    return {
        "dY": bf16_normal((2048, 5120), 0 + s),
        "W": bf16_normal((5120, 5120), 1 + s),
        "X": bf16_normal((2048, 5120), 2 + s),
        "dW0": bf16_normal((5120, 5120), 3 + s, std=0.02),
    }


# ---------------------------------------------------------------- block-scaled E4M3 operands

def ue8m0_bytes(shape, seed: int, lo: int = 120, hi: int = 134) -> np.ndarray:
    """Seeded UE8M0 scale bytes, uniform integers in [lo, hi] (2^-7 .. 2^7 around 1)."""
    rng = np.random.default_rng(seed)
    return rng.integers(lo, hi + 1, size=shape, dtype=np.int64).astype(np.uint8)


def mx_operands(M: int, N: int, K: int, seeds=(0, 1, 2, 3), kind: str = "e4m3"):
    """Synthetic block-scaled operands: A [M][K] and B [N][K] E4M3 codes (N(0,1) clamped to
    +-448, or integers in [-8, 8] for kind "int8"), with one scale byte per row and 32
    elements of K (SA [M][ceil(K/32)], SB [N][ceil(K/32)]) drawn by ue8m0_bytes."""
    nb = (K + 31) // 32
    if kind == "int8":
        A, B = ints((M, K), seeds[0], -8, 8, E4M3), ints((N, K), seeds[1], -8, 8, E4M3)
    else:
        A, B = e4m3_normal((M, K), seeds[0]), e4m3_normal((N, K), seeds[1])
    return {"A": A, "B": B, "SA": ue8m0_bytes((M, nb), seeds[2]), "SB": ue8m0_bytes((N, nb), seeds[3])}


# The MXFP8 forward at the E4M3 forward shape (one CP8 rank of S = 128K): A [16384][5120],
# B stored [N][K] = [5120][5120], C bf16.
MX_FWD_SHAPE = (16384, 5120, 5120)


# ---------------------------------------------------------------- BLAS3 family operands
# Triangular and symmetric operands are stored as full n x n row-major arrays; only the
# referenced triangle (lower: i >= j, upper: i <= j) carries the matrix.  The other
# triangle -- and the diagonal, for a unit-diagonal operand -- is filled with NaN, so a
# kernel that reads what it must not read produces NaN.

LOWER, UPPER = 0, 1
BF16_NAN = np.uint16(0x7FC0)


def _referenced(n: int, uplo: int, strict: bool = False) -> np.ndarray:
    i = np.arange(n)[:, None]
    j = np.arange(n)[None, :]
    if uplo == LOWER:
        return (i > j) if strict else (i >= j)
    return (i < j) if strict else (i <= j)


def bf16_triangular(n: int, uplo: int, seed: int, unit: bool = False) -> np.ndarray:
    """A well-conditioned triangular operand: off-diagonal entries U[-1,1)/sqrt(n), the
    diagonal 1 + U[0,1) (condition number about 3 at every n, measured; the off-diagonal
    part carries about a quarter of op(T) x).  Unreferenced entries are NaN; with unit
    set the diagonal is NaN too (it must be taken as ones, never read)."""
    rng = np.random.default_rng(seed)
    off = (rng.random((n, n), dtype=np.float32) * np.float32(2.0) - np.float32(1.0)) / np.float32(np.sqrt(n))
    diag = np.float32(1.0) + rng.random(n, dtype=np.float32)
    bits = f32_to_bf16_bits(off)
    dbits = f32_to_bf16_bits(diag)
    out = np.full((n, n), BF16_NAN, dtype=np.uint16)
    strict = _referenced(n, uplo, strict=True)
    out[strict] = bits[strict]
    if not unit:
        out[np.arange(n), np.arange(n)] = dbits
    return out


def bf16_symmetric_stored(n: int, uplo: int, seed: int, kind: str = "uniform") -> np.ndarray:
    """The uplo triangle (diagonal included) of a random matrix, U[-1,1) or N(0,1) in
    bf16; the other triangle NaN."""
    full = draw(kind, (n, n), seed, BF16)
    out = np.full((n, n), BF16_NAN, dtype=np.uint16)
    keep = _referenced(n, uplo)
    out[keep] = full[keep]
    return out


def int_triangular(n: int, uplo: int, seed: int, unit: bool = True, nnz_per_row: int = 4) -> np.ndarray:
    """An integer triangular operand whose inverse and every partial substitution stay
    small exact binary numbers: off-diagonal entries in {-1, +1} only at (odd row, even
    column) positions of the referenced triangle, about nnz_per_row per odd row, so the
    strictly triangular part squares to zero; the diagonal is all ones (unit; stored as
    NaN) or a power of two in {+-1, +-2, +-4}.  The unreferenced triangle is NaN."""
    rng = np.random.default_rng(seed)
    vals = np.zeros((n, n), dtype=np.float32)
    for i in range(1, n, 2):
        cols = np.arange(0, i, 2) if uplo == LOWER else np.arange(i + 1, n, 2)
        if cols.size == 0:
            continue
        pick = rng.choice(cols, size=min(nnz_per_row, cols.size), replace=False)
        vals[i, pick] = rng.choice(np.array([-1.0, 1.0], dtype=np.float32), size=pick.size)
    out = np.full((n, n), BF16_NAN, dtype=np.uint16)
    strict = _referenced(n, uplo, strict=True)
    out[strict] = f32_to_bf16_bits(vals)[strict]
    if not unit:
        d = rng.choice(np.array([-4.0, -2.0, -1.0, 1.0, 2.0, 4.0], dtype=np.float32), size=n)
        out[np.arange(n), np.arange(n)] = f32_to_bf16_bits(d)
    return out
