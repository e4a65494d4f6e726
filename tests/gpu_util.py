"""Helpers shared by the GPU tests: moving storage bits to and from the device,
calling the library through its C-ABI, and comparing with the oracle."""
from __future__ import annotations

import numpy as np

import gemm_inputs as gi
import oracle
import tolerance


def to_device(bits: np.ndarray, kind: str, device: str = "cuda:0"):
    import torch
    bits = np.ascontiguousarray(bits)
    if kind == "bf16":
        return torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(device)
    if kind == "e4m3":
        return torch.from_numpy(bits).view(torch.float8_e4m3fn).to(device)
    if kind == "f32":
        return torch.from_numpy(bits.view(np.float32)).to(device)
    raise ValueError(kind)


def to_host(t) -> np.ndarray:
    import torch
    t = t.detach().cpu().contiguous()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    if t.dtype == torch.float8_e4m3fn:
        return t.view(torch.uint8).numpy()
    if t.dtype == torch.float32:
        return t.numpy().view(np.uint32)
    raise ValueError(t.dtype)


def empty_c(M: int, N: int, c_dtype: str, fill: float = float("nan"), ldc: int = None):
    import torch
    ldc = ldc or N
    dt = torch.float32 if c_dtype == "f32" else torch.bfloat16
    buf = torch.full((M, ldc), fill, dtype=dt, device="cuda:0")
    return buf[:, :N] if ldc != N else buf


def run_gpu(g, problem: gi.Gemm, data, C_init=None, policy=None, ldc=None):
    """Runs `problem` on the GPU with the given storage bits; returns C's bits (M x N)."""
    import torch
    A = to_device(data["A"], problem.in_dtype)
    B = to_device(data["B"], problem.in_dtype)
    if C_init is not None:
        C = to_device(C_init, problem.c_dtype)
    elif "C" in data:
        C = to_device(data["C"], problem.c_dtype)
    else:
        C = empty_c(problem.M, problem.N, problem.c_dtype, ldc=ldc)
    g.set_policy(policy)
    try:
        g(A, B, C, transA=problem.transA, transB=problem.transB, alpha=problem.alpha,
          beta=problem.beta, dtype=problem.dtype_code)
    finally:
        g.set_policy(None)
    torch.cuda.synchronize()
    return to_host(C)


def sample_rows(M: int, tile: int = 256, per_tile: int = 2, seed: int = 0, cap: int = 64):
    """Rows spread over every M tile: each tile's first and last row plus random ones."""
    rng = np.random.default_rng(seed)
    rows = set()
    for t0 in range(0, M, tile):
        t1 = min(M, t0 + tile) - 1
        rows.add(t0)
        rows.add(t1)
        for _ in range(per_tile):
            rows.add(int(rng.integers(t0, t1 + 1)))
    rows = sorted(rows)
    if len(rows) > cap:
        idx = np.linspace(0, len(rows) - 1, cap).round().astype(int)
        rows = sorted(set(rows[i] for i in idx))
    return rows


def compare(problem: gi.Gemm, data, C_bits, rows=None, accumulate="fp32"):
    """Oracle on `rows` (all when None) and the acceptance check of tolerance.py."""
    R, S = oracle.gemm_problem(problem, data, rows=rows)
    got = C_bits if rows is None else C_bits[rows]
    return tolerance.check(got, problem.c_dtype, R, S, problem.K, accumulate=accumulate)


def whole_tiles(M, count=8, tile=256):
    """Every row of `count` 256-row tiles spread evenly from the first to the last (tiles
    that cover different XCDs, raster positions and the ragged end)."""
    n = (M + tile - 1) // tile
    picks = sorted({round(i * (n - 1) / max(count - 1, 1)) for i in range(count)})
    rows = []
    for t in picks:
        rows.extend(range(t * tile, min(M, (t + 1) * tile)))
    return rows
