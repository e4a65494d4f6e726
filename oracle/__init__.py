"""CPU oracle for C = alpha*op(A)*op(B) + beta*C -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this package.  The GPU library never calls it and the
two share no code (see ``oracle_gemm.c`` for the definition it follows and the
formats it decodes).

The C source is compiled with gcc into ``liboracle.so`` next to this file
(``build()``); ``load()`` compiles it on first use if no library is there.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Optional, Sequence, Tuple

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle_gemm.c")
_LIB = os.path.join(_HERE, "liboracle.so")

IN_BF16 = 0
IN_E4M3 = 1
C_F32 = 0
C_BF16 = 1
C_E4M3 = 2

_SAN_LIB = os.path.join(_HERE, "liboracle_san.so")

_lib = None


def build() -> str:
    """Compile the oracle with gcc (-O2, no fast-math, no FP contraction, OpenMP)."""
    tmp = _LIB + ".tmp"
    cmd = ["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-fopenmp", "-ffp-contract=off",
           "-fno-fast-math", "-Wall", "-o", tmp, _SRC, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, _LIB)
    return _LIB


def build_sanitized() -> str:
    """The same source with AddressSanitizer and UndefinedBehaviorSanitizer (clang, whose
    runtime the sanitized GEMM library shares), for the CPU tests' sanitizer run; load it
    with ORACLE_LIB pointing at it."""
    if os.path.exists(_SAN_LIB) and os.path.getmtime(_SAN_LIB) >= os.path.getmtime(_SRC):
        return _SAN_LIB
    tmp = _SAN_LIB + ".tmp"
    cmd = ["/opt/rocm/llvm/bin/clang", "-O1", "-g", "-std=c11", "-fPIC", "-shared", "-fopenmp",
           "-ffp-contract=off", "-fno-fast-math", "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
           "-fno-sanitize-recover=undefined", "-o", tmp, _SRC, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, _SAN_LIB)
    return _SAN_LIB


def load():
    global _lib
    if _lib is not None:
        return _lib
    path = os.environ.get("ORACLE_LIB")
    if not path:
        path = _LIB
        if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
            build()
    lib = ctypes.CDLL(path)
    i64 = ctypes.c_int64
    vp = ctypes.c_void_p
    lib.oracle_gemm.restype = ctypes.c_int
    lib.oracle_gemm.argtypes = [ctypes.c_int, ctypes.c_int, i64, i64, i64, ctypes.c_double,
                                vp, i64, vp, i64, ctypes.c_double, vp, i64, ctypes.c_int,
                                ctypes.c_int, vp, i64, vp, vp, ctypes.c_int]
    lib.oracle_decode.argtypes = [ctypes.c_int, vp, i64, vp]
    lib.oracle_decode.restype = None
    lib.oracle_round_bf16_array.argtypes = [vp, i64, vp]
    lib.oracle_round_bf16_array.restype = None
    lib.oracle_round_f32_array.argtypes = [vp, i64, vp]
    lib.oracle_round_f32_array.restype = None
    lib.oracle_e4m3_value.argtypes = [ctypes.c_uint8]
    lib.oracle_e4m3_value.restype = ctypes.c_double
    lib.oracle_bf16_value.argtypes = [ctypes.c_uint16]
    lib.oracle_bf16_value.restype = ctypes.c_double
    lib.oracle_round_bf16.argtypes = [ctypes.c_double]
    lib.oracle_round_bf16.restype = ctypes.c_uint16
    lib.oracle_gemm_mx.restype = ctypes.c_int
    lib.oracle_gemm_mx.argtypes = [i64, i64, i64, ctypes.c_double, vp, i64, vp, i64, vp, i64, vp, i64,
                                   ctypes.c_double, vp, i64, ctypes.c_int, vp, i64, vp, vp, ctypes.c_int]
    _lib = lib
    return lib


def default_threads() -> int:
    try:
        return max(1, len(os.sched_getaffinity(0)))
    except AttributeError:  # pragma: no cover
        return os.cpu_count() or 1


def _ptr(a: Optional[np.ndarray]):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def gemm(transA: int, transB: int, M: int, N: int, K: int, alpha: float,
         A: np.ndarray, lda: int, B: np.ndarray, ldb: int, beta: float,
         C: Optional[np.ndarray], ldc: int, in_fmt: int, c_fmt: int,
         rows: Optional[Sequence[int]] = None, with_abs: bool = True,
         threads: Optional[int] = None) -> Tuple[np.ndarray, Optional[np.ndarray]]:
    """Returns (R, S): fp64 results and fp64 sums of |products| for the chosen rows.

    A, B (and C) are the storage bits (uint16 for bf16, uint8 for E4M3, uint32
    for fp32 C), laid out row-major with the given leading dimensions.
    """
    lib = load()
    A = np.ascontiguousarray(A)
    B = np.ascontiguousarray(B)
    if C is not None:
        C = np.ascontiguousarray(C)
    if rows is None:
        nrows = M
        rows_arr = None
    else:
        rows_arr = np.ascontiguousarray(np.asarray(rows, dtype=np.int64))
        nrows = int(rows_arr.size)
    R = np.empty((nrows, N), dtype=np.float64)
    S = np.empty((nrows, N), dtype=np.float64) if with_abs else None
    rc = lib.oracle_gemm(int(transA), int(transB), int(M), int(N), int(K), float(alpha),
                         _ptr(A), int(lda), _ptr(B), int(ldb), float(beta), _ptr(C), int(ldc),
                         int(in_fmt), int(c_fmt), _ptr(rows_arr), int(nrows), _ptr(R), _ptr(S),
                         int(threads or default_threads()))
    if rc != 0:
        raise ValueError("oracle_gemm rejected its arguments")
    return R, S


def decode(bits: np.ndarray, fmt: str) -> np.ndarray:
    """Storage bits -> float64 ('bf16', 'e4m3' or 'f32')."""
    lib = load()
    bits = np.ascontiguousarray(bits)
    out = np.empty(bits.shape, dtype=np.float64)
    code = {"bf16": 0, "e4m3": 1, "f32": 2}[fmt]
    lib.oracle_decode(code, _ptr(bits), int(bits.size), _ptr(out))
    return out


def round_bf16(x: np.ndarray) -> np.ndarray:
    lib = load()
    x = np.ascontiguousarray(x, dtype=np.float64)
    out = np.empty(x.shape, dtype=np.uint16)
    lib.oracle_round_bf16_array(_ptr(x), int(x.size), _ptr(out))
    return out


def round_f32(x: np.ndarray) -> np.ndarray:
    lib = load()
    x = np.ascontiguousarray(x, dtype=np.float64)
    out = np.empty(x.shape, dtype=np.uint32)
    lib.oracle_round_f32_array(_ptr(x), int(x.size), _ptr(out))
    return out


def gemm_problem(g, data, rows=None, with_abs=True, threads=None):
    """Runs the oracle on a ``gemm_inputs.Gemm`` description and its storage bits."""
    in_fmt = IN_BF16 if g.in_dtype == "bf16" else IN_E4M3
    c_fmt = C_BF16 if g.c_dtype == "bf16" else C_F32
    A, B = data["A"], data["B"]
    C = data.get("C")
    return gemm(g.transA, g.transB, g.M, g.N, g.K, g.alpha, A, A.shape[1], B, B.shape[1],
                g.beta, C, g.N, in_fmt, c_fmt, rows=rows, with_abs=with_abs, threads=threads)


def gemm_mx(M: int, N: int, K: int, alpha: float, A: np.ndarray, lda: int, SA: np.ndarray, ldsa: int,
            B: np.ndarray, ldb: int, SB: np.ndarray, ldsb: int, beta: float, C: Optional[np.ndarray],
            ldc: int, c_fmt: int, rows: Optional[Sequence[int]] = None, with_abs: bool = True,
            threads: Optional[int] = None) -> Tuple[np.ndarray, Optional[np.ndarray]]:
    """Block-scaled E4M3 GEMM (see oracle_gemm_mx): A [M][lda], B [N][ldb] E4M3 codes, SA
    [M][ldsa], SB [N][ldsb] UE8M0 bytes, one per row and 32-element K block."""
    lib = load()
    A, B = np.ascontiguousarray(A, dtype=np.uint8), np.ascontiguousarray(B, dtype=np.uint8)
    SA, SB = np.ascontiguousarray(SA, dtype=np.uint8), np.ascontiguousarray(SB, dtype=np.uint8)
    if C is not None:
        C = np.ascontiguousarray(C)
    if rows is None:
        nrows, rows_arr = M, None
    else:
        rows_arr = np.ascontiguousarray(np.asarray(rows, dtype=np.int64))
        nrows = int(rows_arr.size)
    R = np.empty((nrows, N), dtype=np.float64)
    S = np.empty((nrows, N), dtype=np.float64) if with_abs else None
    rc = lib.oracle_gemm_mx(int(M), int(N), int(K), float(alpha), _ptr(A), int(lda), _ptr(SA), int(ldsa),
                            _ptr(B), int(ldb), _ptr(SB), int(ldsb), float(beta), _ptr(C), int(ldc),
                            int(c_fmt), _ptr(rows_arr), int(nrows), _ptr(R), _ptr(S),
                            int(threads or default_threads()))
    if rc != 0:
        raise ValueError("oracle_gemm_mx rejected its arguments")
    return R, S


# The 127 non-negative finite E4M3 values in code order (0x00 .. 0x7E).
def _e4m3_grid():
    codes = np.arange(0x7F, dtype=np.uint8)
    return decode(codes, "e4m3"), codes


def _e4m3_code(q: float, grid, gcodes) -> int:
    """E4M3 code of |q| (q >= 0, not NaN): the nearest grid value, ties to the even code,
    448 for everything at or above 448."""
    if q >= 448.0:
        return 0x7E
    hi = int(np.searchsorted(grid, q))  # grid[hi-1] < q <= grid[hi]
    if grid[hi] == q:
        return int(gcodes[hi])
    lo = hi - 1
    dlo, dhi = q - grid[lo], grid[hi] - q
    if dlo < dhi or (dlo == dhi and gcodes[lo] % 2 == 0):
        return int(gcodes[lo])
    return int(gcodes[hi])


def round_e4m3(x: np.ndarray) -> np.ndarray:
    """float64 values -> OCP E4M3 codes: the nearest E4M3 value, ties to the even code,
    saturating at +-448 (an output format with a caller scale has no infinity to go to),
    NaN to the NaN code, sign kept (also for zero).  Element by element on the sorted grid
    of the format's values."""
    x = np.asarray(x, dtype=np.float64)
    grid, gcodes = _e4m3_grid()
    out = np.empty(x.shape, dtype=np.uint8)
    flat, dst = x.reshape(-1), out.reshape(-1)
    for t, v in enumerate(flat):
        c = 0x7F if np.isnan(v) else _e4m3_code(abs(float(v)), grid, gcodes)
        dst[t] = c | (0x80 if np.signbit(v) else 0)
    return out


def quantize_mx(x: np.ndarray) -> Tuple[np.ndarray, np.ndarray]:
    """Quantises each row of x (float64 values, rows x cols) to E4M3 codes with one UE8M0
    scale per 32 consecutive elements of the row (the last block may be shorter).

    The MXFP8 quantisation the fused profile protocol describes (section "SM103 MXFP8
    QKV weight-quantization diagnostics": read, amax of the 32-element group, UE8M0
    scale, E4M3 conversion) with the rule of the OCP microscaling format, which the page
    does not spell out: the scale exponent is floor(log2(amax)) minus 8, the largest
    E4M3 exponent, clamped to the UE8M0 range (stored as that plus 127, 0 .. 254; an
    all-zero block gets 0); each element is x / 2^(e-127) rounded to the nearest E4M3
    value, ties to the even code, saturating at +-448, keeping the sign of x.
    Plain loops over blocks; the nearest value is found on the sorted grid.
    """
    x = np.asarray(x, dtype=np.float64)
    rows, cols = x.shape
    nb = (cols + 31) // 32
    grid, gcodes = _e4m3_grid()
    codes = np.zeros((rows, cols), dtype=np.uint8)
    scales = np.zeros((rows, nb), dtype=np.uint8)
    for i in range(rows):
        for b in range(nb):
            blk = x[i, 32 * b:32 * b + 32]
            amax = float(np.max(np.abs(blk)))
            if amax == 0.0:
                e = 0
            else:
                _f, ex = np.frexp(amax)  # amax = f * 2^ex, f in [0.5, 1)
                e = int(min(254, max(0, (int(ex) - 1) - 8 + 127)))
            scales[i, b] = e
            for t, v in enumerate(blk):
                c = _e4m3_code(abs(float(v)) / 2.0 ** (e - 127), grid, gcodes)
                if np.signbit(v):
                    c |= 0x80
                codes[i, 32 * b + t] = c
    return codes, scales
