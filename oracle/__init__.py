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

_lib = None


def build() -> str:
    """Compile the oracle with gcc (-O2, no fast-math, no FP contraction, OpenMP)."""
    tmp = _LIB + ".tmp"
    cmd = ["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-fopenmp", "-ffp-contract=off",
           "-fno-fast-math", "-Wall", "-o", tmp, _SRC, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, _LIB)
    return _LIB


def load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        build()
    lib = ctypes.CDLL(_LIB)
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
